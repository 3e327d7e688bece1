"""tri_inverse_amd -- Python binding of libgdn (include/gdn.h) for MI355X (gfx950).

Thin ctypes layer: every function here has the name of the C entry point it calls,
checks the tensors' device, dtype, shape and contiguity, and passes data pointers and
the current HIP stream.  Every step of the computation runs in libgdn's HIP kernels;
there is no CPU or PyTorch fallback.  If libgdn.so has not been built, importing this
package raises ImportError (build it with ``python tri_inverse_amd/build.py``).

PyTorch is used only for device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libgdn.so is not built (run `python tri_inverse_amd/build.py`); "
                      "tri_inverse_amd has no fallback path")

_lib = ctypes.CDLL(LIB_PATH)

# dtype and mode codes (gdn.h)
GDN_F32, GDN_BF16, GDN_FP8_E4M3, GDN_INT8, GDN_INT16 = 0, 1, 2, 3, 4
GDN_INV_NEUMANN, GDN_INV_EXACT, GDN_INV_NEUMANN_PRODUCTS = 0, 1, 2
GDN_OK = 0
GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP = 5, 6, 7
FP8_STATS_FIELDS = ("nonfinite", "sat_dynamic", "sat_static", "underflow")

_COMPUTE = {"f32": GDN_F32, "fp32": GDN_F32, "bf16": GDN_BF16, "fp8": GDN_FP8_E4M3,
            "e4m3": GDN_FP8_E4M3, "int8": GDN_INT8, "int16": GDN_INT16}
_TORCH_DTYPE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


class gdn_blocks(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("K", ctypes.c_void_p), ("k_dtype", ctypes.c_int32),
                ("g_cumulative", ctypes.c_int32), ("beta", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("n_blocks", ctypes.c_int64), ("C", ctypes.c_int32),
                ("d_k", ctypes.c_int32)]


class gdn_inverse_cfg(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("N", ctypes.c_int32), ("mask", ctypes.c_int32),
                ("compute", ctypes.c_int32)]


_vp, _i32, _i64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
_P = ctypes.POINTER
_lib.gdn_abi_version.restype = ctypes.c_int
_lib.gdn_status_string.restype = ctypes.c_char_p
_lib.gdn_status_string.argtypes = [_i32]
_lib.gdn_build_A.restype = _i32
_lib.gdn_build_A.argtypes = [_P(gdn_blocks), _vp, _vp]
_lib.gdn_tri_inverse_neumann.restype = _i32
_lib.gdn_tri_inverse_neumann.argtypes = [_P(gdn_blocks), _i32, _i32, _i32, _vp, _i32, _vp, _vp]
_lib.gdn_tri_inverse_exact.restype = _i32
_lib.gdn_tri_inverse_exact.argtypes = [_P(gdn_blocks), _i32, _vp, _i32, _vp]
_lib.gdn_tri_inverse_residual.restype = _i32
_lib.gdn_tri_inverse_residual.argtypes = [_P(gdn_blocks), _i32, _i32, _i32, _i32, _vp, _i32, _vp]
_lib.gdn_tri_inverse_fs.restype = _i32
_lib.gdn_tri_inverse_fs.argtypes = [_P(gdn_blocks), _vp, _i32, _vp]
_lib.gdn_wy.restype = _i32
_lib.gdn_wy.argtypes = [_P(gdn_blocks), _vp, _i32, _P(gdn_inverse_cfg), _vp, _i32, _i32, _vp, _vp,
                        _i32, _vp]
_lib.gdn_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
_lib.gdn_chunk_fwd_workspace_bytes.argtypes = [_i32, _i32, _i64, _i32, _i32, _i32, _P(gdn_inverse_cfg)]
_lib.gdn_chunk_fwd.restype = _i32
_lib.gdn_chunk_fwd.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                               _i64, _i32, _i32, _i32, _f32, _P(gdn_inverse_cfg), _vp, ctypes.c_size_t,
                               _vp, _vp]
_lib.gdn_chunk_fwd_noalloc.restype = _i32
_lib.gdn_chunk_fwd_noalloc.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                       _i64, _i32, _i32, _i32, _f32, _P(gdn_inverse_cfg), _vp, _vp]
_lib.gdn_decode.restype = _i32
_lib.gdn_decode.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                            _i32, _i32, _f32, _vp]

EXPORTED = ("gdn_abi_version", "gdn_status_string", "gdn_build_A", "gdn_tri_inverse_neumann",
            "gdn_tri_inverse_exact", "gdn_tri_inverse_residual", "gdn_tri_inverse_fs", "gdn_wy",
            "gdn_chunk_fwd_workspace_bytes", "gdn_chunk_fwd", "gdn_chunk_fwd_noalloc", "gdn_decode")
GDN_NOALLOC_SCRATCH_BYTES = 64 << 20


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, gdn_status_string(status)))


def gdn_abi_version() -> int:
    return int(_lib.gdn_abi_version())


def gdn_status_string(status: int) -> str:
    return _lib.gdn_status_string(int(status)).decode()


def _check(st: int, where: str) -> None:
    if st != GDN_OK:
        raise GdnError(st, where)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a CUDA (HIP) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    return t


def _compute_code(compute) -> int:
    if isinstance(compute, int):
        return compute
    return _COMPUTE[str(compute)]


def _blocks(A=None, K=None, beta=None, g=None, C=64, g_cumulative=False):
    """Build the gdn_blocks descriptor; returns (desc, n_blocks, d_k)."""
    d = gdn_blocks()
    if A is not None:
        _dev(A, "A", (torch.float32,))
        if A.dim() < 2 or A.shape[-1] != C or A.shape[-2] != C:
            raise ValueError("A must end in [C, C]")
        nb = A.numel() // (C * C)
        d.A, d.n_blocks, d.C, d.d_k = A.data_ptr(), nb, C, 0
        return d, nb, 0
    _dev(K, "K", (torch.bfloat16, torch.float32))
    _dev(beta, "beta", (torch.float32,))
    _dev(g, "g", (torch.float32,))
    dk = K.shape[-1]
    rows = K.numel() // dk
    if rows % C != 0:
        raise ValueError("K has %d rows, not a multiple of C=%d" % (rows, C))
    nb = rows // C
    if beta.numel() != rows or g.numel() != rows:
        raise ValueError("beta and g need one value per K row")
    d.A = None
    d.K = K.data_ptr()
    d.k_dtype = _TORCH_DTYPE[K.dtype]
    d.g_cumulative = int(bool(g_cumulative))
    d.beta, d.g = beta.data_ptr(), g.data_ptr()
    d.n_blocks, d.C, d.d_k = nb, C, dk
    return d, nb, dk


def gdn_build_A(K, beta, g, C: int = 64, g_cumulative: bool = False, out=None, stream=None):
    """A = -tril(diag(beta)(K K^T .* exp(G_i - G_j)), -1) per C-row block -> [n_blocks, C, C] fp32."""
    d, nb, _ = _blocks(K=K, beta=beta, g=g, C=C, g_cumulative=g_cumulative)
    if out is None:
        out = torch.empty((nb, C, C), device=K.device, dtype=torch.float32)
    _dev(out, "out", (torch.float32,))
    _check(_lib.gdn_build_A(ctypes.byref(d), _ptr(out), _stream(stream)), "gdn_build_A")
    return out


def gdn_tri_inverse_neumann(A=None, K=None, beta=None, g=None, C: int = 64, N: int = 3,
                            mask: bool = True, compute="bf16", t_dtype=torch.float32,
                            g_cumulative: bool = False, stats=None, out=None, stream=None):
    """Truncated (optionally band-masked) Neumann inverse per block -> T [n_blocks, C, C].

    Give either A ([.., C, C] fp32) or K/beta/g.  stats: optional CUDA int64 tensor of 4
    (fp8 diagnostics; zeroed then accumulated on the stream)."""
    d, nb, _ = _blocks(A, K, beta, g, C, g_cumulative)
    dev = (A if A is not None else K).device
    if out is None:
        out = torch.empty((nb, C, C), device=dev, dtype=t_dtype)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    if stats is not None:
        _dev(stats, "stats", (torch.int64,))
        if stats.numel() < 4:
            raise ValueError("stats needs 4 elements")
    st = _lib.gdn_tri_inverse_neumann(ctypes.byref(d), int(N), int(bool(mask)),
                                      _compute_code(compute), _ptr(out), _TORCH_DTYPE[out.dtype],
                                      _ptr(stats), _stream(stream))
    _check(st, "gdn_tri_inverse_neumann")
    return out


def gdn_tri_inverse_exact(A=None, K=None, beta=None, g=None, C: int = 64, compute="bf16",
                          t_dtype=torch.float32, g_cumulative: bool = False, out=None, stream=None):
    """Exact doubling-product inverse per block -> T [n_blocks, C, C]."""
    d, nb, _ = _blocks(A, K, beta, g, C, g_cumulative)
    dev = (A if A is not None else K).device
    if out is None:
        out = torch.empty((nb, C, C), device=dev, dtype=t_dtype)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    st = _lib.gdn_tri_inverse_exact(ctypes.byref(d), _compute_code(compute), _ptr(out),
                                    _TORCH_DTYPE[out.dtype], _stream(stream))
    _check(st, "gdn_tri_inverse_exact")
    return out


def gdn_tri_inverse_residual(A=None, K=None, beta=None, g=None, C: int = 64, N: int = 3,
                             mask: bool = True, S: int = 8, compute="f32", t_dtype=torch.float32,
                             g_cumulative: bool = False, out=None, stream=None):
    """Truncated (optionally band-masked) Neumann sum refined by the parallel residual
    correction T = T0 sum_{s<=S} E^s, E = I - (I - A) T0 -> T [n_blocks, C, C]."""
    d, nb, _ = _blocks(A, K, beta, g, C, g_cumulative)
    dev = (A if A is not None else K).device
    if out is None:
        out = torch.empty((nb, C, C), device=dev, dtype=t_dtype)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    st = _lib.gdn_tri_inverse_residual(ctypes.byref(d), int(N), int(bool(mask)), int(S),
                                       _compute_code(compute), _ptr(out), _TORCH_DTYPE[out.dtype],
                                       _stream(stream))
    _check(st, "gdn_tri_inverse_residual")
    return out


def gdn_tri_inverse_fs(A=None, K=None, beta=None, g=None, C: int = 64, t_dtype=torch.float32,
                       g_cumulative: bool = False, out=None, stream=None):
    """Forward substitution (fp32), the sequential baseline -> T [n_blocks, C, C]."""
    d, nb, _ = _blocks(A, K, beta, g, C, g_cumulative)
    dev = (A if A is not None else K).device
    if out is None:
        out = torch.empty((nb, C, C), device=dev, dtype=t_dtype)
    _dev(out, "out", (torch.float32, torch.bfloat16))
    st = _lib.gdn_tri_inverse_fs(ctypes.byref(d), _ptr(out), _TORCH_DTYPE[out.dtype], _stream(stream))
    _check(st, "gdn_tri_inverse_fs")
    return out


def _inv_cfg(mode, N, mask, compute):
    c = gdn_inverse_cfg()
    if mode in ("exact", GDN_INV_EXACT):
        c.mode = GDN_INV_EXACT
    elif mode in ("neumann_products", GDN_INV_NEUMANN_PRODUCTS):
        c.mode = GDN_INV_NEUMANN_PRODUCTS
    else:
        c.mode = GDN_INV_NEUMANN
    c.N, c.mask, c.compute = int(N), int(bool(mask)), _compute_code(compute)
    return c


def gdn_wy(K, beta, g, V, C: int = 64, T=None, mode="neumann", N: int = 3, mask: bool = True,
           compute="bf16", gate_k: bool = False, out_dtype=torch.bfloat16,
           g_cumulative: bool = False, W_out=None, U_out=None, stream=None):
    """WY products per block: W = T diag(s) K, U = T diag(beta) V (s = beta, or beta*e^G
    with gate_k).  T given ([n_blocks, C, C] fp32/bf16) or formed on the fly."""
    d, nb, dk = _blocks(None, K, beta, g, C, g_cumulative)
    _dev(V, "V", (torch.bfloat16,))
    dv = V.shape[-1]
    if V.numel() != nb * C * dv:
        raise ValueError("V must hold n_blocks * C rows")
    if T is not None:
        _dev(T, "T", (torch.float32, torch.bfloat16))
        if T.numel() != nb * C * C:
            raise ValueError("T must be [n_blocks, C, C]")
    if W_out is None:
        W_out = torch.empty((nb, C, dk), device=K.device, dtype=out_dtype)
    if U_out is None:
        U_out = torch.empty((nb, C, dv), device=K.device, dtype=out_dtype)
    _dev(W_out, "W_out", (torch.float32, torch.bfloat16))
    _dev(U_out, "U_out", (W_out.dtype,))
    cfg = _inv_cfg(mode, N, mask, compute)
    st = _lib.gdn_wy(ctypes.byref(d), _ptr(T), _TORCH_DTYPE[T.dtype] if T is not None else 0,
                     ctypes.byref(cfg), _ptr(V), int(dv), int(bool(gate_k)), _ptr(W_out),
                     _ptr(U_out), _TORCH_DTYPE[W_out.dtype], _stream(stream))
    _check(st, "gdn_wy")
    return W_out, U_out


def gdn_chunk_fwd_workspace_bytes(B: int, H: int, T: int, d_k: int, d_v: int, C: int = 64,
                                  mode="neumann", N: int = 3, mask: bool = True, compute="bf16") -> int:
    """Device workspace (bytes) gdn_chunk_fwd needs for these arguments (0: none)."""
    cfg = _inv_cfg(mode, N, mask, compute)
    return int(_lib.gdn_chunk_fwd_workspace_bytes(int(B), int(H), int(T), int(d_k), int(d_v), int(C),
                                                  ctypes.byref(cfg)))


def gdn_chunk_fwd(Q, K, V, beta, g, C: int = 64, scale: float | None = None, S0=None,
                  mode="neumann", N: int = 3, mask: bool = True, compute="bf16",
                  o_dtype=torch.bfloat16, stats=None, O=None, S_out=None, workspace=None, stream=None):
    """Chunk-wise gated delta rule forward.  Q, K [B,H,T,d_k], V [B,H,T,d_v] bf16;
    beta, g [B,H,T] fp32 -> (O [B,H,T,d_v], S_out [B,H,d_k,d_v] fp32).

    workspace: a CUDA uint8 tensor of at least gdn_chunk_fwd_workspace_bytes(...) bytes,
    or None to have one allocated here (through torch) when the variant needs it."""
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, n, (torch.bfloat16,))
    _dev(beta, "beta", (torch.float32,))
    _dev(g, "g", (torch.float32,))
    if K.dim() != 4 or Q.shape != K.shape:
        raise ValueError("Q and K must both be [B, H, T, d_k]")
    B, H, T, dk = K.shape
    dv = V.shape[-1]
    if V.shape[:3] != (B, H, T) or beta.shape != (B, H, T) or g.shape != (B, H, T):
        raise ValueError("V, beta, g must match Q/K in [B, H, T]")
    if S0 is not None:
        _dev(S0, "S0", (torch.float32,))
        if S0.shape != (B, H, dk, dv):
            raise ValueError("S0 must be [B, H, d_k, d_v]")
    if O is None:
        O = torch.empty((B, H, T, dv), device=K.device, dtype=o_dtype)
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), device=K.device, dtype=torch.float32)
    _dev(O, "O", (torch.float32, torch.bfloat16))
    _dev(S_out, "S_out", (torch.float32,))
    if stats is not None:
        _dev(stats, "stats", (torch.int64,))
        if stats.numel() < 4:
            raise ValueError("stats needs 4 elements")
    if scale is None:
        scale = dk ** -0.5
    cfg = _inv_cfg(mode, N, mask, compute)
    need = int(_lib.gdn_chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, ctypes.byref(cfg)))
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=K.device, dtype=torch.uint8)
    if workspace is not None:
        _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = _lib.gdn_chunk_fwd(_ptr(Q), _ptr(K), _ptr(V), GDN_BF16, _ptr(beta), _ptr(g), _ptr(S0),
                            _ptr(O), _TORCH_DTYPE[O.dtype], _ptr(S_out), B, H, T, dk, dv, C,
                            float(scale), ctypes.byref(cfg), _ptr(workspace), ws_bytes, _ptr(stats),
                            _stream(stream))
    _check(st, "gdn_chunk_fwd")
    return O, S_out


def gdn_chunk_fwd_noalloc(Q, K, V, beta, g, C: int = 64, scale: float | None = None, S0=None,
                          mode="neumann", N: int = 3, mask: bool = True, compute="bf16",
                          o_dtype=torch.bfloat16, stats=None, O=None, S_out=None, stream=None):
    """gdn_chunk_fwd with the library's fixed device scratch instead of a workspace
    (for callers that cannot allocate).  Arguments and results as gdn_chunk_fwd; O and
    S_out are still the caller's (pass them to allocate nothing here either)."""
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, n, (torch.bfloat16,))
    _dev(beta, "beta", (torch.float32,))
    _dev(g, "g", (torch.float32,))
    if K.dim() != 4 or Q.shape != K.shape:
        raise ValueError("Q and K must both be [B, H, T, d_k]")
    B, H, T, dk = K.shape
    dv = V.shape[-1]
    if V.shape[:3] != (B, H, T) or beta.shape != (B, H, T) or g.shape != (B, H, T):
        raise ValueError("V, beta, g must match Q/K in [B, H, T]")
    if S0 is not None:
        _dev(S0, "S0", (torch.float32,))
    if O is None:
        O = torch.empty((B, H, T, dv), device=K.device, dtype=o_dtype)
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), device=K.device, dtype=torch.float32)
    _dev(O, "O", (torch.float32, torch.bfloat16))
    _dev(S_out, "S_out", (torch.float32,))
    if stats is not None:
        _dev(stats, "stats", (torch.int64,))
    if scale is None:
        scale = dk ** -0.5
    cfg = _inv_cfg(mode, N, mask, compute)
    st = _lib.gdn_chunk_fwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), GDN_BF16, _ptr(beta), _ptr(g), _ptr(S0),
                                    _ptr(O), _TORCH_DTYPE[O.dtype], _ptr(S_out), B, H, T, dk, dv, C,
                                    float(scale), ctypes.byref(cfg), _ptr(stats), _stream(stream))
    _check(st, "gdn_chunk_fwd_noalloc")
    return O, S_out


def gdn_decode(Q, K, V, beta, g, S=None, scale: float | None = None, S_out=None, O=None,
               o_dtype=torch.bfloat16, stream=None):
    """Gated delta rule token by token with the state kept on chip for all n tokens.
    Q, K [B,H,n,d_k], V [B,H,n,d_v] (bf16 or fp32, one dtype); beta, g [B,H,n] fp32;
    S [B,H,d_k,d_v] fp32 or None (zeros).  Pass S_out=S to update the state in place.
    Returns (O [B,H,n,d_v], S_out [B,H,d_k,d_v] fp32)."""
    for t, n_ in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, n_, (torch.bfloat16, torch.float32))
    if not (Q.dtype == K.dtype == V.dtype):
        raise ValueError("Q, K and V must share one dtype")
    _dev(beta, "beta", (torch.float32,))
    _dev(g, "g", (torch.float32,))
    if K.dim() != 4 or Q.shape != K.shape:
        raise ValueError("Q and K must both be [B, H, n, d_k]")
    B, H, n, dk = K.shape
    dv = V.shape[-1]
    if V.shape[:3] != (B, H, n) or beta.shape != (B, H, n) or g.shape != (B, H, n):
        raise ValueError("V, beta, g must match Q/K in [B, H, n]")
    if S is not None:
        _dev(S, "S", (torch.float32,))
        if S.shape != (B, H, dk, dv):
            raise ValueError("S must be [B, H, d_k, d_v]")
    if O is None:
        O = torch.empty((B, H, n, dv), device=K.device, dtype=o_dtype)
    if S_out is None:
        S_out = torch.empty((B, H, dk, dv), device=K.device, dtype=torch.float32)
    _dev(O, "O", (torch.float32, torch.bfloat16))
    _dev(S_out, "S_out", (torch.float32,))
    if scale is None:
        scale = dk ** -0.5
    st = _lib.gdn_decode(_ptr(Q), _ptr(K), _ptr(V), _TORCH_DTYPE[K.dtype], _ptr(beta), _ptr(g),
                         _ptr(S), _ptr(S_out), _ptr(O), _TORCH_DTYPE[O.dtype], B, H, n, dk, dv,
                         float(scale), _stream(stream))
    _check(st, "gdn_decode")
    return O, S_out
