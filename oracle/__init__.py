"""fp64 CPU oracle for the chunk-wise Gated DeltaNet intra-chunk solve.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
(``tri_inverse_amd``) never imports, links or calls it, and the two share no code.

The arithmetic lives in ``gdn_oracle.c`` (plain fp64 C loops, OpenMP over independent
blocks or heads); this module only builds it with gcc and marshals numpy arrays.
Every function takes and returns float64 arrays; callers upcast bf16/fp32 inputs
exactly (every bf16 and fp32 value is representable in fp64).

Pages cited (titles): [GEO] "When Good Enough Is Optimal: Multiplication-Only Matrix
Inversion Approximation for Quantized Gated DeltaNet"; [PSDA] "A Persistent-State
Dataflow Accelerator for Memory-Bound Linear Attention Decode on FPGA".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

INV_NEUMANN = 0
INV_EXACT = 1
INV_FS = 2
INV_FP8 = 3


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into liboracle.so with gcc (fp64, no fast-math)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(ctypes.c_double)
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_version.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_max_threads.restype = i32
    lib.oracle_build_A.argtypes = [i64, i32, i32, P, P, P, i32, P]
    lib.oracle_fs_inverse.argtypes = [i64, i32, P, P]
    lib.oracle_neumann.argtypes = [i64, i32, P, i32, i32, P]
    lib.oracle_doubling.argtypes = [i64, i32, P, P]
    lib.oracle_neumann_int8.argtypes = [i64, i32, P, i32, i32, P]
    lib.oracle_neumann_int16.argtypes = [i64, i32, P, i32, i32, P]
    U64P = ctypes.POINTER(ctypes.c_uint64)
    lib.oracle_neumann_fp8.argtypes = [i64, i32, P, i32, i32, P, U64P, P]
    lib.oracle_e4m3_round.argtypes = [i64, P, P]
    lib.oracle_residual.argtypes = [i64, i32, P, i32, i32, i32, P]
    lib.oracle_wy.argtypes = [i64, i32, i32, i32, P, P, P, P, P, i32, i32, P, P]
    lib.oracle_chunk_fwd.argtypes = [i32, i32, i64, i32, i32, i32, P, P, P, P, P, P, f64,
                                     i32, i32, i32, P, P]
    lib.oracle_recurrence.argtypes = [i32, i32, i64, i32, i32, P, P, P, P, P, P, f64, P, P]
    for fn in ("oracle_build_A", "oracle_fs_inverse", "oracle_neumann", "oracle_neumann_int8",
               "oracle_neumann_int16",
               "oracle_neumann_fp8", "oracle_e4m3_round",
               "oracle_doubling",
               "oracle_residual", "oracle_wy", "oracle_chunk_fwd", "oracle_recurrence",
               "oracle_set_threads"):
        getattr(lib, fn).restype = None
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def build_A(K, beta, g, g_cumulative: bool = False) -> np.ndarray:
    """A = -tril(diag(beta)(K K^T .* exp(G_i - G_j)), -1) per block.

    K: [nb, C, dk]; beta, g: [nb, C] ([GEO] problem statement: A strictly lower)."""
    K, beta, g = _f64(K), _f64(beta), _f64(g)
    nb, C, dk = K.shape
    assert beta.shape == (nb, C) and g.shape == (nb, C)
    A = np.empty((nb, C, C))
    _load().oracle_build_A(nb, C, dk, _ptr(K), _ptr(beta), _ptr(g), int(bool(g_cumulative)), _ptr(A))
    return A


def fs_inverse(A) -> np.ndarray:
    """T = (I - A)^-1 by forward substitution ([GEO] problem statement baseline)."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    _load().oracle_fs_inverse(nb, C, _ptr(A), _ptr(T))
    return T


def neumann(A, N: int, mask: bool) -> np.ndarray:
    """Truncated sum_{n<=N} A^n (Horner), optionally band-masked ([GEO] Methodologie 1-2)."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    _load().oracle_neumann(nb, C, _ptr(A), int(N), int(bool(mask)), _ptr(T))
    return T


def neumann_int8(A, N: int, mask: bool) -> np.ndarray:
    """The Horner chain on int8 codes with per-block power-of-two scales ([GEO]
    "Adaptation a la Quantification"; reading in gdn_oracle.c).  A holds fp32 values."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    _load().oracle_neumann_int8(nb, C, _ptr(A), int(N), int(bool(mask)), _ptr(T))
    return T


def neumann_int16(A, N: int, mask: bool) -> np.ndarray:
    """The same chain on 16-bit codes (|code| <= 32639 = 127 * 257, two signed 8-bit digits),
    each sum formed in fp64 and rounded to fp32 ([GEO] "Adaptation a la Quantification";
    reading in gdn_oracle.c).  A holds fp32 values."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    _load().oracle_neumann_int16(nb, C, _ptr(A), int(N), int(bool(mask)), _ptr(T))
    return T


def e4m3_round(y) -> np.ndarray:
    """Nearest OCP e4m3 value of each element (|y| <= 448), ties to the even code."""
    y = _f64(y)
    q = np.empty_like(y)
    _load().oracle_e4m3_round(y.size, _ptr(y), _ptr(q))
    return q


def neumann_fp8(A, N: int, mask: bool):
    """The Horner chain on fp8 e4m3 operands with per-block absmax/448 scales ([GEO]
    "Adaptation a la Quantification"; reading in gdn_oracle.c).  A holds fp32 values.
    Returns (T [nb,C,C], counts [nb,4] uint64: non-finite, dynamic-scale saturations,
    static-scale saturations, underflows; amax [nb,N+1]: absmax of A, X_1..X_{N-1}, X_N)."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    counts = np.zeros((nb, 4), dtype=np.uint64)
    amax = np.zeros((nb, int(N) + 1))
    _load().oracle_neumann_fp8(nb, C, _ptr(A), int(N), int(bool(mask)), _ptr(T),
                               counts.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), _ptr(amax))
    return T, counts, amax


def doubling(A) -> np.ndarray:
    """Exact prod_i (I + A^(2^i)), valid because A is nilpotent."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    _load().oracle_doubling(nb, C, _ptr(A), _ptr(T))
    return T


def residual(A, N: int, mask: bool, S: int) -> np.ndarray:
    """T(0) sum_{s<=S} E^s with E = I - (I - A) T(0) ([GEO] Methodologie 3)."""
    A = _f64(A)
    nb, C, _ = A.shape
    T = np.empty_like(A)
    _load().oracle_residual(nb, C, _ptr(A), int(N), int(bool(mask)), int(S), _ptr(T))
    return T


def wy(T, K, V, beta, g, gate_k: bool, g_cumulative: bool = False):
    """W = T diag(s) K, U = T diag(beta) V; s = beta, or beta*exp(G) when gate_k."""
    T, K, V, beta, g = _f64(T), _f64(K), _f64(V), _f64(beta), _f64(g)
    nb, C, dk = K.shape
    dv = V.shape[2]
    W = np.empty((nb, C, dk))
    U = np.empty((nb, C, dv))
    _load().oracle_wy(nb, C, dk, dv, _ptr(T), _ptr(K), _ptr(V), _ptr(beta), _ptr(g),
                      int(bool(g_cumulative)), int(bool(gate_k)), _ptr(W), _ptr(U))
    return W, U


def chunk_fwd(Q, K, V, beta, g, C: int, scale: float, inv_mode: int = INV_NEUMANN,
              N: int = 3, mask: bool = True, S0=None):
    """Chunk-wise forward: returns (O [B,H,T,dv], S_out [B,H,dk,dv])."""
    Q, K, V, beta, g = _f64(Q), _f64(K), _f64(V), _f64(beta), _f64(g)
    B, H, Tn, dk = K.shape
    dv = V.shape[3]
    assert Tn % C == 0
    O = np.empty((B, H, Tn, dv))
    S_out = np.empty((B, H, dk, dv))
    s0 = _f64(S0) if S0 is not None else None
    s0p = _ptr(s0) if s0 is not None else ctypes.POINTER(ctypes.c_double)()
    _load().oracle_chunk_fwd(B, H, Tn, dk, dv, C, _ptr(Q), _ptr(K), _ptr(V), _ptr(beta),
                             _ptr(g), s0p, float(scale), int(inv_mode), int(N),
                             int(bool(mask)), _ptr(O), _ptr(S_out))
    return O, S_out


def recurrence(Q, K, V, beta, g, scale: float, S0=None):
    """Token-by-token gated delta rule: returns (O, S_out)."""
    Q, K, V, beta, g = _f64(Q), _f64(K), _f64(V), _f64(beta), _f64(g)
    B, H, Tn, dk = K.shape
    dv = V.shape[3]
    O = np.empty((B, H, Tn, dv))
    S_out = np.empty((B, H, dk, dv))
    s0 = _f64(S0) if S0 is not None else None
    s0p = _ptr(s0) if s0 is not None else ctypes.POINTER(ctypes.c_double)()
    _load().oracle_recurrence(B, H, Tn, dk, dv, _ptr(Q), _ptr(K), _ptr(V), _ptr(beta),
                              _ptr(g), s0p, float(scale), _ptr(O), _ptr(S_out))
    return O, S_out
