"""C-ABI checks that run without a GPU: the library loads, exports every symbol the
header declares, and every validation path returns its documented status before any
HIP call is made (all pointers below are fake host addresses that are never touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tri = pytest.importorskip("tri_inverse_amd", reason="libgdn.so not built")
lib = tri._lib


def header_functions():
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_A-Z0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert "gdn_chunk_fwd" in names and "gdn_tri_inverse_neumann" in names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(tri.EXPORTED)


def test_version_and_status_strings():
    assert tri.gdn_abi_version() == 2
    for s in range(8):
        assert tri.gdn_status_string(s).startswith("GDN_")
    assert "unknown" in tri.gdn_status_string(99)


FAKE = 0x10000  # aligned, never dereferenced: validation fails or returns before use


def blocks(**kw):
    d = tri.gdn_blocks()
    d.A = kw.get("A", None)
    d.K = kw.get("K", FAKE)
    d.k_dtype = kw.get("k_dtype", tri.GDN_BF16)
    d.g_cumulative = 0
    d.beta = kw.get("beta", FAKE)
    d.g = kw.get("g", FAKE)
    d.n_blocks = kw.get("n_blocks", 4)
    d.C = kw.get("C", 64)
    d.d_k = kw.get("d_k", 128)
    return d


def neumann(d, N=3, mask=1, compute=tri.GDN_BF16, T=FAKE, t_dtype=tri.GDN_F32, stats=None):
    return lib.gdn_tri_inverse_neumann(ctypes.byref(d) if d is not None else None, N, mask, compute,
                                       T, t_dtype, stats, None)


def test_neumann_validation():
    assert neumann(None) == 1                                   # NULL descriptor
    assert neumann(blocks(K=None)) == 1                         # NULL K
    assert neumann(blocks(), T=None) == 1                       # NULL output
    assert neumann(blocks(C=48)) == 5                           # unsupported chunk
    assert neumann(blocks(d_k=48)) == 5                         # unsupported head dim
    assert neumann(blocks(n_blocks=-1)) == 2                    # negative size
    assert neumann(blocks(), N=0) == 2                          # N out of range
    assert neumann(blocks(), N=64) == 2
    assert neumann(blocks(), mask=2) == 2
    assert neumann(blocks(), compute=7) == 3                    # bad dtype codes
    assert neumann(blocks(), t_dtype=tri.GDN_FP8_E4M3) == 3
    assert neumann(blocks(k_dtype=9)) == 3
    assert neumann(blocks(k_dtype=tri.GDN_F32)) == 5            # fp32 K only for build_A
    assert neumann(blocks(K=FAKE + 2)) == 4                     # misaligned
    assert neumann(blocks(), T=FAKE + 8) == 4
    assert neumann(blocks(n_blocks=0)) == 0                     # empty batch: nothing launched
    assert neumann(blocks(A=FAKE, K=None, beta=None, g=None, n_blocks=0)) == 0
    assert neumann(blocks(K=None, beta=None, g=None, n_blocks=0), T=None) == 0  # NULLs allowed when empty
    assert neumann(blocks(n_blocks=0), N=0) == 2                # sizes still validated


def test_exact_and_build_A_validation():
    ex = lambda d, compute=tri.GDN_BF16, T=FAKE: lib.gdn_tri_inverse_exact(
        ctypes.byref(d), compute, T, tri.GDN_F32, None)
    assert ex(blocks(), compute=tri.GDN_FP8_E4M3) == 5
    assert ex(blocks(C=24)) == 5
    assert ex(blocks(), T=None) == 1
    assert ex(blocks(n_blocks=0)) == 0
    bA = lambda d, out=FAKE: lib.gdn_build_A(ctypes.byref(d), out, None)
    assert bA(blocks(A=FAKE)) == 5                               # A is the output here
    assert bA(blocks(), out=None) == 1
    assert bA(blocks(beta=None)) == 1
    assert bA(blocks(n_blocks=0)) == 0
    assert bA(blocks(n_blocks=0, k_dtype=tri.GDN_F32)) == 0


def test_large_chunk_routing():
    """C = 128 and 256 take bf16 keys and bf16 products: the masked sum with N <= 16 on
    the band kernel, every other Neumann / exact / given-T request on the full-triangle
    kernel.  fp32 or fp8 products, A given, or head sizes outside {64, 128} report
    GDN_ERR_UNSUPPORTED (5) up front; sizes are still range-checked (2)."""
    for C in (128, 256):
        assert neumann(blocks(C=C, n_blocks=0)) == 0
        assert neumann(blocks(C=C, n_blocks=0), N=17) == 0            # full-triangle kernel
        assert neumann(blocks(C=C, n_blocks=0), mask=0) == 0
        assert neumann(blocks(C=C, n_blocks=0), compute=tri.GDN_F32) == 5
        assert neumann(blocks(C=C, n_blocks=0), compute=tri.GDN_FP8_E4M3) == 5
        assert neumann(blocks(C=C, n_blocks=0, A=FAKE, K=None, beta=None, g=None)) == 5  # A given
        assert neumann(blocks(C=C), N=C) == 2                         # N still range-checked
        ex = lib.gdn_tri_inverse_exact(ctypes.byref(blocks(C=C, n_blocks=0)), tri.GDN_BF16, FAKE,
                                       tri.GDN_F32, None)
        assert ex == 0
        ex = lib.gdn_tri_inverse_exact(ctypes.byref(blocks(C=C, n_blocks=0)), tri.GDN_F32, FAKE,
                                       tri.GDN_F32, None)
        assert ex == 5
    inv = tri.gdn_inverse_cfg()
    inv.mode, inv.N, inv.mask, inv.compute = tri.GDN_INV_NEUMANN, 3, 1, tri.GDN_BF16
    wy = lambda d, T=None, inv=inv, d_v=128: lib.gdn_wy(ctypes.byref(d), T, tri.GDN_F32, ctypes.byref(inv),
                                                          FAKE, d_v, 0, FAKE, FAKE, tri.GDN_BF16, None)
    for C in (128, 256):
        assert wy(blocks(C=C, n_blocks=0)) == 0
        assert wy(blocks(C=C, n_blocks=0), T=FAKE) == 0               # given T: full-triangle kernel
        assert wy(blocks(C=C, n_blocks=0), d_v=96) == 5
        assert wy(blocks(C=C, n_blocks=0, d_k=256)) == 5
    inv.mask = 0
    assert wy(blocks(C=128, n_blocks=0)) == 0
    inv.compute = tri.GDN_FP8_E4M3
    assert wy(blocks(C=128, n_blocks=0)) == 5


def test_residual_validation():
    res = lambda d, N=3, mask=1, S=8, compute=tri.GDN_F32, T=FAKE: lib.gdn_tri_inverse_residual(
        ctypes.byref(d) if d is not None else None, N, mask, S, compute, T, tri.GDN_F32, None)
    assert res(None) == 1
    assert res(blocks(), T=None) == 1
    assert res(blocks(), S=-1) == 2
    assert res(blocks(), S=65) == 2
    assert res(blocks(), N=0) == 2
    assert res(blocks(), mask=3) == 2
    assert res(blocks(), compute=9) == 3
    assert res(blocks(), compute=tri.GDN_BF16) == 5            # E needs fp32 products
    assert res(blocks(C=128, n_blocks=0)) == 5
    assert res(blocks(n_blocks=0)) == 0
    assert res(blocks(A=FAKE, K=None, beta=None, g=None, n_blocks=0), S=0) == 0


def test_fs_validation():
    fs = lambda d, T=FAKE, t=tri.GDN_F32: lib.gdn_tri_inverse_fs(ctypes.byref(d) if d is not None else None,
                                                                  T, t, None)
    assert fs(None) == 1
    assert fs(blocks(), T=None) == 1
    assert fs(blocks(), t=tri.GDN_FP8_E4M3) == 3
    assert fs(blocks(C=128, n_blocks=0)) == 0
    assert fs(blocks(C=256, n_blocks=0)) == 5
    assert fs(blocks(C=128, d_k=256, n_blocks=0)) == 5
    assert fs(blocks(n_blocks=0)) == 0
    assert fs(blocks(), T=FAKE + 4) == 4


def test_decode_validation():
    def dec(Q=FAKE, S_in=None, S_out=FAKE, qd=tri.GDN_BF16, od=tri.GDN_BF16, B=1, H=1, n=1,
            dk=128, dv=128):
        return lib.gdn_decode(Q, FAKE, FAKE, qd, FAKE, FAKE, S_in, S_out, FAKE, od, B, H, n, dk,
                              dv, 1.0, None)
    assert dec(B=-1) == 2
    assert dec(n=-1) == 2
    assert dec(qd=tri.GDN_FP8_E4M3) == 3
    assert dec(od=tri.GDN_FP8_E4M3) == 3
    assert dec(dk=96) == 5
    assert dec(dv=48) == 5
    assert dec(dv=288) == 5
    assert dec(B=0) == 0
    assert dec(S_out=None) == 1
    assert dec(Q=None) == 1
    assert dec(S_in=FAKE + 8) == 4


def test_int8_compute_routing():
    """int8 and int16 compute are accepted by the Neumann entry point at C <= 64 only."""
    neu = lambda d, c: lib.gdn_tri_inverse_neumann(ctypes.byref(d), 3, 1, c, FAKE, tri.GDN_F32,
                                                   None, None)
    assert neu(blocks(n_blocks=0), tri.GDN_INT8) == 0
    assert neu(blocks(n_blocks=0), tri.GDN_INT16) == 0
    assert neu(blocks(C=128, n_blocks=0), tri.GDN_INT16) == 5
    assert lib.gdn_tri_inverse_exact(ctypes.byref(blocks(n_blocks=0)), tri.GDN_INT16, FAKE,
                                      tri.GDN_F32, None) == 5
    assert neu(blocks(n_blocks=0), 9) == 3
    assert neu(blocks(C=128, n_blocks=0), tri.GDN_INT8) == 5
    assert lib.gdn_tri_inverse_exact(ctypes.byref(blocks(n_blocks=0)), tri.GDN_INT8, FAKE,
                                      tri.GDN_F32, None) == 5
    assert lib.gdn_tri_inverse_residual(ctypes.byref(blocks(n_blocks=0)), 3, 1, 8, tri.GDN_INT8,
                                        FAKE, tri.GDN_F32, None) == 5


def _inv(mode=tri.GDN_INV_NEUMANN, N=3, mask=1, compute=tri.GDN_BF16):
    c = tri.gdn_inverse_cfg()
    c.mode, c.N, c.mask, c.compute = mode, N, mask, compute
    return c


def test_chunk_fwd_workspace_query():
    """The band path (N <= 3, masked, bf16) needs no workspace; the masked fp8 chain with
    N <= 3 needs 512 bytes per chunk for its band pre-pass's rows; every other variant
    needs 6144 bytes per chunk for the pre-pass's T - I packs; arguments the call would
    reject query as 0."""
    q = lambda inv, B=4, H=16, T=8192, dk=128, dv=128, C=64: lib.gdn_chunk_fwd_workspace_bytes(
        B, H, T, dk, dv, C, ctypes.byref(inv) if inv is not None else None)
    chunks = 4 * 16 * 8192 // 64
    assert q(_inv()) == 0
    assert q(_inv(N=2)) == 0
    assert q(_inv(N=4)) == chunks * 6144
    assert q(_inv(mask=0)) == chunks * 6144
    assert q(_inv(mode=tri.GDN_INV_EXACT)) == chunks * 6144
    assert q(_inv(compute=tri.GDN_FP8_E4M3)) == chunks * 512       # the e4m3 chain in band form
    assert q(_inv(N=2, compute=tri.GDN_FP8_E4M3)) == chunks * 512
    assert q(_inv(N=4, compute=tri.GDN_FP8_E4M3)) == chunks * 6144
    assert q(_inv(mask=0, compute=tri.GDN_FP8_E4M3)) == chunks * 6144
    assert q(_inv(mode=tri.GDN_INV_NEUMANN_PRODUCTS)) == chunks * 6144   # Horner products asked for
    assert q(_inv(mode=tri.GDN_INV_NEUMANN_PRODUCTS, compute=tri.GDN_FP8_E4M3)) == chunks * 6144
    assert q(_inv(mode=3)) == 0
    assert q(None) == 0
    assert q(_inv(), T=100) == 0                     # T % C != 0
    assert q(_inv(), C=32) == 0                      # unsupported chunk size
    assert q(_inv(compute=tri.GDN_F32)) == 0
    assert tri.gdn_chunk_fwd_workspace_bytes(1, 2, 256, 128, 128, mask=False) == 2 * 4 * 6144


def test_chunk_fwd_validation():
    def cf(inv, ws=None, ws_bytes=0, B=1, H=2, T=256, dk=128, dv=128, C=64, Q=FAKE, qd=tri.GDN_BF16,
           od=tri.GDN_BF16, stats=None):
        return lib.gdn_chunk_fwd(Q, FAKE, FAKE, qd, FAKE, FAKE, None, FAKE, od, FAKE, B, H, T, dk, dv, C,
                                 0.1, ctypes.byref(inv) if inv is not None else None, ws, ws_bytes, stats,
                                 None)
    need = 2 * 4 * 6144
    assert cf(None) == 1
    assert cf(_inv(), T=100) == 2
    assert cf(_inv(), qd=tri.GDN_F32) == 5
    assert cf(_inv(), qd=9) == 3
    assert cf(_inv(), C=32) == 5
    assert cf(_inv(), dk=96) == 5
    assert cf(_inv(compute=tri.GDN_FP8_E4M3, mode=tri.GDN_INV_EXACT)) == 5
    assert cf(_inv(), Q=None) == 1
    assert cf(_inv(), stats=FAKE + 8) == 4
    # workspace: needed and missing or short -> GDN_ERR_WORKSPACE (6); misaligned -> 4
    unmasked = _inv(mask=0)
    assert cf(unmasked) == 6
    assert cf(unmasked, ws=FAKE, ws_bytes=need - 1) == 6
    assert cf(unmasked, ws=FAKE + 8, ws_bytes=need) == 4
    assert cf(_inv(mask=0, compute=tri.GDN_FP8_E4M3)) == 6
    assert cf(_inv(compute=tri.GDN_FP8_E4M3)) == 6
    # empty problems enqueue nothing and need no workspace
    assert cf(unmasked, B=0) == 0
    assert cf(unmasked, T=0) == 0
