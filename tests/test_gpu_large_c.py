"""GPU parity of the large-chunk paths (C = 128, 256; also C = 64 where the same call
routes there) against the fp64 oracle running the same algorithm on the same seeded
inputs.

The masked truncated sum with N <= 16 runs as independent 32-row windows, one per
16-row tile; the oracle computes the whole C x C block, so these tests also check the
window argument (entry (i, j) of the masked sum depends on A only on rows and columns
j..i).  Tolerances: relative Frobenius error 2e-3 (bf16 operands) on T, on T - I, and
on W and U.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, eye_off, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")

TOL = 2e-3


def _cumulative(g, C):
    return np.cumsum(f64(g).reshape(-1, C), axis=1)


@pytest.mark.parametrize("C", [128, 256])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 16])
def test_band_inverse_large_chunks(C, N):
    nb = 7   # not a multiple of the 8-way workgroup swizzle
    say(f"band inverse C={C} N={N}")
    inp = synth.blocks(21, nb, C, 128, k_dtype="bf16")
    T = tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C,
                                    N=N, mask=True, compute="bf16", t_dtype=torch.float32)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    Tr = oracle.neumann(A64, N, True)
    T = f64(T)
    assert relF(T, Tr) <= TOL, relF(T, Tr)
    assert relF(eye_off(T), eye_off(Tr)) <= TOL, relF(eye_off(T), eye_off(Tr))
    # outside the band the result is exactly zero, on the diagonal exactly one
    i, j = np.indices((C, C))
    assert np.all(T[:, (i - j > N) | (j > i)] == 0)
    assert np.all(T[:, i == j] == 1)


@pytest.mark.parametrize("C", [128, 256])
def test_band_inverse_cumulative_gates_bf16_out(C):
    nb = 5
    say(f"band inverse cumulative C={C}")
    inp = synth.blocks(22, nb, C, 64, k_dtype="bf16")
    G = _cumulative(inp["g"], C).astype(np.float32)
    T = tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(torch.from_numpy(G)),
                                    C=C, N=3, mask=True, compute="bf16", g_cumulative=True,
                                    t_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), G, g_cumulative=True)
    Tr = oracle.neumann(A64, 3, True)
    assert relF(f64(T), Tr) <= TOL


@pytest.mark.parametrize("C", [128, 256])
@pytest.mark.parametrize("gate_k", [False, True])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
def test_band_wy_large_chunks(C, gate_k, dk, dv):
    nb = 6
    say(f"band wy C={C} gate_k={gate_k} dk={dk} dv={dv}")
    inp = synth.blocks(23, nb, C, dk, k_dtype="bf16", d_v=dv)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]), C=C,
                      mode="neumann", N=3, mask=True, gate_k=gate_k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    T64 = oracle.neumann(A64, 3, True)
    Wr, Ur = oracle.wy(T64, f64(inp["K"]), f64(inp["V"]), f64(inp["beta"]), f64(inp["g"]), gate_k)
    assert relF(f64(W), Wr) <= TOL, relF(f64(W), Wr)
    assert relF(f64(U), Ur) <= TOL, relF(f64(U), Ur)


def test_band_wy_cumulative_key_gate():
    C, nb = 256, 4
    say("band wy cumulative gate_k")
    inp = synth.blocks(24, nb, C, 128, k_dtype="bf16", d_v=128)
    G = _cumulative(inp["g"], C).astype(np.float32)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(torch.from_numpy(G)), cuda(inp["V"]), C=C,
                      mode="neumann", N=2, mask=True, gate_k=True, g_cumulative=True,
                      out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), G, g_cumulative=True)
    T64 = oracle.neumann(A64, 2, True)
    Wr, Ur = oracle.wy(T64, f64(inp["K"]), f64(inp["V"]), f64(inp["beta"]), G, True, g_cumulative=True)
    assert relF(f64(W), Wr) <= TOL
    assert relF(f64(U), Ur) <= TOL


def test_band_wy_full_size_sampled_blocks():
    """B=2, H=16, seq 16384 at C = 256: 2048 blocks, bf16 outputs; 48 blocks checked."""
    C = 256
    nb = 2 * 16 * 16384 // C
    say("band wy full size C=256")
    inp = synth.blocks(2, nb, C, 128, k_dtype="bf16", d_v=128)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]), C=C,
                      mode="neumann", N=3, mask=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = np.random.default_rng(1).choice(nb, 48, replace=False)
    sub = {k: v[idx] for k, v in inp.items()}
    T64 = oracle.neumann(oracle.build_A(f64(sub["K"]), f64(sub["beta"]), f64(sub["g"])), 3, True)
    Wr, Ur = oracle.wy(T64, f64(sub["K"]), f64(sub["V"]), f64(sub["beta"]), f64(sub["g"]), False)
    assert relF(f64(W[idx]), Wr) <= TOL
    assert relF(f64(U[idx]), Ur) <= TOL


@pytest.mark.parametrize("variant", [("neumann", 3, True), ("neumann", 3, False), ("exact", 0, False)])
def test_wy_full_size_C128_sampled_blocks(variant):
    """B=2, H=16, seq 16384 at C = 128 (4096 blocks, bf16 outputs), the launches of the
    chunk-size sweep: band kernel for the masked sum, full-triangle kernel otherwise;
    24 sampled blocks against the oracle."""
    mode, N, mask = variant
    C = 128
    nb = 2 * 16 * 16384 // C
    say(f"wy full size C=128 {variant}")
    inp = synth.blocks(4, nb, C, 128, k_dtype="bf16", d_v=128)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]), C=C,
                      mode=mode, N=max(N, 1), mask=mask, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = np.random.default_rng(5).choice(nb, 24, replace=False)
    sub = {k: v[idx] for k, v in inp.items()}
    A64 = oracle.build_A(f64(sub["K"]), f64(sub["beta"]), f64(sub["g"]))
    T64 = oracle.doubling(A64) if mode == "exact" else oracle.neumann(A64, N, mask)
    Wr, Ur = oracle.wy(T64, f64(sub["K"]), f64(sub["V"]), f64(sub["beta"]), f64(sub["g"]), False)
    assert relF(f64(W[idx]), Wr) <= TOL, relF(f64(W[idx]), Wr)
    assert relF(f64(U[idx]), Ur) <= TOL, relF(f64(U[idx]), Ur)


# ------------------------------------------------------------------ full lower triangle

@pytest.mark.parametrize("C", [128, 256])
@pytest.mark.parametrize("variant", [("neumann", 2, False), ("neumann", 3, False), ("neumann", 4, False),
                                     ("neumann", 20, True), ("exact", 0, False)])
def test_dense_inverse_large_chunks(C, variant):
    mode, N, mask = variant
    nb = 5
    say(f"dense inverse C={C} {variant}")
    inp = synth.blocks(31, nb, C, 128, k_dtype="bf16")
    kw = dict(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C, compute="bf16",
              t_dtype=torch.float32)
    if mode == "exact":
        T = tri.gdn_tri_inverse_exact(**kw)
    else:
        T = tri.gdn_tri_inverse_neumann(N=N, mask=mask, **kw)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    Tr = oracle.doubling(A64) if mode == "exact" else oracle.neumann(A64, N, mask)
    T = f64(T)
    assert relF(T, Tr) <= TOL, relF(T, Tr)
    assert relF(eye_off(T), eye_off(Tr)) <= TOL, relF(eye_off(T), eye_off(Tr))
    i, j = np.indices((C, C))
    assert np.all(T[:, j > i] == 0) and np.all(T[:, i == j] == 1)
    if mask:
        assert np.all(T[:, i - j > N] == 0)


@pytest.mark.parametrize("C", [128, 256])
@pytest.mark.parametrize("source", ["neumann_unmasked", "exact", "given_f32", "given_bf16"])
@pytest.mark.parametrize("gate_k", [False, True])
def test_dense_wy_large_chunks(C, source, gate_k):
    nb = 3
    dk, dv = (128, 64) if C == 128 else (64, 128)
    say(f"dense wy C={C} {source} gate_k={gate_k}")
    inp = synth.blocks(32, nb, C, dk, k_dtype="bf16", d_v=dv)
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    args = (cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]))
    if source.startswith("given"):
        Tt = torch.from_numpy(oracle.neumann(A64, 3, False)).to(torch.float32 if source == "given_f32"
                                                                else torch.bfloat16)
        T64 = f64(Tt)
        W, U = tri.gdn_wy(*args, C=C, T=cuda(Tt), gate_k=gate_k, out_dtype=torch.float32)
    elif source == "exact":
        T64 = oracle.doubling(A64)
        W, U = tri.gdn_wy(*args, C=C, mode="exact", gate_k=gate_k, out_dtype=torch.float32)
    else:
        T64 = oracle.neumann(A64, 3, False)
        W, U = tri.gdn_wy(*args, C=C, mode="neumann", N=3, mask=False, gate_k=gate_k,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    Wr, Ur = oracle.wy(T64, f64(inp["K"]), f64(inp["V"]), f64(inp["beta"]), f64(inp["g"]), gate_k)
    assert relF(f64(W), Wr) <= TOL, relF(f64(W), Wr)
    assert relF(f64(U), Ur) <= TOL, relF(f64(U), Ur)


def test_dense_exact_cumulative_gates_many_blocks():
    """Cumulative gates, T in bf16, 37 blocks of 256 (more blocks than one wave of
    workgroups per XCD); sampled blocks against the oracle."""
    C, nb = 256, 37
    say("dense exact cumulative C=256")
    inp = synth.blocks(33, nb, C, 128, k_dtype="bf16")
    G = _cumulative(inp["g"], C).astype(np.float32)
    T = tri.gdn_tri_inverse_exact(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(torch.from_numpy(G)), C=C,
                                  compute="bf16", g_cumulative=True, t_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = [0, 17, 36]
    A64 = oracle.build_A(f64(inp["K"])[idx], f64(inp["beta"])[idx], G[idx], g_cumulative=True)
    assert relF(f64(T[idx]), oracle.doubling(A64)) <= TOL
