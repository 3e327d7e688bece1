"""GPU parity of the parallel residual correction ([GEO] Methodologie SS3) against the
fp64 oracle running the same algorithm, and the accuracy it recovers against the exact
inverse.  All products are fp32 MFMA: tolerance 1e-5 relative Frobenius on T, 1e-4 on
T - I (whose norm is far smaller), as for the other fp32 inverses."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, eye_off, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")

TOL32 = 1e-5


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("N,mask,S", [(3, True, 8), (3, True, 0), (3, True, 1), (2, False, 4), (4, True, 2)])
def test_residual_parity(C, N, mask, S):
    nb = 37
    say(f"residual C={C} N={N} mask={mask} S={S}")
    inp = synth.blocks(41, nb, C, 128, k_dtype="bf16")
    T = tri.gdn_tri_inverse_residual(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C, N=N,
                                     mask=mask, S=S, compute="f32")
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    Tr = oracle.residual(A64, N, mask, S)
    T = f64(T)
    assert relF(T, Tr) <= TOL32, relF(T, Tr)
    assert relF(eye_off(T), eye_off(Tr)) <= 10 * TOL32, relF(eye_off(T), eye_off(Tr))


def test_residual_recovers_the_exact_inverse():
    """Masked N = 3 alone is off by ~1e-2 on T - I; with S = 8 the result is exact on
    subdiagonals below (S+1)(N+1) = 36, and at C = 64 the rest is below fp32 noise."""
    C, nb = 64, 64
    say("residual accuracy recovery")
    inp = synth.blocks(42, nb, C, 128, k_dtype="bf16")
    kw = dict(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C)
    Tm = f64(tri.gdn_tri_inverse_neumann(N=3, mask=True, compute="f32", **kw))
    Tc = f64(tri.gdn_tri_inverse_residual(N=3, mask=True, S=8, compute="f32", **kw))
    torch.cuda.synchronize()
    Tx = oracle.fs_inverse(oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"])))
    before = relF(eye_off(Tm), eye_off(Tx))
    after = relF(eye_off(Tc), eye_off(Tx))
    say(f"approximation error on T - I: masked N=3 {before:.2e}, with the correction {after:.2e}")
    assert before > 1e-3
    assert after <= 10 * TOL32


def test_residual_from_given_A_bf16_out():
    """A given in fp32 (the correctness workload's form), T written as bf16."""
    C, nb = 64, 16
    say("residual from A, bf16 out")
    inp = synth.blocks(0, nb, C, 128, k_dtype="f64")
    A32 = oracle.build_A(inp["K"], inp["beta"], inp["g"]).astype(np.float32)
    T = tri.gdn_tri_inverse_residual(A=cuda(torch.from_numpy(A32)), C=C, N=3, mask=True, S=8, compute="f32",
                                     t_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Tr = oracle.residual(A32.astype(np.float64), 3, True, 8)
    assert relF(f64(T), Tr) <= 2e-3   # the bf16 rounding of T itself


def test_residual_full_size_sampled_blocks():
    """2048 blocks of 64 from bf16 keys, N = 3 masked, S = 8, T fp32: the launch the
    benchmark times; 64 sampled blocks against the oracle."""
    nb, C = 2048, 64
    say("residual full size")
    inp = synth.blocks(1, nb, C, 128, k_dtype="bf16")
    T = tri.gdn_tri_inverse_residual(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C,
                                     N=3, mask=True, S=8, compute="f32")
    torch.cuda.synchronize()
    idx = np.random.default_rng(2).choice(nb, 64, replace=False)
    A = oracle.build_A(f64(inp["K"][idx]), f64(inp["beta"][idx]), f64(inp["g"][idx]))
    Tr = oracle.residual(A, 3, True, 8)
    Tg = f64(T)[idx]
    assert relF(Tg, Tr) <= TOL32, relF(Tg, Tr)
