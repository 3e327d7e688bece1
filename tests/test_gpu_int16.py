"""GPU parity of the INT16 power chain (gdn_tri_inverse_neumann with compute = int16)
against the oracle's 16-bit chain.

With a given fp32 A the result is exactly determined: power-of-two scales make every
scaling exact, the four 8-bit digit products are exact in int32 and their recombination
exact in fp64, and each intermediate sum is formed in fp64 and rounded to fp32 in that
order on both sides.  So the comparison is bit for bit.  With A built in-kernel from bf16
keys the kernel's fp32 A differs from the oracle's fp64 A in its last bits; there the
bar is 1e-4 on T - I (16-bit codes: steps of 2^-15 of each operand's range)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")


def _A32(seed, nb, C):
    inp = synth.blocks(seed, nb, C, 128, k_dtype="f64")
    return oracle.build_A(inp["K"], inp["beta"].double().numpy(),
                          inp["g"].double().numpy()).astype(np.float32)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 7])
@pytest.mark.parametrize("mask", [True, False])
def test_int16_bit_exact_from_given_A(C, N, mask):
    if N >= C:
        pytest.skip("N < C")
    nb = 37
    say(f"int16 given A C={C} N={N} mask={mask}")
    A32 = _A32(60 + N, nb, C)
    T = tri.gdn_tri_inverse_neumann(A=cuda(torch.from_numpy(A32)), C=C, N=N, mask=mask, compute="int16")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(T), oracle.neumann_int16(A32.astype(np.float64), N, mask))


@pytest.mark.parametrize("rho", [0.25, 0.5])
@pytest.mark.parametrize("mask", [True, False])
def test_int16_closed_form_stress_input(rho, mask):
    """A = -rho L given exactly: the closed-form truncated sum at N = 4 (where the int8
    chain loses the band unmasked), bit for bit."""
    C, N = 64, 4
    say(f"int16 closed form rho={rho} mask={mask}")
    A = (-rho * np.tril(np.ones((C, C)), -1))[None].repeat(4, axis=0).astype(np.float32)
    T = tri.gdn_tri_inverse_neumann(A=cuda(torch.from_numpy(A)), C=C, N=N, mask=mask, compute="int16")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(T), oracle.neumann(A.astype(np.float64), N, mask))


@pytest.mark.parametrize("mask", [True, False])
def test_int16_from_bf16_keys(mask):
    C, nb, N = 64, 99, 3
    say(f"int16 from keys mask={mask}")
    inp = synth.blocks(61, nb, C, 128, k_dtype="bf16")
    T = tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C, N=N,
                                    mask=mask, compute="int16")
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    Tr = oracle.neumann_int16(A64.astype(np.float32).astype(np.float64), N, mask)
    eye = np.eye(C)
    assert relF(f64(T) - eye, Tr - eye) <= 1e-4, relF(f64(T) - eye, Tr - eye)
    assert relF(f64(T), oracle.neumann(A64, N, mask)) <= 1e-4
