"""GPU parity of the INT8 power chain (gdn_tri_inverse_neumann with compute = int8)
against the oracle's int8 chain.

With a given fp32 A the result is exactly determined (power-of-two scales make every
scaling exact, products of codes are exact in int32, each intermediate sum is rounded
once to fp32), so the comparison is bit for bit.  With A built in-kernel from bf16 keys
the kernel's fp32 A differs from the oracle's fp64 A in its last bits, which can move a
code across a rounding boundary: there the comparison allows 5e-3 relative error on
T - I and requires 99 % of the entries to be identical."""
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
def test_int8_bit_exact_from_given_A(C, N, mask):
    if N >= C:
        pytest.skip("N < C")
    nb = 37
    say(f"int8 given A C={C} N={N} mask={mask}")
    A32 = _A32(20 + N, nb, C)
    T = tri.gdn_tri_inverse_neumann(A=cuda(torch.from_numpy(A32)), C=C, N=N, mask=mask,
                                    compute="int8")
    torch.cuda.synchronize()
    Tr = oracle.neumann_int8(A32.astype(np.float64), N, mask)
    np.testing.assert_array_equal(f64(T), Tr)


def test_int8_bf16_output_is_the_rounded_result():
    C, nb, N = 64, 29, 3
    say("int8 given A, T bf16")
    A32 = _A32(5, nb, C)
    T = tri.gdn_tri_inverse_neumann(A=cuda(torch.from_numpy(A32)), C=C, N=N, mask=True,
                                    compute="int8", t_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    Tr = torch.from_numpy(oracle.neumann_int8(A32.astype(np.float64), N, True).astype(np.float32))
    assert torch.equal(T.cpu(), Tr.to(torch.bfloat16))


@pytest.mark.parametrize("mask", [True, False])
def test_int8_closed_form_stress_input(mask):
    """A = -rho L with rho = 1/4 given exactly: the chain reproduces the closed-form
    truncated sum (every operand exactly representable), and the oracle agrees."""
    C, N = 64, 3
    say(f"int8 closed form mask={mask}")
    A = np.repeat((-0.25 * np.tril(np.ones((C, C)), -1))[None], 3, axis=0).astype(np.float32)
    T = tri.gdn_tri_inverse_neumann(A=cuda(torch.from_numpy(A)), C=C, N=N, mask=mask,
                                    compute="int8")
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(T), oracle.neumann_int8(A.astype(np.float64), N, mask))
    np.testing.assert_array_equal(f64(T), oracle.neumann(A.astype(np.float64), N, mask))


@pytest.mark.parametrize("nb", [45, 2048])
def test_int8_from_keys(nb):
    """A built in-kernel from bf16 keys (nb = 2048 is the B=1 H=16 seq 8192 workload the
    benchmark times); the oracle chain runs on the oracle's own A."""
    C, N = 64, 3
    say(f"int8 from keys nb={nb}")
    inp = synth.blocks(1, nb, C, 128, k_dtype="bf16")
    T = f64(tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]),
                                        C=C, N=N, mask=True, compute="int8"))
    torch.cuda.synchronize()
    sel = np.arange(nb) if nb <= 64 else np.random.default_rng(0).choice(nb, 64, replace=False)
    A = oracle.build_A(f64(inp["K"][sel]), f64(inp["beta"][sel]), f64(inp["g"][sel]))
    Tr = oracle.neumann_int8(A.astype(np.float32).astype(np.float64), N, True)
    I = np.eye(C)
    assert relF(T[sel] - I, Tr - I) <= 5e-3, relF(T[sel] - I, Tr - I)
    assert np.mean(T[sel] == Tr) >= 0.99
    assert np.all(np.diagonal(T, axis1=1, axis2=2) == 1.0) and np.all(np.triu(T, 1) == 0.0)
