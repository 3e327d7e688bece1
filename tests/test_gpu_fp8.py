"""GPU parity of the fp8 (OCP e4m3) power chain against the oracle's emulation of it.

[GEO] "Adaptation a la Quantification": the power chain runs on low-bit operands and the
structural mask keeps the intermediates in range.  The reading (e4m3 rounding, absmax/448
scales, Horner on X = H - I, counters) is stated in oracle/gdn_oracle.c and pinned in
tests/test_oracle.py.

Bars:
  - A = -rho L with rho in {7/32, 7/16, 7/8}: every scale is a power of two times an
    fp32 quotient the kernel and the oracle both round correctly, the codes of A and of
    X_1 are exact, and every sum of code products is an exact fp32 value, so the GPU
    result and its counters must equal the oracle's bit for bit (N <= 3).
  - Random A (c1-like, fp32): the MFMA's fp32 accumulation can differ from the exact sum
    in the last bit, and such a difference can move a later code by one e4m3 step.  T - I
    must match the emulation within 5e-3 (relative Frobenius), with at least 99 % of its
    entries identical; counters within 1 % (+2).
  - Both against the unquantised fp64 sum: 5e-2, the stated fp8 tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tri_inverse_amd as tri
from helpers import cuda, f64, relF, say

pytestmark = pytest.mark.gpu

RHOS = (7 / 32, 7 / 16, 7 / 8)


def _rho_L(nb, C, rho):
    return np.broadcast_to(-rho * np.tril(np.ones((C, C)), -1), (nb, C, C)).copy()


def _run(A64, N, mask, t_dtype=torch.float32):
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    A = torch.from_numpy(A64.astype(np.float32)).cuda()
    C = A64.shape[-1]
    T = tri.gdn_tri_inverse_neumann(A=A, C=C, N=N, mask=mask, compute="fp8", t_dtype=t_dtype, stats=stats)
    torch.cuda.synchronize()
    return f64(T), stats.cpu().numpy().astype(np.uint64)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("rho", RHOS)
@pytest.mark.parametrize("N", [1, 2, 3])
@pytest.mark.parametrize("mask", [True, False])
def test_fp8_bit_exact_on_rho_L(C, rho, N, mask):
    say(f"fp8 rho L C={C} rho={rho} N={N} mask={mask}")
    A = _rho_L(6, C, rho)
    Tg, st = _run(A, N, mask)
    Tr, cnt, _ = oracle.neumann_fp8(A, N, mask)
    np.testing.assert_array_equal(Tg, Tr)
    np.testing.assert_array_equal(st, cnt.sum(axis=0))


@pytest.mark.parametrize("mask", [True, False])
def test_fp8_rho_L_mask_removes_static_saturation(mask):
    """The pages' point on the stress input: unmasked, the powers outgrow A's range
    (static saturations); masked, nothing leaves it."""
    A = _rho_L(4, 64, 7 / 16)
    _, st = _run(A, 3, mask)
    if mask:
        assert st.tolist() == [0, 0, 0, 0]
    else:
        # X_2 alone saturates 1711 entries per block under A's scale (derived by hand in
        # tests/test_oracle.py); X_3 adds more
        assert st[2] > 4 * 1711 and st[0] == 0 and st[1] == 0


@pytest.mark.parametrize("N", [2, 3, 4])
@pytest.mark.parametrize("mask", [True, False])
def test_fp8_random_A_against_emulation(N, mask):
    say(f"fp8 random A N={N} mask={mask}")
    inp = synth.blocks(41, 128, 64, 128, k_dtype="f64")
    A = oracle.build_A(inp["K"], f64(inp["beta"]), f64(inp["g"])).astype(np.float32).astype(np.float64)
    Tg, st = _run(A, N, mask)
    Tr, cnt, _ = oracle.neumann_fp8(A, N, mask)
    eye = np.eye(64)
    assert np.all(np.triu(Tg, 1) == 0) and np.all(np.diagonal(Tg, axis1=1, axis2=2) == 1)
    assert relF(Tg - eye, Tr - eye) <= 5e-3, relF(Tg - eye, Tr - eye)
    low = np.tril(np.ones((64, 64), dtype=bool), -1)
    same = np.mean(Tg[:, low] == Tr[:, low])
    assert same >= 0.99, same
    ref = cnt.sum(axis=0).astype(np.int64)
    assert np.all(np.abs(st.astype(np.int64) - ref) <= 0.01 * ref + 2), (st, ref)
    assert relF(Tg, oracle.neumann(A, N, mask)) <= 5e-2


@pytest.mark.parametrize("mask", [True, False])
def test_fp8_from_keys_against_emulation(mask):
    """A built in the kernel from bf16 keys (fp32 Gram on the MFMA) against the emulation
    run on the oracle's A rounded to fp32: same bars as for a given random A."""
    say(f"fp8 keys mask={mask}")
    inp = synth.blocks(43, 128, 64, 128, k_dtype="bf16")
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    T = tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=64,
                                    N=3, mask=mask, compute="fp8", stats=stats)
    torch.cuda.synchronize()
    Tg, st = f64(T), stats.cpu().numpy().astype(np.int64)
    A = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    Tr, cnt, _ = oracle.neumann_fp8(A.astype(np.float32).astype(np.float64), 3, mask)
    eye = np.eye(64)
    assert relF(Tg - eye, Tr - eye) <= 5e-3, relF(Tg - eye, Tr - eye)
    ref = cnt.sum(axis=0).astype(np.int64)
    assert np.all(np.abs(st - ref) <= 0.01 * ref + 2), (st, ref)
    assert relF(Tg, oracle.neumann(A, 3, mask)) <= 5e-2


def test_fp8_bf16_output_is_the_rounded_fp32_output():
    A = _rho_L(4, 64, 7 / 16)
    T32, _ = _run(A, 3, False)
    T16, _ = _run(A, 3, False, t_dtype=torch.bfloat16)
    np.testing.assert_array_equal(T16, f64(torch.from_numpy(T32.astype(np.float32)).to(torch.bfloat16)))
