"""GPU parity of the batched inverse kernels against the fp64 oracle (same algorithm,
same inputs).  Tolerances (relative Frobenius error over the whole output):
  fp32 MFMA compute: 1e-5; bf16 compute: 2e-3; fp8 e4m3 compute: 5e-2.
Structural exactness is checked bit for bit: the upper triangle of T is exactly 0 and
its diagonal exactly 1 (the products of lower-triangular operands add exact zeros).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, eye_off, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")

TOL = {"f32": 1e-5, "bf16": 2e-3, "fp8": 5e-2}


def _structure_exact(T):
    C = T.shape[-1]
    iu = np.triu_indices(C, 1)
    assert np.all(T[:, iu[0], iu[1]] == 0.0), "upper triangle not exactly zero"
    assert np.all(T[:, np.arange(C), np.arange(C)] == 1.0), "diagonal not exactly one"


def _oracle_T(A64, mode, N, mask):
    return oracle.doubling(A64) if mode == "exact" else oracle.neumann(A64, N, mask)


# The identity dominates relF over T (|I|_F = 8 at C = 64), so T - I and each of its
# first sub-diagonals are checked on their own.  Bar for bf16 operands: 2.2e-3, the
# error of T - I when every MFMA operand is rounded to bf16 (RNE) and accumulated
# exactly, on c1-like blocks (the rounding emulation of the scope table's error model).
TOL_TI = {"f32": 1e-5, "bf16": 2.2e-3, "bf16_out": 3.3e-3}


def _band_checks(Tg, Tr, compute, dmax):
    eye = np.eye(Tg.shape[-1])
    assert relF(Tg - eye, Tr - eye) <= TOL_TI[compute], relF(Tg - eye, Tr - eye)
    for d in range(1, dmax + 1):
        eg = np.diagonal(Tg, offset=-d, axis1=1, axis2=2)
        er = np.diagonal(Tr, offset=-d, axis1=1, axis2=2)
        assert relF(eg, er) <= TOL_TI[compute], (d, relF(eg, er))


def _fp32_A_workload(nb=256, C=64, seed=0):
    """fp32 A built in fp64 from unit keys, uniform beta and log-sigmoid gates, rounded."""
    inp = synth.blocks(seed, nb, C, 128, k_dtype="f64")
    A64 = oracle.build_A(inp["K"], f64(inp["beta"]), f64(inp["g"]))
    A32 = torch.from_numpy(A64.astype(np.float32))
    return A32, f64(A32)


@pytest.mark.parametrize("compute", ["f32", "bf16"])
@pytest.mark.parametrize("mode,N,mask", [("neumann", 3, True), ("neumann", 3, False),
                                         ("neumann", 2, True), ("neumann", 1, True),
                                         ("neumann", 63, True), ("exact", 0, False)])
def test_inverse_from_fp32_A(compute, mode, N, mask):
    say(f"inverse from fp32 A: 256 blocks C=64 mode={mode} N={N} mask={mask} compute={compute}")
    A32, A64 = _fp32_A_workload()
    dA = cuda(A32)
    if mode == "exact":
        T = tri.gdn_tri_inverse_exact(A=dA, C=64, compute=compute)
    else:
        T = tri.gdn_tri_inverse_neumann(A=dA, C=64, N=N, mask=mask, compute=compute)
    torch.cuda.synchronize()
    Tg = f64(T)
    Tr = _oracle_T(A64, mode, N, mask)
    _structure_exact(Tg)
    assert relF(Tg, Tr) <= TOL[compute], relF(Tg, Tr)
    assert relF(eye_off(Tg), eye_off(Tr)) <= 10 * TOL[compute]
    if mask and mode == "neumann":
        i, j = np.indices((64, 64))
        assert np.all(Tg[:, (i - j) > N] == 0.0)


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("variant", [("neumann", 2, True), ("neumann", 3, True),
                                     ("neumann", 4, True), ("neumann", 2, False),
                                     ("neumann", 3, False), ("neumann", 4, False),
                                     ("exact", 0, False)])
def test_inverse_from_bf16_K(C, variant):
    mode, N, mask = variant
    nb = 99  # ragged against the 4 blocks a workgroup takes
    say(f"inverse from bf16 K: nb={nb} C={C} {variant}")
    inp = synth.blocks(1, nb, C, 128, k_dtype="bf16")
    K, beta, g = cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"])
    if mode == "exact":
        T = tri.gdn_tri_inverse_exact(K=K, beta=beta, g=g, C=C, compute="bf16")
    else:
        T = tri.gdn_tri_inverse_neumann(K=K, beta=beta, g=g, C=C, N=N, mask=mask, compute="bf16")
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    Tr = _oracle_T(A64, mode, N, mask)
    Tg = f64(T)
    _structure_exact(Tg)
    assert relF(Tg, Tr) <= TOL["bf16"], relF(Tg, Tr)
    _band_checks(Tg, Tr, "bf16", min(N if mode == "neumann" else 3, C - 1))


@pytest.mark.parametrize("C", [16, 32, 64])
@pytest.mark.parametrize("N", [2, 3, 4])
@pytest.mark.parametrize("mask", [True, False])
@pytest.mark.parametrize("ab_beta", [(0.5, 0.5, 1.0), (1.0, 1.0, 0.5)])
def test_inverse_dyadic_correlated_keys_closed_form(C, N, mask, ab_beta):
    """Keys k_i = a e_0 + b e_{i+1} (exact in bf16), beta constant, no gate: A = -rho L
    with rho = beta a^2 (1/4 and 1/2), so every power's cross terms are O(1).  Closed
    forms ([GEO] Methodologie 1-2, pinned on the CPU): the truncated sum has
    sum_{n=1}^{N} (-rho)^n binom(d-1, n-1) on sub-diagonal d; the masked one is the exact
    inverse -rho (1 - rho)^(d-1) for d <= N and zero beyond.  Every operand the bf16
    products meet is then exactly representable (masked, and unmasked for N <= 3), so T
    must equal the closed form bit for bit; unmasked N = 4 rounds the third power's
    sum to bf16 and is held to the bf16 bar."""
    a, b, beta = ab_beta
    rho = beta * a * a
    say(f"dyadic keys C={C} N={N} mask={mask} rho={rho}")
    inp = synth.dyadic_keys(5, C, 128, a, b, beta)
    T = tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C,
                                    N=N, mask=mask, compute="bf16")
    torch.cuda.synchronize()
    d = np.subtract.outer(np.arange(C), np.arange(C))
    if mask:
        ref = np.where((d >= 1) & (d <= N), -rho * (1 - rho) ** np.maximum(d - 1, 0), 0.0)
    else:
        ref = sum((-rho) ** n * np.where(d >= 1, np.vectorize(math.comb)(np.maximum(d - 1, 0), n - 1), 0)
                  for n in range(1, N + 1))
    ref = np.eye(C) + ref
    Tg = f64(T)
    _structure_exact(Tg)
    if mask or N <= 3:
        np.testing.assert_array_equal(Tg, np.broadcast_to(ref, Tg.shape))
    else:
        _band_checks(Tg, np.broadcast_to(ref, Tg.shape), "bf16", N)


@pytest.mark.parametrize("k_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("C", [16, 64])
def test_build_A(k_dtype, C):
    say(f"build_A k_dtype={k_dtype} C={C}")
    inp = synth.blocks(2, 37, C, 64, k_dtype=k_dtype)
    A = tri.gdn_build_A(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), C=C)
    torch.cuda.synchronize()
    Ag = f64(A)
    Ar = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    iu = np.triu_indices(C)
    assert np.all(Ag[:, iu[0], iu[1]] == 0.0)
    assert relF(Ag, Ar) <= 1e-5, relF(Ag, Ar)


def test_build_A_cumulative_gate_and_special_cases():
    say("build_A cumulative gate / beta=0 / orthogonal keys")
    inp = synth.blocks(4, 8, 64, 128, k_dtype="f32")
    G = torch.cumsum(inp["g"].double(), dim=1).float()
    A1 = tri.gdn_build_A(cuda(inp["K"]), cuda(inp["beta"]), cuda(G), C=64, g_cumulative=True)
    Ar = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(G), g_cumulative=True)
    assert relF(f64(A1), Ar) <= 1e-5
    A0 = tri.gdn_build_A(cuda(inp["K"]), cuda(torch.zeros_like(inp["beta"])), cuda(inp["g"]), C=64)
    assert torch.all(A0 == 0)
    Ke = torch.zeros(2, 32, 64, dtype=torch.bfloat16)
    Ke[:, torch.arange(32), torch.arange(32)] = 1
    ones = torch.ones(2, 32)
    T = tri.gdn_tri_inverse_neumann(K=cuda(Ke), beta=cuda(ones), g=cuda(torch.zeros(2, 32)), C=32,
                                    N=3, mask=True)
    torch.cuda.synchronize()
    assert torch.equal(T.cpu(), torch.eye(32).expand(2, 32, 32))


def test_full_size_batched_inverse_all_blocks():
    """2048 blocks of 64x64 from bf16 K (B=1, H=16, seq 8192), the launch the bench times."""
    nb = 2048
    inp = synth.blocks(1, nb, 64, 128, k_dtype="bf16")
    K, beta, g = cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"])
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    for mode, N, mask, t_dtype in [("neumann", 3, True, torch.float32),
                                   ("neumann", 2, True, torch.float32),
                                   ("neumann", 4, True, torch.float32),
                                   ("neumann", 2, False, torch.float32),
                                   ("neumann", 3, False, torch.float32),
                                   ("neumann", 4, False, torch.float32),
                                   ("neumann", 3, True, torch.bfloat16),
                                   ("exact", 0, False, torch.float32),
                                   ("exact", 0, False, torch.bfloat16)]:
        say(f"full-size inverse {mode} N={N} mask={mask} {t_dtype}")
        if mode == "exact":
            T = tri.gdn_tri_inverse_exact(K=K, beta=beta, g=g, C=64, t_dtype=t_dtype)
        else:
            T = tri.gdn_tri_inverse_neumann(K=K, beta=beta, g=g, C=64, N=N, mask=mask, t_dtype=t_dtype)
        torch.cuda.synchronize()
        Tr = _oracle_T(A64, mode, N, mask)
        Tg = f64(T)
        _structure_exact(Tg)
        assert relF(Tg, Tr) <= TOL["bf16"]
        # T stored as bf16 adds its own rounding (at most 2^-9 relative, RMS about
        # 1.1e-3): the bar for T - I grows by that much
        _band_checks(Tg, Tr, "bf16" if t_dtype == torch.float32 else "bf16_out",
                     N if mode == "neumann" else 3)


def test_fp8_inverse_and_counters():
    say("fp8 inverse, random blocks and correlated-key stress")
    inp = synth.blocks(5, 64, 64, 128, k_dtype="bf16")
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    for mask in (True, False):
        T = tri.gdn_tri_inverse_neumann(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]),
                                        C=64, N=3, mask=mask, compute="fp8", stats=stats)
        torch.cuda.synchronize()
        Tg = f64(T)
        _structure_exact(Tg)
        assert relF(Tg, oracle.neumann(A64, 3, mask)) <= TOL["fp8"]
        s = stats.cpu().tolist()
        assert s[0] == 0 and s[1] == 0
    # stress: A = -rho L; unmasked powers outgrow A's range, masked ones do not
    st = synth.correlated_keys(16, 64, 128, 0.5)
    counts = {}
    for mask in (True, False):
        T = tri.gdn_tri_inverse_neumann(K=cuda(st["K"]), beta=cuda(st["beta"]), g=cuda(st["g"]), C=64,
                                        N=3, mask=mask, compute="fp8", stats=stats)
        torch.cuda.synchronize()
        counts[mask] = stats.cpu().tolist()
        A64 = oracle.build_A(f64(st["K"]), f64(st["beta"]), f64(st["g"]))
        assert relF(f64(T), oracle.neumann(A64, 3, mask)) <= TOL["fp8"]
    assert counts[True][0] == 0 and counts[False][0] == 0
    assert counts[True][1] == 0 and counts[False][1] == 0
    assert counts[False][2] > counts[True][2]


@pytest.mark.parametrize("N", [1, 2, 3, 4])
@pytest.mark.parametrize("strong", [False, True])
def test_bf16_output_is_the_rounded_fp32_output(N, strong):
    """Masked sum from bf16 keys: T in bf16 (for N = 2, 3 formed in two halves of rows,
    the first stored while the second half's keys still arrive) must be exactly the bf16
    rounding of T in fp32 (formed in one piece), with ordinary gates and with gates that
    force the exponential-of-difference form; 3000 blocks, so the grid ends in a part-filled
    workgroup."""
    say(f"bf16 vs fp32 output N={N} strong={strong}")
    inp = synth.blocks(8, 3000, 64, 128, k_dtype="bf16")
    g = inp["g"] * 4.0 - 1.0 if strong else inp["g"]
    K, beta, gg = cuda(inp["K"]), cuda(inp["beta"]), cuda(g)
    T32 = tri.gdn_tri_inverse_neumann(K=K, beta=beta, g=gg, C=64, N=N, mask=True, t_dtype=torch.float32)
    T16 = tri.gdn_tri_inverse_neumann(K=K, beta=beta, g=gg, C=64, N=N, mask=True, t_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(T16, T32.to(torch.bfloat16))


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("strong", [False, True])
def test_exact_bf16_output_is_the_rounded_fp32_output(dk, strong):
    """Exact doubling from bf16 keys: T in bf16 (formed in two halves of rows, the first
    stored while the second half's keys still arrive, the second reading the first
    half's rows of every square) must be exactly the bf16 rounding of T in fp32 (formed
    in one piece); ordinary gates and gates that force the exponential-of-difference
    form; 3000 blocks, so the grid ends in a part-filled workgroup."""
    say(f"exact bf16 vs fp32 output dk={dk} strong={strong}")
    inp = synth.blocks(9, 3000, 64, dk, k_dtype="bf16")
    g = inp["g"] * 4.0 - 1.0 if strong else inp["g"]
    K, beta, gg = cuda(inp["K"]), cuda(inp["beta"]), cuda(g)
    T32 = tri.gdn_tri_inverse_exact(K=K, beta=beta, g=gg, C=64, t_dtype=torch.float32)
    T16 = tri.gdn_tri_inverse_exact(K=K, beta=beta, g=gg, C=64, t_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(T16, T32.to(torch.bfloat16))


def test_empty_batch_is_a_noop():
    K = torch.zeros(0, 64, 128, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(0, 64, device="cuda")
    T = tri.gdn_tri_inverse_neumann(K=K, beta=b, g=b, C=64)
    assert T.shape == (0, 64, 64)


@pytest.mark.parametrize("mode", ["neumann", "exact"])
def test_strong_gates_take_the_elementwise_exp_path(mode):
    """Gates summing below -80 inside a chunk (exp(-G) would overflow fp32): the kernel
    must switch to exp(G_i - G_j) per element and still match the oracle."""
    say(f"strong gates mode={mode}")
    inp = synth.blocks(6, 40, 64, 128, k_dtype="bf16")
    g = inp["g"] * 4.0 - 1.0            # mean about -4 per token: G reaches about -250
    assert float(torch.cumsum(g.double(), 1).min()) < -100
    K, beta = cuda(inp["K"]), cuda(inp["beta"])
    if mode == "exact":
        T = tri.gdn_tri_inverse_exact(K=K, beta=beta, g=cuda(g), C=64)
    else:
        T = tri.gdn_tri_inverse_neumann(K=K, beta=beta, g=cuda(g), C=64, N=3, mask=False)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(g))
    Tr = _oracle_T(A64, mode, 3, False)
    Tg = f64(T)
    assert np.all(np.isfinite(Tg))
    _structure_exact(Tg)
    assert relF(Tg, Tr) <= TOL["bf16"]
