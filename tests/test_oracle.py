"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check is a hand-derived fixture
(tests/golden), a closed form, an algebraic identity, an independent library
routine, or a second independent algorithm (e.g. the token recurrence against the
chunk form).  Pages cited by title:
  [GEO]  When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
         Approximation for Quantized Gated DeltaNet
  [PSDA] A Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
         Decode on FPGA
"""
import math

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth
from conftest import load_golden


def _rand_A(seed, nb, C, dk=128):
    inp = synth.blocks(seed, nb, C, dk, k_dtype="f64")
    return oracle.build_A(inp["K"], inp["beta"].double().numpy(), inp["g"].double().numpy())


def _relF(x, ref):
    return float(np.linalg.norm(x - ref) / np.linalg.norm(ref))


# ---------------------------------------------------------------- golden fixtures

def test_golden_tri4_integer():
    """Hand-derived 4x4 integer example ([GEO] problem statement, Methodologie 1-2)."""
    gold = load_golden("tri4_integer.txt")
    A = gold["A"][None]
    np.testing.assert_array_equal(oracle.fs_inverse(A)[0], gold["T_exact"])
    np.testing.assert_array_equal(oracle.doubling(A)[0], gold["T_exact"])
    for N in (1, 2, 3):
        key = "neumann_N%d_unmasked" % N
        np.testing.assert_array_equal(oracle.neumann(A, N, False)[0], gold[key])
    for N in (1, 2):
        np.testing.assert_array_equal(oracle.neumann(A, N, True)[0], gold["neumann_N%d_masked" % N])
    # the residual correction of the N=1 masked sum reaches the exact inverse
    np.testing.assert_array_equal(oracle.residual(A, 1, True, 2)[0], gold["T_exact"])


def test_golden_build_A_3tok():
    gold = load_golden("build_A_3tok.txt")
    A = oracle.build_A(gold["K"][None], gold["beta"], gold["gamma"])[0]
    np.testing.assert_allclose(A, gold["A"], rtol=0, atol=1e-15)
    # same block given its cumulative gate directly
    G = np.cumsum(gold["gamma"][0])[None]
    A2 = oracle.build_A(gold["K"][None], gold["beta"], G, g_cumulative=True)[0]
    np.testing.assert_allclose(A2, gold["A"], rtol=0, atol=1e-15)


def test_golden_recurrence_2tok():
    gold = load_golden("recurrence_2tok.txt")
    shp = lambda x: x[None, None]
    O, S = oracle.recurrence(shp(gold["Q"]), shp(gold["K"]), shp(gold["V"]),
                             gold["beta"][None], gold["gamma"][None], 1.0)
    np.testing.assert_allclose(O[0, 0], gold["O"], atol=1e-15)
    np.testing.assert_allclose(S[0, 0], gold["S"], atol=1e-15)
    # the chunk form with one 2-token chunk reaches the same numbers
    for mode in (oracle.INV_NEUMANN, oracle.INV_EXACT, oracle.INV_FS):
        O2, S2 = oracle.chunk_fwd(shp(gold["Q"]), shp(gold["K"]), shp(gold["V"]),
                                  gold["beta"][None], gold["gamma"][None], C=2, scale=1.0,
                                  inv_mode=mode, N=1, mask=False)
        np.testing.assert_allclose(O2[0, 0], gold["O"], atol=1e-15)
        np.testing.assert_allclose(S2[0, 0], gold["S"], atol=1e-15)


# ---------------------------------------------------------------- A and Lemma 3.1

def test_build_A_structure_and_special_cases():
    inp = synth.blocks(3, 8, 64, 128, k_dtype="f64")
    K, beta, g = inp["K"], inp["beta"].double().numpy(), inp["g"].double().numpy()
    A = oracle.build_A(K, beta, g)
    iu = np.triu_indices(64)
    assert np.all(A[:, iu[0], iu[1]] == 0.0)            # strictly lower, exactly
    # beta == 0 -> A == 0
    assert np.all(oracle.build_A(K, np.zeros_like(beta), g) == 0.0)
    # orthonormal keys -> A == 0 -> T == I
    Ke = np.zeros((2, 16, 32))
    Ke[:, np.arange(16), np.arange(16)] = 1.0
    A0 = oracle.build_A(Ke, np.ones((2, 16)), np.zeros((2, 16)))
    assert np.all(A0 == 0.0)
    np.testing.assert_array_equal(oracle.neumann(A0, 3, True), np.broadcast_to(np.eye(16), (2, 16, 16)))
    # A / (-beta_i e^{G_i - G_j}) is the Gram matrix of the keys (library matmul)
    G = np.cumsum(g, axis=1)
    gram = np.einsum("bid,bjd->bij", K, K)
    scale = -beta[:, :, None] * np.exp(G[:, :, None] - G[:, None, :])
    np.testing.assert_allclose(A, np.tril(gram * scale, -1), rtol=1e-13, atol=1e-15)


def test_build_A_gate_restarts_each_block_sign_convention():
    """identical unit keys, beta = 1, gamma = 0 -> A = -L (L strictly lower ones)."""
    K = np.zeros((1, 8, 4))
    K[..., 0] = 1.0
    A = oracle.build_A(K, np.ones((1, 8)), np.zeros((1, 8)))
    np.testing.assert_array_equal(A[0], -np.tril(np.ones((8, 8)), -1))


def test_lemma_3_1_structural_zeros():
    """[GEO] Methodologie 1, Lemma 3.1: A^n vanishes above its n-th subdiagonal."""
    A = _rand_A(5, 4, 64)[0]
    P = np.eye(64)
    for n in range(1, 8):
        P = P @ A
        i, j = np.indices((64, 64))
        assert np.all(P[(i - j) < n] == 0.0), n
    P = np.linalg.matrix_power(A, 64)
    assert np.all(P == 0.0)


# ---------------------------------------------------------------- inverses

@pytest.mark.parametrize("C", [2, 16, 64])
def test_fs_inverse_is_the_inverse(C):
    A = _rand_A(7, 16, C)
    T = oracle.fs_inverse(A)
    I = np.eye(C)
    for b in range(A.shape[0]):
        res = np.linalg.norm((I - A[b]) @ T[b] - I)
        assert res < 1e-12
        ref = scipy.linalg.solve_triangular(I - A[b], I, lower=True, unit_diagonal=True)
        np.testing.assert_allclose(T[b], ref, rtol=1e-12, atol=1e-14)
    iu = np.triu_indices(C, 1)
    assert np.all(T[:, iu[0], iu[1]] == 0.0)
    assert np.all(T[:, np.arange(C), np.arange(C)] == 1.0)


def test_C2_closed_form():
    A = np.zeros((3, 2, 2))
    A[:, 1, 0] = [0.25, -3.0, 7.5]
    for T in (oracle.fs_inverse(A), oracle.doubling(A), oracle.neumann(A, 1, True),
              oracle.neumann(A, 1, False)):
        np.testing.assert_array_equal(T[:, 0], [[1, 0]] * 3)
        np.testing.assert_array_equal(T[:, 1, 0], A[:, 1, 0])
        np.testing.assert_array_equal(T[:, 1, 1], [1, 1, 1])


@pytest.mark.parametrize("C", [16, 64])
def test_full_neumann_and_doubling_are_exact(C):
    """Nilpotency: sum_{n<=C-1} A^n and prod (I + A^(2^i)) both equal (I - A)^-1."""
    A = _rand_A(11, 12, C)
    Tfs = oracle.fs_inverse(A)
    assert _relF(oracle.neumann(A, C - 1, False), Tfs) < 1e-13
    assert _relF(oracle.neumann(A, C - 1, True), Tfs) < 1e-13
    Td = oracle.doubling(A)
    assert _relF(Td, Tfs) < 1e-13
    I = np.eye(C)
    for b in range(A.shape[0]):
        assert np.linalg.norm((I - A[b]) @ Td[b] - I) < 1e-12


@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_truncated_telescoping(N):
    """(I - A) sum_{n<=N} A^n = I - A^(N+1) (unmasked)."""
    A = _rand_A(13, 6, 64)
    T = oracle.neumann(A, N, False)
    I = np.eye(64)
    for b in range(A.shape[0]):
        lhs = (I - A[b]) @ T[b]
        rhs = I - np.linalg.matrix_power(A[b], N + 1)
        assert np.max(np.abs(lhs - rhs)) < 1e-14


@pytest.mark.parametrize("N", [1, 2, 3, 4])
def test_masked_equals_band_of_exact(N):
    """[GEO] Methodologie 2: M^(N) .* T(0) keeps subdiagonals 0..N, which are exact."""
    A = _rand_A(17, 6, 64)
    Tm = oracle.neumann(A, N, True)
    Tfs = oracle.fs_inverse(A)
    i, j = np.indices((64, 64))
    band = (i - j <= N)
    np.testing.assert_allclose(Tm, np.where(band, Tfs, 0.0), rtol=0, atol=1e-14)
    # masking A and every Horner intermediate instead gives the same result
    for b in range(A.shape[0]):
        Ab = np.where(band, A[b], 0.0)
        H = np.eye(64)
        for _ in range(N):
            H = np.where(band, np.eye(64) + Ab @ H, 0.0)
        np.testing.assert_allclose(H, Tm[b], rtol=0, atol=1e-15)


@pytest.mark.parametrize("N", [1, 2, 3])
def test_band_recurrence_from_subdiagonals(N):
    """The band of the masked sum for N <= 3 from A's first three sub-diagonals alone
    (every chain from i down to j has at most i - j steps), the form the chunk forward
    evaluates element by element:
    t1 = a1(i), t2 = a2(i) + a1(i) a1(i-1),
    t3 = a3(i) + a1(i) a2(i-1) + a2(i) a1(i-2) + a1(i) a1(i-1) a1(i-2)."""
    A = _rand_A(23, 5, 64)
    Tm = oracle.neumann(A, N, True)
    for b in range(A.shape[0]):
        a = {d: np.array([A[b, i, i - d] if i >= d and d <= N else 0.0 for i in range(64)])
             for d in (1, 2, 3)}
        sh = lambda x, k: np.concatenate([np.zeros(k), x[:-k]])  # x(i - k), 0 before row 0
        t = {1: a[1],
             2: a[2] + a[1] * sh(a[1], 1),
             3: a[3] + a[1] * sh(a[2], 1) + a[2] * sh(a[1], 2) + a[1] * sh(a[1], 1) * sh(a[1], 2)}
        T = np.eye(64)
        for d in range(1, N + 1):
            for i in range(d, 64):
                T[i, i - d] = t[d][i]
        np.testing.assert_allclose(T, Tm[b], rtol=0, atol=1e-14)


@pytest.mark.parametrize("rho", [0.25, 0.5])
def test_correlated_keys_closed_form(rho):
    """keys with k_i.k_j = rho, beta = 1, g = 0 give A = -rho L.  Then
    T_ij = -rho (1 - rho)^(i-j-1) (i > j) and the truncated sum has entries
    sum_{n=1}^{N} (-rho)^n binom(i-j-1, n-1)."""
    C = 64
    inp = synth.correlated_keys(1, C, 128, rho)
    A = oracle.build_A(inp["K64"], inp["beta"].double().numpy(), inp["g"].double().numpy())
    np.testing.assert_allclose(A[0], -rho * np.tril(np.ones((C, C)), -1), rtol=1e-14, atol=1e-15)
    i, j = np.indices((C, C))
    m = i - j
    T_exact = np.where(m > 0, -rho * (1 - rho) ** np.maximum(m - 1, 0), 0.0) + np.eye(C)
    np.testing.assert_allclose(oracle.fs_inverse(A)[0], T_exact, rtol=1e-12, atol=1e-14)
    for N in (2, 3, 4):
        closed = np.eye(C)
        for n in range(1, N + 1):
            coef = np.vectorize(lambda mm: math.comb(mm - 1, n - 1) if mm >= 1 else 0)(m)
            closed = closed + ((-rho) ** n) * coef
        np.testing.assert_allclose(oracle.neumann(A, N, False)[0], closed, rtol=1e-12, atol=1e-12)
    if rho == 0.5:
        # dynamic-range blow-up of higher truncation orders ([GEO] Adaptation a la Quantification)
        assert abs(np.max(np.abs(oracle.neumann(A, 3, False))) - 221.375) < 1e-9
        assert abs(np.max(np.abs(oracle.neumann(A, 4, False))) - 2142.375) < 1e-9
        assert np.max(np.abs(oracle.neumann(A, 3, True))) == 1.0


def test_residual_correction_support():
    """[GEO] Methodologie 3: T(0) sum_{s<=S} E^s is exact below subdiagonal (S+1)(N+1)."""
    A = _rand_A(19, 4, 64)
    Tfs = oracle.fs_inverse(A)
    i, j = np.indices((64, 64))
    for N, S in ((3, 8), (2, 3), (1, 5)):
        lim = (S + 1) * (N + 1)
        for mask in (True, False):
            T = oracle.residual(A, N, mask, S)
            sel = (i - j) < lim
            np.testing.assert_allclose(T[:, sel], Tfs[:, sel], rtol=0, atol=1e-13)
    # E is supported on subdiagonals >= N+1
    N = 3
    T0 = oracle.neumann(A, N, True)
    E = np.eye(64) - (np.eye(64) - A[0]) @ T0[0]
    assert np.max(np.abs(E[(i - j) <= N])) < 1e-15
    # S = 0 leaves T(0) unchanged
    np.testing.assert_array_equal(oracle.residual(A, 3, True, 0), T0)


# ---------------------------------------------------------------- WY

@pytest.mark.parametrize("gate_k", [False, True])
def test_wy_solves_the_triangular_system(gate_k):
    """With the exact T, (I - A) W = diag(s) K and (I - A) U = diag(beta) V."""
    nb, C, dk, dv = 5, 32, 24, 40
    inp = synth.blocks(23, nb, C, dk, k_dtype="f64", d_v=dv)
    K = inp["K"]
    V = inp["V"].double().numpy()
    beta = inp["beta"].double().numpy()
    g = inp["g"].double().numpy()
    A = oracle.build_A(K, beta, g)
    T = oracle.fs_inverse(A)
    W, U = oracle.wy(T, K, V, beta, g, gate_k)
    G = np.cumsum(g, axis=1)
    s = beta * (np.exp(G) if gate_k else 1.0)
    I = np.eye(C)
    for b in range(nb):
        np.testing.assert_allclose((I - A[b]) @ W[b], s[b][:, None] * K[b], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose((I - A[b]) @ U[b], beta[b][:, None] * V[b], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- chunk form vs recurrence

def _small_prefill(seed, B=2, H=2, T=48, dk=8, dv=6, family="sigmoid"):
    inp = synth.prefill(seed, B, H, T, dk, dv, family=family)
    return {k: v.double().numpy() for k, v in inp.items()}


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16])
def test_chunk_form_equals_token_recurrence(C):
    x = _small_prefill(29)
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((2, 2, 8, 6))
    scale = 8 ** -0.5
    O_r, S_r = oracle.recurrence(x["Q"], x["K"], x["V"], x["beta"], x["g"], scale, S0=S0)
    modes = [(oracle.INV_FS, 3, True), (oracle.INV_EXACT, 3, True),
             (oracle.INV_NEUMANN, max(C - 1, 0), False)]
    for mode, N, mask in modes:
        O_c, S_c = oracle.chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], C, scale,
                                    inv_mode=mode, N=N, mask=mask, S0=S0)
        assert np.max(np.abs(O_c - O_r)) < 1e-13, (C, mode)
        assert np.max(np.abs(S_c - S_r)) < 1e-13, (C, mode)


def test_chunk_form_wrong_gate_on_W_is_detected():
    """Guard: the ungated correction W = T diag(beta) K does NOT reproduce the
    recurrence when the gate is non-trivial, so the pins above would catch it."""
    x = _small_prefill(31, T=32)
    O_r, _ = oracle.recurrence(x["Q"], x["K"], x["V"], x["beta"], x["g"], 1.0)
    O_c, _ = oracle.chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], 8, 1.0,
                              inv_mode=oracle.INV_EXACT)
    assert np.max(np.abs(O_c - O_r)) < 1e-13
    # emulate the ungated variant for one chunk with numpy and check it differs
    Q, K, V, beta, g = (x[k][0, 0, :8] for k in ("Q", "K", "V", "beta", "g"))
    Kb = K[None]
    A = oracle.build_A(Kb, beta[None], g[None])[0]
    T = oracle.fs_inverse(A[None])[0]
    G = np.cumsum(g)
    W_gated, _ = oracle.wy(T[None], Kb, V[None], beta[None], g[None], True)
    W_plain, _ = oracle.wy(T[None], Kb, V[None], beta[None], g[None], False)
    assert np.max(np.abs(W_gated - W_plain)) > 1e-3
    assert np.all(G < 0)


def test_chunk_size_invariance_and_split_sequence():
    x = _small_prefill(37, T=64, dk=16, dv=8, family="uniform")
    scale = 0.25
    ref_O, ref_S = oracle.chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], 64, scale,
                                    inv_mode=oracle.INV_FS)
    for C in (8, 16, 32):
        O, S = oracle.chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], C, scale,
                                inv_mode=oracle.INV_EXACT)
        assert np.max(np.abs(O - ref_O)) < 1e-12
        assert np.max(np.abs(S - ref_S)) < 1e-12
    # process [0, 32) then [32, 64) with the state carried
    h = lambda a: a[:, :, :32]
    t = lambda a: a[:, :, 32:]
    O1, S1 = oracle.chunk_fwd(h(x["Q"]), h(x["K"]), h(x["V"]), h(x["beta"]), h(x["g"]), 16, scale,
                              inv_mode=oracle.INV_EXACT)
    O2, S2 = oracle.chunk_fwd(t(x["Q"]), t(x["K"]), t(x["V"]), t(x["beta"]), t(x["g"]), 16, scale,
                              inv_mode=oracle.INV_EXACT, S0=S1)
    assert np.max(np.abs(np.concatenate([O1, O2], axis=2) - ref_O)) < 1e-12
    assert np.max(np.abs(S2 - ref_S)) < 1e-12


def test_recurrence_special_cases():
    x = _small_prefill(41, B=1, H=2, T=24, dk=8, dv=5)
    rng = np.random.default_rng(2)
    S0 = rng.standard_normal((1, 2, 8, 5))
    # beta == 0: the state only decays; O = scale e^{G_t} q_t^T S0 with G the global cumsum
    zb = np.zeros_like(x["beta"])
    O, S = oracle.recurrence(x["Q"], x["K"], x["V"], zb, x["g"], 0.5, S0=S0)
    Gt = np.cumsum(x["g"], axis=2)
    O_ref = 0.5 * np.exp(Gt)[..., None] * np.einsum("bhtd,bhde->bhte", x["Q"], S0)
    np.testing.assert_allclose(O, O_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S, np.exp(Gt[:, :, -1])[..., None, None] * S0, rtol=1e-12)
    # delta-rule retrieval: beta = 1, no decay, unit key -> S_t^T k_t = v_t after the step
    ones = np.ones_like(x["beta"][:, :, :1])
    k1 = x["K"][:, :, :1] / np.linalg.norm(x["K"][:, :, :1], axis=-1, keepdims=True)
    O1, S1 = oracle.recurrence(k1, k1, x["V"][:, :, :1], ones, np.zeros_like(ones), 1.0, S0=S0)
    np.testing.assert_allclose(O1[:, :, 0], x["V"][:, :, 0], rtol=1e-12, atol=1e-13)
    # O is linear in V when S0 = 0
    Oa, _ = oracle.recurrence(x["Q"], x["K"], x["V"], x["beta"], x["g"], 1.0)
    Ob, _ = oracle.recurrence(x["Q"], x["K"], 3.0 * x["V"], x["beta"], x["g"], 1.0)
    np.testing.assert_allclose(Ob, 3.0 * Oa, rtol=1e-12, atol=1e-14)


def test_threads_do_not_change_results():
    A = _rand_A(43, 32, 64)
    oracle.set_threads(1)
    T1 = oracle.neumann(A, 3, True)
    oracle.set_threads(4)
    T4 = oracle.neumann(A, 3, True)
    np.testing.assert_array_equal(T1, T4)


# ---------------------------------------------------------------- INT8 power chain

def _closed_form_truncated(C, rho, N, mask):
    """I + sum_{n=1}^{N} (-rho)^n binom(i-j-1, n-1) for A = -rho L (L strictly lower ones)."""
    i, j = np.indices((C, C))
    m = i - j
    T = np.eye(C)
    for n in range(1, N + 1):
        coef = np.vectorize(lambda mm: math.comb(mm - 1, n - 1) if mm >= 1 else 0)(m)
        T = T + ((-rho) ** n) * coef
    if mask:
        T = np.where(m > N, 0.0, T)
    return T


@pytest.mark.parametrize("rho", [0.125, 0.25])
@pytest.mark.parametrize("N", [1, 2, 3])
@pytest.mark.parametrize("mask", [False, True])
def test_int8_chain_exact_on_closed_form(rho, N, mask):
    """A = -rho L with rho a power of two: every operand of the chain (A and the N <= 3
    intermediates) is an exact multiple of its power-of-two scale with codes <= 127, and
    every integer sum fits fp32, so the int8 chain must reproduce the closed-form
    truncated sum exactly (a dropped term, a wrong sign, scale or index breaks this)."""
    C = 64
    A = (-rho * np.tril(np.ones((C, C)), -1))[None]
    T = oracle.neumann_int8(A, N, mask)[0]
    np.testing.assert_array_equal(T, _closed_form_truncated(C, rho, N, mask))


@pytest.mark.parametrize("mask", [False, True])
def test_int8_chain_exact_on_dyadic_inputs_N2(mask):
    """A with entries code * 2^-9 (|code| <= 127, one code of 127): the codes of A and
    of X_1 = A are exact, the product of codes is exact and the single fp32 rounding is
    exact (sums below 2^24), so N = 2 equals the fp64 Horner sum I + A + A^2."""
    rng = np.random.default_rng(11)
    C, nb = 64, 6
    codes = np.tril(rng.integers(-127, 128, size=(nb, C, C)), -1)
    codes[:, 5, 1] = 127
    A = codes * 2.0 ** -9
    np.testing.assert_array_equal(oracle.neumann_int8(A, 2, mask), oracle.neumann(A, 2, mask))


def test_int8_quantiser_properties():
    """N = 1 returns I + A' with A' the dequantised A: A' is a multiple of one power of
    two 2^e per block with codes in [-127, 127], |A' - A| <= 2^(e-1) (round to nearest),
    and the scale is the finest one that does not saturate (127 * 2^(e-1) < max|A|)."""
    A = _rand_A(12, 16, 64).astype(np.float32).astype(np.float64)
    Ad = oracle.neumann_int8(A, 1, False) - np.eye(64)
    for b in range(A.shape[0]):
        amax = np.max(np.abs(A[b]))
        e = math.frexp(amax / 127.0)[1]  # 2^(e-1) <= amax/127 < 2^e, or amax/127 = 2^(e-1)
        if amax <= 127.0 * 2.0 ** (e - 1):
            e -= 1
        q = Ad[b] * 2.0 ** -e
        np.testing.assert_array_equal(q, np.round(q))
        assert np.max(np.abs(q)) <= 127
        assert np.max(np.abs(Ad[b] - A[b])) <= 2.0 ** (e - 1)
        assert 127.0 * 2.0 ** (e - 1) < amax <= 127.0 * 2.0 ** e


def test_int8_mask_keeps_the_band_accurate():
    """[GEO] Adaptation a la Quantification: without the mask, the large out-of-band
    entries of the powers set coarse int8 scales and the entries that matter (the band)
    lose their precision; with the mask they keep it.  Stress input A = -0.5 L with
    N = 4, where the unmasked third power reaches 221 (an int8 step of 2)."""
    C, N = 64, 4
    A = (-0.5 * np.tril(np.ones((C, C)), -1))[None]
    i, j = np.indices((C, C))
    band = (i - j >= 0) & (i - j <= N)
    ref = oracle.neumann(A, N, True)[0]
    err_masked = np.max(np.abs(oracle.neumann_int8(A, N, True)[0] - ref)[band])
    err_unmasked = np.max(np.abs(oracle.neumann_int8(A, N, False)[0] - ref)[band])
    assert err_masked == 0.0
    assert err_unmasked > 0.05


def test_int8_chain_close_to_fp64_on_c1_inputs():
    """On c1-like blocks the masked int8 chain stays within a few quantisation steps of
    the fp64 masked sum (relative error of T - I below 2e-2)."""
    A = _rand_A(13, 24, 64).astype(np.float32).astype(np.float64)
    T8 = oracle.neumann_int8(A, 3, True)
    Tf = oracle.neumann(A, 3, True)
    I = np.eye(64)
    assert _relF(T8 - I, Tf - I) < 2e-2
    assert np.all(np.diagonal(T8, axis1=1, axis2=2) == 1.0)
    assert np.all(np.triu(T8, 1) == 0.0)


# ---------------------------------------------------------------- int16 chain
# The same Horner chain on 16-bit codes (|code| <= 32639 = 127 * 257, each sum formed in
# fp64 then rounded to fp32); reading in oracle/gdn_oracle.c.

@pytest.mark.parametrize("rho", [0.125, 0.25, 0.5])
@pytest.mark.parametrize("N", [1, 2, 3, 4])
@pytest.mark.parametrize("mask", [False, True])
def test_int16_chain_exact_on_closed_form(rho, N, mask):
    """A = -rho L, rho a power of two: every operand through N = 4 is a multiple of its
    power-of-two scale with codes <= 32639 (the unmasked third power reaches 221.375 at
    rho = 1/2, still 3 fractional bits below a 2^-7 step), so the 16-bit chain
    reproduces the closed-form truncated sum exactly, where the int8 chain does not."""
    C = 64
    A = (-rho * np.tril(np.ones((C, C)), -1))[None]
    np.testing.assert_array_equal(oracle.neumann_int16(A, N, mask)[0], _closed_form_truncated(C, rho, N, mask))
    if rho == 0.5 and N == 4 and not mask:
        assert np.max(np.abs(oracle.neumann_int8(A, N, mask)[0] - _closed_form_truncated(C, rho, N, mask))) > 1.0


def test_int16_quantiser_properties():
    """N = 1 returns I + A': codes in [-32639, 32639] under one power-of-two scale 2^e per
    block, round to nearest (|A' - A| <= 2^(e-1)), and the finest scale that does not
    exceed the code range."""
    A = _rand_A(14, 16, 64).astype(np.float32).astype(np.float64)
    Ad = oracle.neumann_int16(A, 1, False) - np.eye(64)
    for b in range(A.shape[0]):
        amax = np.max(np.abs(A[b]))
        e = math.frexp(amax / 32639.0)[1]
        if amax <= 32639.0 * 2.0 ** (e - 1):
            e -= 1
        q = Ad[b] * 2.0 ** -e
        np.testing.assert_array_equal(q, np.round(q))
        assert np.max(np.abs(q)) <= 32639
        assert np.max(np.abs(Ad[b] - A[b])) <= 2.0 ** (e - 1)
        assert 32639.0 * 2.0 ** (e - 1) < amax <= 32639.0 * 2.0 ** e


def test_int16_code_range_splits_into_two_int8_digits():
    """The reading's code bound: every q with |q| <= 32639 is 256 hi + lo with both balanced
    digits in [-128, 127] (the form in which 8-bit matrix units take it), and 32640 is
    not (its hi digit would be 128)."""
    q = np.arange(-32639, 32640)
    lo = ((q + 128) & 255) - 128
    hi = (q - lo) >> 8
    np.testing.assert_array_equal(256 * hi + lo, q)
    assert lo.min() >= -128 and lo.max() <= 127 and hi.min() >= -128 and hi.max() <= 127
    assert ((32640 - (((32640 + 128) & 255) - 128)) >> 8) == 128


def test_int16_chain_close_to_fp64_on_c1_inputs():
    """16-bit codes keep T - I within 1e-4 of the fp64 masked sum (int8: 2e-2)."""
    A = _rand_A(13, 24, 64).astype(np.float32).astype(np.float64)
    T16 = oracle.neumann_int16(A, 3, True)
    Tf = oracle.neumann(A, 3, True)
    I = np.eye(64)
    assert _relF(T16 - I, Tf - I) < 1e-4
    assert _relF(T16 - I, Tf - I) < 0.01 * _relF(oracle.neumann_int8(A, 3, True) - I, Tf - I)


# ---------------------------------------------------------------- fp8 (e4m3) chain
# [GEO] "Adaptation a la Quantification" runs the power chain on low-bit operands; the
# e4m3 reading (format, rounding, scales, counters) is stated in oracle/gdn_oracle.c.
# These pins are independent of the oracle's arithmetic: the e4m3 value set is decoded
# from the bit layout and searched exhaustively, and the chain is checked on
# A = -(7/16) L, whose scales are powers of two, against closed forms derived by hand.

def _e4m3_table():
    """All finite non-negative e4m3 values with their codes, decoded from the bits
    (sign | 4 exponent bits, bias 7 | 3 mantissa bits; code 0x7f is NaN)."""
    vals, codes = [], []
    for code in range(0x7f):
        e, m = code >> 3, code & 7
        vals.append(m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
        codes.append(code)
    return np.array(vals), np.array(codes)


def _e4m3_nearest(y):
    """Exhaustive nearest e4m3 value, ties to the even code."""
    vals, codes = _e4m3_table()
    y = np.asarray(y, dtype=np.float64)
    d = np.abs(np.abs(y)[..., None] - vals)
    dmin = d.min(axis=-1, keepdims=True)
    # among the nearest, prefer the even code (there are at most two candidates)
    score = np.where(d == dmin, (codes & 1).astype(np.float64), np.inf)
    pick = vals[np.argmin(score, axis=-1)]
    return np.copysign(pick, y)


def test_e4m3_value_set_and_rounding_match_the_code_table():
    vals, _ = _e4m3_table()
    assert vals.max() == 448.0 and vals[1] == 2.0 ** -9 and len(np.unique(vals)) == 127
    # every representable value rounds to itself
    np.testing.assert_array_equal(oracle.e4m3_round(vals), vals)
    np.testing.assert_array_equal(oracle.e4m3_round(-vals), -vals)
    # midpoints between neighbours are ties: they go to the even code
    mids = (vals[1:] + vals[:-1]) / 2
    np.testing.assert_array_equal(oracle.e4m3_round(mids), _e4m3_nearest(mids))
    rng = np.random.default_rng(7)
    y = np.sign(rng.standard_normal(20000)) * np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448.0), 20000))
    np.testing.assert_array_equal(oracle.e4m3_round(y), _e4m3_nearest(y))
    # hand values: 2^-10 is half the smallest subnormal (tie -> code 0); 1.0625 lies
    # between 1 (code 0x38) and 1.125 (0x39): tie -> 1; 17 -> 16 (0x58) over 18 (0x59)
    np.testing.assert_array_equal(oracle.e4m3_round([2.0 ** -10, 1.5 * 2.0 ** -10, 1.0625, 1.1875, -17.0]),
                                  [0.0, 2.0 ** -9, 1.0, 1.25, -16.0])


def _rho_L(C, rho):
    return (-rho * np.tril(np.ones((C, C)), -1))[None]


def _f32_quant_dequant(x, s):
    """s * e4m3(clamp(x * (1/s))) with every scalar step in fp32 (the stated reading)."""
    s = np.float32(s)
    inv = np.float32(1.0) / s
    y = (np.asarray(x, dtype=np.float32) * inv).astype(np.float32)
    y = np.clip(y, np.float32(-448), np.float32(448))
    return (_e4m3_nearest(y).astype(np.float32) * s).astype(np.float32)


def test_fp8_chain_closed_form_rho_7_16():
    """A = -(7/16) L (L strictly lower, all ones), C = 64.  absmax(A) = 7/16 = 448 2^-10, so
    s_A = 2^-10, every code of A is -448 and A' = A.  X_1 = A', so its codes are -448 too,
    and the first product is exact: X_2(d) = -7/16 + (49/256)(d - 1) on subdiagonal d.
    Static saturations of X_2: |X_2| 2^10 >= 464 iff d >= 6, i.e. sum_{d=6}^{63}(64 - d)
    = 1711 entries; the mask (N = 2) keeps d <= 2, where |X_2| <= 7/16: none."""
    C = 64
    A = _rho_L(C, 7 / 16)
    d = np.subtract.outer(np.arange(C), np.arange(C))
    x2 = np.where(d >= 1, -7 / 16 + 49 / 256 * (d - 1), 0.0)
    # N = 1: T = I + A' = I + A (A is exactly representable)
    T, cnt, am = oracle.neumann_fp8(A, 1, False)
    np.testing.assert_array_equal(T[0], np.eye(C) + A[0])
    np.testing.assert_array_equal(cnt[0], [0, 0, 0, 0])
    # N = 2, unmasked: T - I = s_T e4m3(X_2 / s_T), s_T = absmax(X_2) / 448
    T, cnt, am = oracle.neumann_fp8(A, 2, False)
    assert am[0].tolist() == [7 / 16, 7 / 16, -7 / 16 + 49 / 256 * 62]
    sT = np.float32(np.float32(am[0][2]) / np.float32(448.0))
    np.testing.assert_array_equal(T[0], np.eye(C) + _f32_quant_dequant(x2, sT))
    np.testing.assert_array_equal(cnt[0], [0, 0, 1711, 0])
    # N = 2, masked: band d <= 2 of X_2 = {-7/16, -63/256}; s_T = 2^-10 again, and
    # -63/256 * 2^10 = -252 rounds to -256 (step 16 in [128, 256)): T - I = -1/4 there
    T, cnt, _ = oracle.neumann_fp8(A, 2, True)
    expect = np.where(d == 1, -7 / 16, np.where(d == 2, -0.25, 0.0))
    np.testing.assert_array_equal(T[0], np.eye(C) + expect)
    np.testing.assert_array_equal(cnt[0], [0, 0, 0, 0])


@pytest.mark.parametrize("N", [2, 3, 4])
def test_fp8_mask_keeps_the_static_range(N):
    """With the mask, T - I of A = -rho L is -rho (1 - rho)^(d-1) on d <= N: no entry
    exceeds rho = absmax(A), so under A's (static) scale nothing saturates; unmasked,
    the powers' binomial growth saturates it ([GEO] Methodologie 2)."""
    A = _rho_L(64, 7 / 16)
    _, cm, _ = oracle.neumann_fp8(A, N, True)
    _, cu, _ = oracle.neumann_fp8(A, N, False)
    assert cm[0].tolist() == [0, 0, 0, 0]
    assert cu[0][2] >= 1711 and cu[0][0] == 0 and cu[0][1] == 0


@pytest.mark.parametrize("mask", [True, False])
def test_fp8_chain_close_to_fp64_on_c1_inputs(mask):
    """Within the fp8 tolerance of the unquantised sum on c1-like blocks: e4m3 keeps 3
    mantissa bits (relative step 2^-3, rounding error <= 2^-4 per quantisation)."""
    A = _rand_A(31, 48, 64).astype(np.float32).astype(np.float64)
    T8, cnt, am = oracle.neumann_fp8(A, 3, mask)
    T64 = oracle.neumann(A, 3, mask)
    assert _relF(T8, T64) <= 5e-2
    eye = np.eye(64)
    assert _relF(T8 - eye, T64 - eye) <= 6e-2
    assert np.all(np.triu(T8[:, :, :], 1) == 0) and np.all(np.diagonal(T8, axis1=1, axis2=2) == 1)
    assert cnt[:, 0].sum() == 0 and cnt[:, 1].sum() == 0
    assert np.all(am[:, 0] > 0)
