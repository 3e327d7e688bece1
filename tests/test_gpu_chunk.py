"""GPU parity of the WY products and of the chunk-wise forward against the fp64 oracle
running the same algorithm (same inverse variant) on the same seeded inputs.

Tolerances (relative Frobenius error over the whole output, or over the sampled heads
at full size): bf16 operands 2e-3, fp8 inverse 5e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")

TOL = {"bf16": 2e-3, "fp8": 5e-2}
INV = {"neumann": oracle.INV_NEUMANN, "exact": oracle.INV_EXACT}


# ------------------------------------------------------------------ WY products

def _wy_ref(inp, C, T64, gate_k):
    K = f64(inp["K"])
    return oracle.wy(T64, K, f64(inp["V"]), f64(inp["beta"]), f64(inp["g"]), gate_k)


@pytest.mark.parametrize("gate_k", [False, True])
@pytest.mark.parametrize("t_dtype", [torch.float32, torch.bfloat16])
def test_wy_with_given_T(gate_k, t_dtype):
    C, nb = 64, 45
    say(f"wy given T gate_k={gate_k} t_dtype={t_dtype}")
    inp = synth.blocks(7, nb, C, 128, k_dtype="bf16", d_v=128)
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    T64 = oracle.neumann(A64, 3, True)
    Tt = torch.from_numpy(T64).to(t_dtype)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]), C=C,
                      T=cuda(Tt), gate_k=gate_k, out_dtype=torch.float32)
    torch.cuda.synchronize()
    Wr, Ur = _wy_ref(inp, C, f64(Tt), gate_k)
    assert relF(f64(W), Wr) <= TOL["bf16"], relF(f64(W), Wr)
    assert relF(f64(U), Ur) <= TOL["bf16"], relF(f64(U), Ur)


@pytest.mark.parametrize("C", [32, 64])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("variant", [("neumann", 3, True), ("neumann", 3, False), ("exact", 0, False)])
def test_wy_forms_T(C, dk, dv, variant):
    mode, N, mask = variant
    nb = 37
    say(f"wy forms T C={C} dk={dk} dv={dv} {variant}")
    inp = synth.blocks(8, nb, C, dk, k_dtype="bf16", d_v=dv)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]), C=C,
                      mode=mode, N=N, mask=mask, out_dtype=torch.float32)
    torch.cuda.synchronize()
    A64 = oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"]))
    T64 = oracle.doubling(A64) if mode == "exact" else oracle.neumann(A64, N, mask)
    Wr, Ur = _wy_ref(inp, C, T64, False)
    assert relF(f64(W), Wr) <= TOL["bf16"], relF(f64(W), Wr)
    assert relF(f64(U), Ur) <= TOL["bf16"], relF(f64(U), Ur)


def test_wy_full_size_sampled_blocks():
    """B=2, H=16, seq 16384, C=64: 8192 blocks, bf16 outputs; 192 sampled blocks checked."""
    nb, C = 8192, 64
    say("wy full size 8192 blocks")
    inp = synth.blocks(2, nb, C, 128, k_dtype="bf16", d_v=128)
    W, U = tri.gdn_wy(cuda(inp["K"]), cuda(inp["beta"]), cuda(inp["g"]), cuda(inp["V"]), C=C,
                      mode="neumann", N=3, mask=True, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = np.random.default_rng(0).choice(nb, 192, replace=False)
    sub = {k: v[idx] for k, v in inp.items()}
    A64 = oracle.build_A(f64(sub["K"]), f64(sub["beta"]), f64(sub["g"]))
    Wr, Ur = _wy_ref(sub, C, oracle.neumann(A64, 3, True), False)
    assert relF(f64(W[idx]), Wr) <= TOL["bf16"]
    assert relF(f64(U[idx]), Ur) <= TOL["bf16"]


# ------------------------------------------------------------------ chunk forward

def _chunk_case(seed, B, H, T, dk, dv, family="sigmoid"):
    x = synth.prefill(seed, B, H, T, dk, dv, family=family)
    return x, {k: f64(v) for k, v in x.items()}


def _run_chunk(x, **kw):
    O, S = tri.gdn_chunk_fwd(cuda(x["Q"]), cuda(x["K"]), cuda(x["V"]), cuda(x["beta"]), cuda(x["g"]),
                             **kw)
    torch.cuda.synchronize()
    return f64(O), f64(S)


@pytest.mark.parametrize("variant", [("neumann", 3, True), ("neumann", 3, False), ("neumann", 2, True),
                                     ("neumann", 1, True), ("neumann", 5, True), ("exact", 0, False)])
def test_chunk_fwd_small(variant):
    mode, N, mask = variant
    B, H, T, dk, dv = 1, 3, 320, 128, 128   # 3 heads: the non-multiple-of-8 grid path
    say(f"chunk fwd small {variant}")
    x, x64 = _chunk_case(11, B, H, T, dk, dv)
    scale = dk ** -0.5
    O, S = _run_chunk(x, C=64, scale=scale, mode=mode, N=N, mask=mask, o_dtype=torch.float32)
    Or, Sr = oracle.chunk_fwd(x64["Q"], x64["K"], x64["V"], x64["beta"], x64["g"], 64, scale,
                              inv_mode=INV[mode], N=N, mask=mask)
    assert relF(O, Or) <= TOL["bf16"], relF(O, Or)
    assert relF(S, Sr) <= TOL["bf16"], relF(S, Sr)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 96)])
def test_chunk_fwd_shapes_and_initial_state(dk, dv):
    B, H, T = 2, 4, 256
    say(f"chunk fwd dk={dk} dv={dv} with S0")
    x, x64 = _chunk_case(12, B, H, T, dk, dv, family="uniform")
    S0 = torch.from_numpy(np.random.default_rng(3).standard_normal((B, H, dk, dv)).astype(np.float32) * 0.1)
    O, S = _run_chunk(x, C=64, scale=0.2, S0=cuda(S0), o_dtype=torch.bfloat16)
    Or, Sr = oracle.chunk_fwd(x64["Q"], x64["K"], x64["V"], x64["beta"], x64["g"], 64, 0.2,
                              N=3, mask=True, S0=f64(S0))
    assert relF(O, Or) <= TOL["bf16"], relF(O, Or)
    assert relF(S, Sr) <= TOL["bf16"], relF(S, Sr)


def test_chunk_fwd_exact_matches_token_recurrence():
    """With the exact inverse the chunk form is the token recurrence (pinned on the
    CPU); the GPU result must match the brute-force recurrence too."""
    B, H, T, dk, dv = 1, 2, 192, 64, 64
    say("chunk fwd exact vs recurrence")
    x, x64 = _chunk_case(13, B, H, T, dk, dv)
    O, S = _run_chunk(x, C=64, scale=0.125, mode="exact", o_dtype=torch.float32)
    Or, Sr = oracle.recurrence(x64["Q"], x64["K"], x64["V"], x64["beta"], x64["g"], 0.125)
    assert relF(O, Or) <= TOL["bf16"]
    assert relF(S, Sr) <= TOL["bf16"]


def test_chunk_fwd_split_sequence_carries_state():
    B, H, T, dk, dv = 1, 2, 256, 128, 64
    say("chunk fwd split sequence")
    x, _ = _chunk_case(14, B, H, T, dk, dv)
    O, S = _run_chunk(x, C=64, scale=0.1, o_dtype=torch.float32)
    h = {k: v[:, :, :128].contiguous() for k, v in x.items()}
    t = {k: v[:, :, 128:].contiguous() for k, v in x.items()}
    O1, S1 = _run_chunk(h, C=64, scale=0.1, o_dtype=torch.float32)
    O2, S2 = _run_chunk(t, C=64, scale=0.1, o_dtype=torch.float32, S0=cuda(torch.from_numpy(S1).float()))
    # the second half re-rounds the carried state once: bf16-level agreement
    assert relF(np.concatenate([O1, O2], axis=2), O) <= 1e-3
    assert relF(S2, S) <= 1e-3


def test_chunk_fwd_special_cases():
    B, H, T, dk, dv = 1, 2, 128, 64, 64
    say("chunk fwd beta=0 / empty")
    x, x64 = _chunk_case(15, B, H, T, dk, dv)
    z = dict(x)
    z["beta"] = torch.zeros_like(x["beta"])
    S0 = torch.from_numpy(np.random.default_rng(4).standard_normal((B, H, dk, dv)).astype(np.float32))
    O, S = _run_chunk(z, C=64, scale=1.0, S0=cuda(S0), o_dtype=torch.float32)
    # beta = 0: the state only decays, O = e^{G_t} q_t S0 with G the running gate sum
    Gt = np.cumsum(x64["g"], axis=2)
    Or = np.exp(Gt)[..., None] * np.einsum("bhtd,bhde->bhte", x64["Q"], f64(S0))
    assert relF(O, Or) <= TOL["bf16"]
    assert relF(S, np.exp(Gt[:, :, -1])[..., None, None] * f64(S0)) <= 1e-5
    # empty sequence
    e = {k: v[:, :, :0].contiguous() for k, v in x.items()}
    O0, S0o = tri.gdn_chunk_fwd(cuda(e["Q"]), cuda(e["K"]), cuda(e["V"]), cuda(e["beta"]),
                                cuda(e["g"]), C=64)
    assert O0.shape == (B, H, 0, dv)


@pytest.mark.parametrize("T", [64, 192])
@pytest.mark.parametrize("N,mask", [(3, True), (3, False)])
def test_chunk_fwd_short_sequences(T, N, mask):
    """One and three chunks: the staging, gate and product rings run their first and
    last iterations back to back."""
    B, H, dk, dv = 1, 2, 128, 128
    say(f"chunk fwd T={T} N={N} mask={mask}")
    x, x64 = _chunk_case(17, B, H, T, dk, dv)
    O, S = _run_chunk(x, C=64, scale=dk ** -0.5, N=N, mask=mask, o_dtype=torch.float32)
    Or, Sr = oracle.chunk_fwd(x64["Q"], x64["K"], x64["V"], x64["beta"], x64["g"], 64, dk ** -0.5,
                              N=N, mask=mask)
    assert relF(O, Or) <= TOL["bf16"], relF(O, Or)
    assert relF(S, Sr) <= TOL["bf16"], relF(S, Sr)


@pytest.mark.parametrize("N,mask", [(3, True), (3, False)])
def test_chunk_fwd_strong_gates(N, mask):
    """Log-gates near -2.6 per token: G falls below -80 inside every chunk, so exp(-G)
    would overflow fp32 and every gate factor is taken as exp of a difference."""
    B, H, T, dk, dv = 1, 2, 256, 128, 128
    say(f"chunk fwd strong gates N={N} mask={mask}")
    x = synth.prefill(16, B, H, T, dk, dv)
    x["g"] = (x["g"] - 2.5).contiguous()
    x64 = {k: f64(v) for k, v in x.items()}
    assert x64["g"][..., :32].sum(axis=-1).max() < -80.0
    O, S = _run_chunk(x, C=64, scale=dk ** -0.5, N=N, mask=mask, o_dtype=torch.float32)
    Or, Sr = oracle.chunk_fwd(x64["Q"], x64["K"], x64["V"], x64["beta"], x64["g"], 64, dk ** -0.5,
                              N=N, mask=mask)
    assert np.isfinite(O).all() and np.isfinite(S).all()
    assert relF(O, Or) <= TOL["bf16"], relF(O, Or)
    assert relF(S, Sr) <= TOL["bf16"], relF(S, Sr)


def test_chunk_fwd_fp8_inverse():
    B, H, T, dk, dv = 1, 4, 512, 128, 128
    say("chunk fwd fp8 inverse")
    x, x64 = _chunk_case(16, B, H, T, dk, dv)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    for mask in (True, False):
        O, S = _run_chunk(x, C=64, scale=dk ** -0.5, N=3, mask=mask, compute="fp8", stats=stats,
                          o_dtype=torch.float32)
        Or, Sr = oracle.chunk_fwd(x64["Q"], x64["K"], x64["V"], x64["beta"], x64["g"], 64, dk ** -0.5,
                                  N=3, mask=mask)
        assert relF(O, Or) <= TOL["fp8"], relF(O, Or)
        assert relF(S, Sr) <= TOL["fp8"], relF(S, Sr)
        s = stats.cpu().tolist()
        assert s[0] == 0 and s[1] == 0


def test_chunk_fwd_full_size_sampled_heads():
    """B=4, H=16, seq 8192, d_k = d_v = 128 (the prefill workload the bench times);
    two heads are recomputed by the oracle and compared."""
    B, H, T, dk, dv = 4, 16, 8192, 128, 128
    say("chunk fwd full size")
    x = synth.prefill(3, B, H, T, dk, dv)
    O, S = _run_chunk(x, C=64, scale=dk ** -0.5, N=3, mask=True, o_dtype=torch.bfloat16)
    for (b, h) in [(0, 0), (3, 15)]:
        sel = {k: f64(v[b:b + 1, h:h + 1]) for k, v in x.items()}
        Or, Sr = oracle.chunk_fwd(sel["Q"], sel["K"], sel["V"], sel["beta"], sel["g"], 64, dk ** -0.5,
                                  N=3, mask=True)
        assert relF(O[b:b + 1, h:h + 1], Or) <= TOL["bf16"], relF(O[b:b + 1, h:h + 1], Or)
        assert relF(S[b:b + 1, h:h + 1], Sr) <= TOL["bf16"], relF(S[b:b + 1, h:h + 1], Sr)


def test_chunk_fwd_fp8_full_size_sampled_heads():
    """B=4, H=16, seq 32768 with the fp8 inverse (the launch the fp8 measurement times),
    masked and unmasked: one head against the oracle, and no non-finite value or
    dynamic-scale saturation anywhere."""
    B, H, T, dk, dv = 4, 16, 32768, 128, 128
    say("chunk fwd fp8 full size")
    x = synth.prefill(3, B, H, T, dk, dv)
    stats = torch.zeros(4, dtype=torch.int64, device="cuda")
    sel = {k: f64(v[1:2, 7:8]) for k, v in x.items()}
    for mask in (True, False):
        O, S = _run_chunk(x, C=64, scale=dk ** -0.5, N=3, mask=mask, compute="fp8", stats=stats,
                          o_dtype=torch.bfloat16)
        s = stats.cpu().tolist()
        assert s[0] == 0 and s[1] == 0
        Or, Sr = oracle.chunk_fwd(sel["Q"], sel["K"], sel["V"], sel["beta"], sel["g"], 64, dk ** -0.5,
                                  N=3, mask=mask)
        assert relF(O[1:2, 7:8], Or) <= TOL["fp8"], relF(O[1:2, 7:8], Or)
        assert relF(S[1:2, 7:8], Sr) <= TOL["fp8"], relF(S[1:2, 7:8], Sr)
