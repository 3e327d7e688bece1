"""GPU parity of the decode kernel (gated delta rule token by token, state on chip for
the whole call) against the oracle's token recurrence on the same seeded inputs.

Tolerances (relative Frobenius error over the whole output): fp32 arithmetic, 1e-5 on
O and S (d_k-term fp32 dot products per token, error growth over <= 64 tokens stays far
below that); O stored in bf16 adds its rounding, at most 2^-9 relative per element, so
2e-3 there."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")

TOL32, TOLO16 = 1e-5, 2e-3


def _state(seed, B, H, dk, dv):
    rng = np.random.default_rng(seed)
    return torch.from_numpy((0.5 * rng.standard_normal((B, H, dk, dv))).astype(np.float32))


def _ref(x, S0, scale):
    return oracle.recurrence(f64(x["Q"]), f64(x["K"]), f64(x["V"]), f64(x["beta"]), f64(x["g"]),
                             scale, None if S0 is None else f64(S0))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 256), (64, 96)])
@pytest.mark.parametrize("n", [1, 3, 5, 64])
def test_decode_parity(dk, dv, n):
    B, H = 2, 3
    say(f"decode dk={dk} dv={dv} n={n}")
    x = synth.prefill(40 + n, B, H, n, dk, dv)
    S0 = _state(n, B, H, dk, dv)
    O, S = tri.gdn_decode(*(cuda(x[k]) for k in ("Q", "K", "V", "beta", "g")), S=cuda(S0),
                          o_dtype=torch.float32)
    torch.cuda.synchronize()
    Or, Sr = _ref(x, S0, dk ** -0.5)
    assert relF(f64(O), Or) <= TOL32, relF(f64(O), Or)
    assert relF(f64(S), Sr) <= TOL32, relF(f64(S), Sr)


def test_decode_fp32_inputs_zero_state_bf16_out():
    B, H, n, dk, dv = 3, 2, 17, 128, 128
    say("decode fp32 inputs, S0 = 0, O bf16")
    x = synth.prefill(5, B, H, n, dk, dv, family="uniform")
    x32 = {k: (v.float() if k in ("Q", "K", "V") else v) for k, v in x.items()}
    rng = np.random.default_rng(9)
    x32["V"] = torch.from_numpy(rng.standard_normal((B, H, n, dv)).astype(np.float32))
    O, S = tri.gdn_decode(*(cuda(x32[k]) for k in ("Q", "K", "V", "beta", "g")), scale=0.3)
    torch.cuda.synchronize()
    assert O.dtype == torch.bfloat16
    Or, Sr = _ref(x32, None, 0.3)
    assert relF(f64(O), Or) <= TOLO16, relF(f64(O), Or)
    assert relF(f64(S), Sr) <= TOL32, relF(f64(S), Sr)


def test_decode_in_place_and_split_calls():
    """S_out = S updates the state in place; n tokens in one call equal the same tokens
    fed one call at a time with the state carried."""
    B, H, n, dk, dv = 2, 4, 9, 128, 128
    say("decode in place, split calls")
    x = synth.prefill(77, B, H, n, dk, dv)
    S0 = _state(3, B, H, dk, dv)
    xd = {k: cuda(v) for k, v in x.items()}
    S = cuda(S0)
    O_all, _ = tri.gdn_decode(xd["Q"], xd["K"], xd["V"], xd["beta"], xd["g"], S=S, S_out=S,
                              o_dtype=torch.float32)
    S2 = cuda(S0)
    outs = []
    for t in range(n):
        sl = lambda k: xd[k][:, :, t:t + 1].contiguous()
        o, _ = tri.gdn_decode(sl("Q"), sl("K"), sl("V"), sl("beta"), sl("g"), S=S2, S_out=S2,
                              o_dtype=torch.float32)
        outs.append(o)
    torch.cuda.synchronize()
    Or, Sr = _ref(x, S0, dk ** -0.5)
    assert relF(f64(O_all), Or) <= TOL32
    assert relF(f64(S), Sr) <= TOL32
    O_split = torch.cat(outs, dim=2)
    assert relF(f64(O_split), f64(O_all)) <= 1e-6
    assert relF(f64(S2), f64(S)) <= 1e-6


def test_decode_zero_tokens_copies_state():
    B, H, dk, dv = 2, 2, 64, 64
    say("decode n = 0")
    x = synth.prefill(1, B, H, 0, dk, dv)
    S0 = cuda(_state(4, B, H, dk, dv))
    xd = [cuda(x[k]) for k in ("Q", "K", "V", "beta", "g")]
    _, S = tri.gdn_decode(*xd, S=S0)
    _, Z = tri.gdn_decode(*xd)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)
    assert torch.count_nonzero(Z).item() == 0


@pytest.mark.parametrize("B,H,n", [(64, 32, 1), (1, 32, 64)])
def test_decode_bench_shapes(B, H, n):
    """The two timed decode workloads: one step for a batch of 64 sequences, and 64
    tokens of one sequence with the state kept on chip (32 heads, d = 128)."""
    dk = dv = 128
    say(f"decode bench shape B={B} H={H} n={n}")
    x = synth.prefill(6, B, H, n, dk, dv)
    S0 = _state(6, B, H, dk, dv)
    O, S = tri.gdn_decode(*(cuda(x[k]) for k in ("Q", "K", "V", "beta", "g")), S=cuda(S0))
    torch.cuda.synchronize()
    Or, Sr = _ref(x, S0, dk ** -0.5)
    assert relF(f64(O), Or) <= TOLO16, relF(f64(O), Or)
    assert relF(f64(S), Sr) <= TOL32, relF(f64(S), Sr)
