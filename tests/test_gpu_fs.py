"""GPU forward substitution (the sequential baseline) against the oracle's forward
substitution on the same inputs: fp32, tolerance 1e-5 relative Frobenius on T and 1e-4
on T - I; upper triangle exactly zero, diagonal exactly one."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import cuda, eye_off, f64, relF, say

pytestmark = pytest.mark.gpu

tri = pytest.importorskip("tri_inverse_amd")


@pytest.mark.parametrize("C", [16, 32, 64, 128])
def test_fs_parity_from_keys(C):
    nb = 45 if C <= 64 else 11
    say(f"fs from keys C={C}")
    inp = synth.blocks(51, nb, C, 128, k_dtype="bf16")
    T = f64(tri.gdn_tri_inverse_fs(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C))
    torch.cuda.synchronize()
    Tr = oracle.fs_inverse(oracle.build_A(f64(inp["K"]), f64(inp["beta"]), f64(inp["g"])))
    assert relF(T, Tr) <= 1e-5, relF(T, Tr)
    assert relF(eye_off(T), eye_off(Tr)) <= 1e-4, relF(eye_off(T), eye_off(Tr))
    i, j = np.indices((C, C))
    assert np.all(T[:, j > i] == 0) and np.all(T[:, i == j] == 1)


def test_fs_from_given_A_matches_exact_products():
    """A given in fp32; forward substitution and the exact doubling product both give
    (I - A)^-1."""
    C, nb = 64, 32
    say("fs from A")
    inp = synth.blocks(0, nb, C, 128, k_dtype="f64")
    A32 = oracle.build_A(inp["K"], inp["beta"], inp["g"]).astype(np.float32)
    Ad = cuda(torch.from_numpy(A32))
    T = f64(tri.gdn_tri_inverse_fs(A=Ad, C=C))
    Tx = f64(tri.gdn_tri_inverse_exact(A=Ad, C=C, compute="f32"))
    torch.cuda.synchronize()
    Tr = oracle.fs_inverse(A32.astype(np.float64))
    assert relF(T, Tr) <= 1e-5
    assert relF(T, Tx) <= 2e-5


@pytest.mark.parametrize("t_dtype", [torch.float32, torch.bfloat16])
def test_fs128_from_given_A(t_dtype):
    """C = 128 with A given in fp32 (the oracle's A rounded to fp32); bf16 output is the
    rounded fp32 result."""
    C, nb = 128, 7
    say(f"fs128 from A t_dtype={t_dtype}")
    inp = synth.blocks(3, nb, C, 128, k_dtype="f64")
    A32 = oracle.build_A(inp["K"], inp["beta"], inp["g"]).astype(np.float32)
    T = tri.gdn_tri_inverse_fs(A=cuda(torch.from_numpy(A32)), C=C, t_dtype=t_dtype)
    torch.cuda.synchronize()
    Tr = oracle.fs_inverse(A32.astype(np.float64))
    tol = 1e-5 if t_dtype == torch.float32 else 4e-3
    assert relF(f64(T), Tr) <= tol, relF(f64(T), Tr)
    i, j = np.indices((C, C))
    Tn = f64(T)
    assert np.all(Tn[:, j > i] == 0) and np.all(Tn[:, i == j] == 1)


@pytest.mark.parametrize("C", [32, 64, 128])
def test_fs_full_size_sampled_blocks(C):
    """B=1, H=16, seq 8192 (4096 / 2048 / 1024 blocks): the launches the speedup
    measurement times; 32 sampled blocks against the oracle."""
    nb = 16 * 8192 // C
    say(f"fs full size C={C}")
    inp = synth.blocks(1, nb, C, 128, k_dtype="bf16")
    T = f64(tri.gdn_tri_inverse_fs(K=cuda(inp["K"]), beta=cuda(inp["beta"]), g=cuda(inp["g"]), C=C))
    torch.cuda.synchronize()
    idx = np.random.default_rng(3).choice(nb, 32, replace=False)
    Tr = oracle.fs_inverse(oracle.build_A(f64(inp["K"][idx]), f64(inp["beta"][idx]), f64(inp["g"][idx])))
    assert relF(T[idx], Tr) <= 1e-5, relF(T[idx], Tr)
