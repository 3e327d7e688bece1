"""gdn_chunk_fwd_noalloc (the allocation-free chunk forward, for callers that cannot
allocate) against gdn_chunk_fwd with a caller workspace: same kernels on the same
inputs, so the results must be identical, on two calls in a row with the second
smaller (the scratch keeps the first call's contents and must not leak into the
second), for variants that use the scratch (pre-pass) and one that does not."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from helpers import cuda, say

tri = pytest.importorskip("tri_inverse_amd")


def _inv(mode="neumann", N=3, mask=True, compute="bf16"):
    return tri._inv_cfg(mode, N, mask, compute)


def test_noalloc_rejects_oversize_before_any_launch():
    """4 x 16 heads of 32768 tokens need 32768 chunks x 6144 bytes, past the 64 MiB the
    library holds: GDN_ERR_WORKSPACE (6) before anything is enqueued (fake pointers,
    never touched)."""
    FAKE = 0x10000
    cfg = _inv(mask=False)
    st = tri._lib.gdn_chunk_fwd_noalloc(FAKE, FAKE, FAKE, tri.GDN_BF16, FAKE, FAKE, None, FAKE, tri.GDN_BF16,
                                        FAKE, 4, 16, 32768, 128, 128, 64, 0.1, ctypes.byref(cfg), None, None)
    assert st == tri.GDN_ERR_WORKSPACE
    assert tri.gdn_chunk_fwd_workspace_bytes(4, 16, 32768, 128, 128, mask=False) > tri.GDN_NOALLOC_SCRATCH_BYTES


@pytest.mark.gpu
@pytest.mark.parametrize("variant", [("neumann", 3, False, "bf16"), ("neumann", 3, True, "fp8"),
                                     ("exact", 0, False, "bf16"), ("neumann", 3, True, "bf16")])
def test_noalloc_matches_workspace_entry_point(variant):
    mode, N, mask, compute = variant
    for (B, H, T, seed) in ((2, 8, 2048, 51), (1, 3, 320, 52)):
        say(f"noalloc {variant} B={B} H={H} T={T}")
        x = {k: cuda(v) for k, v in synth.prefill(seed, B, H, T, 128, 128).items()}
        st_a = torch.zeros(4, dtype=torch.int64, device="cuda")
        st_b = torch.zeros(4, dtype=torch.int64, device="cuda")
        O_a, S_a = tri.gdn_chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], C=64, mode=mode, N=N,
                                     mask=mask, compute=compute, stats=st_a)
        O_b, S_b = tri.gdn_chunk_fwd_noalloc(x["Q"], x["K"], x["V"], x["beta"], x["g"], C=64, mode=mode,
                                             N=N, mask=mask, compute=compute, stats=st_b)
        torch.cuda.synchronize()
        assert torch.equal(O_a, O_b)
        assert torch.equal(S_a, S_b)
        assert torch.equal(st_a, st_b)
