"""Throughput of the GDN intra-chunk solve on one MI355X.

Headline workload (one "step"): the batched 64x64 tri-inverse over B=1, H=16,
seq 8192 -> 2048 blocks, bf16 keys (d_k = 128), fp32 beta and log-gates, A built in
the kernel, T = band-masked truncated Neumann sum with N = 3 (the pages' method),
T written as fp32.  value = 64x64 blocks per second.

The same JSON line also carries the other inverse variants of that workload and, when
the library has it, the full chunk-wise prefill forward (B=4, H=16, seq 8192,
d_k = d_v = 128, C = 64) in tokens per second, each with its roofline.

Inputs are seeded synthetic tensors (see synth/), resident in HBM before timing.
Eight input/output buffer sets are rotated so that successive launches do not hit
the 256 MB Infinity Cache.  Kernel durations come from HIP events recorded on the
stream the kernels are launched on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only c1|c3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA
INT8_PEAK_TOPS = 5000.0        # dense int8 MFMA
N_SETS = 8


def source_digest(files=None) -> str:
    """Hash of HIP sources (all of csrc/, or the named files of it): recorded next to
    counter-derived traffic figures so a stale measurement is never reported for a
    changed kernel."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tri_inverse_amd", "csrc")
    names = files if files else [n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp", ".cpp", ".h"))]
    for name in sorted(names):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it was taken
    on the current sources of that kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    ent = data.get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest(ent.get("source_files")):
        return None
    return ent.get("hbm_bytes_per_launch")


def time_launches(torch, launch, n_sets, steps, warmup, repeats=7):
    """Run `launch(set_index)` `warmup` times eagerly, then capture exactly `steps`
    launches (rotating buffer sets) in one HIP graph.  The graph is replayed once
    untimed, then `repeats` times, each replay timed on its own with HIP events on the
    replay stream (each timed region holds exactly `steps` launches).  Returns the
    median ms per launch and the list of all repeats.  Replaying a graph keeps Python's
    per-call overhead out of the timed region, so back-to-back kernels run without
    host-induced gaps; the median of several replays keeps clock ramps and one-off
    stalls out of the figure."""
    for i in range(warmup):
        launch(i % n_sets)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(steps):
            launch(k % n_sets)
    graph.replay()  # untimed: first replay uploads the graph
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(repeats):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) / steps)
    del graph
    ms = sorted(per)[len(per) // 2]
    return ms, per


# ------------------------------------------------------------------ c1: tri-inverse

C1 = dict(B=1, H=16, T=8192, C=64, d_k=128)


def c1_bytes_flops(variant, t_bytes=4):
    C, dk = C1["C"], C1["d_k"]
    n_blocks = C1["B"] * C1["H"] * C1["T"] // C
    per_block_bytes = C * dk * 2 + 2 * C * 4 + C * C * t_bytes
    gram = 2 * C * C * dk
    if variant[0] == "exact":
        m = (C - 1).bit_length()
        prods = 2 * (m - 1)
    elif variant[0] == "residual":  # N-1 for T0, 1 for E, S Horner steps, 1 for T0 R
        prods = variant[1] - 1 + 1 + variant[4] + 1
    else:
        prods = variant[1] - 1
    flops = gram + prods * 2 * C ** 3
    return n_blocks, n_blocks * per_block_bytes, n_blocks * flops


def bench_c1(torch, tri, synth, steps, warmup):
    C = C1["C"]
    n_blocks = C1["B"] * C1["H"] * C1["T"] // C
    sets = []
    for s in range(N_SETS):
        inp = synth.blocks(1 if s == 0 else 1000 + s, n_blocks, C, C1["d_k"], k_dtype="bf16")
        sets.append({k: v.cuda() for k, v in inp.items()})
    outs32 = [torch.empty((n_blocks, C, C), device="cuda") for _ in range(N_SETS)]
    outs16 = [torch.empty((n_blocks, C, C), device="cuda", dtype=torch.bfloat16) for _ in range(N_SETS)]

    def mk(variant, t_dtype):
        outs = outs32 if t_dtype == torch.float32 else outs16

        def launch(i):
            x = sets[i]
            if variant[0] == "exact":
                tri.gdn_tri_inverse_exact(K=x["K"], beta=x["beta"], g=x["g"], C=C, compute="bf16",
                                          out=outs[i])
            elif variant[0] == "int8":
                tri.gdn_tri_inverse_neumann(K=x["K"], beta=x["beta"], g=x["g"], C=C, N=variant[1],
                                            mask=variant[2], compute="int8", out=outs[i])
            elif variant[0] == "residual":
                tri.gdn_tri_inverse_residual(K=x["K"], beta=x["beta"], g=x["g"], C=C, N=variant[1],
                                             mask=variant[2], S=variant[4], compute="f32", out=outs[i])
            else:
                tri.gdn_tri_inverse_neumann(K=x["K"], beta=x["beta"], g=x["g"], C=C, N=variant[1],
                                            mask=variant[2], compute="bf16", out=outs[i])
        return launch

    results = {}
    variants = [("neumann", 3, True, torch.float32), ("neumann", 2, True, torch.float32),
                ("neumann", 4, True, torch.float32), ("neumann", 2, False, torch.float32),
                ("neumann", 3, False, torch.float32), ("neumann", 4, False, torch.float32),
                ("exact", 0, False, torch.float32), ("exact", 0, False, torch.bfloat16),
                ("neumann", 3, True, torch.bfloat16), ("residual", 3, True, torch.float32, 8),
                ("int8", 3, True, torch.float32), ("int8", 3, False, torch.float32)]
    for v in variants:
        name = ("exact" if v[0] == "exact" else "N%d_%s" % (v[1], "masked" if v[2] else "unmasked"))
        if v[0] == "residual":
            name = "N%d_masked_residual_S%d_f32" % (v[1], v[4])
        elif v[0] == "int8":
            name = "N%d_%s_int8" % (v[1], "masked" if v[2] else "unmasked")
        name += "_T" + ("f32" if v[3] == torch.float32 else "bf16")
        st = steps if v == variants[0] else max(10, steps // 2)
        ms_step, reps = time_launches(torch, mk(v, v[3]), N_SETS, st, warmup)
        ms_kernel = ms_step
        nb, by, fl = c1_bytes_flops(v, 4 if v[3] == torch.float32 else 2)
        if v[0] == "int8":  # bf16 Gram, int8 products: MFMA time at each one's peak
            gram = nb * 2 * C * C * C1["d_k"]
            t_mfma = gram / (BF16_PEAK_TFLOPS * 1e12) + (fl - gram) / (INT8_PEAK_TOPS * 1e12)
        else:
            t_mfma = fl / (BF16_PEAK_TFLOPS * 1e12)
        results[name] = {
            "ms_per_step": ms_step, "ms_kernel": ms_kernel,
            "repeats_ms": [round(x, 5) for x in reps],
            "blocks_per_s": nb / (ms_step * 1e-3),
            "hbm_frac": by / (ms_kernel * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_frac": t_mfma / (ms_kernel * 1e-3),
            "bytes": by, "flops": fl,
        }
    return results


def bench_fs_speedup(torch, tri, synth, steps, warmup):
    """The pages' headline metric: speedup of the multiplication-only inverses over
    forward substitution, here both on MI355X.  B=1, H=16, seq 8192 at C = 32, 64 and
    128 (4096 / 2048 / 1024 blocks), A built in-kernel from bf16 keys, T fp32; forward
    substitution in fp32 (the sequential baseline), the masked N=3 sum and exact
    doubling in bf16."""
    res = {}
    for C in (32, 64, 128):
        nb = C1["B"] * C1["H"] * C1["T"] // C
        sets = [{k: v.cuda() for k, v in synth.blocks(1 if s == 0 else 1000 + s, nb, C, C1["d_k"],
                                                       k_dtype="bf16").items()} for s in range(N_SETS)]
        outs = [torch.empty((nb, C, C), device="cuda") for _ in range(N_SETS)]
        calls = {
            "fs": lambda x, o: tri.gdn_tri_inverse_fs(K=x["K"], beta=x["beta"], g=x["g"], C=C, out=o),
            "N3_masked": lambda x, o: tri.gdn_tri_inverse_neumann(K=x["K"], beta=x["beta"], g=x["g"], C=C, N=3,
                                                                  mask=True, compute="bf16", out=o),
            "exact": lambda x, o: tri.gdn_tri_inverse_exact(K=x["K"], beta=x["beta"], g=x["g"], C=C,
                                                            compute="bf16", out=o),
        }
        ms = {}
        for name, f in calls.items():
            ms[name], _ = time_launches(torch, lambda i, f=f: f(sets[i], outs[i]), N_SETS, steps, warmup)
        res[f"C{C}"] = {"n_blocks": nb, "us_fs": ms["fs"] * 1e3, "us_N3_masked": ms["N3_masked"] * 1e3,
                        "us_exact": ms["exact"] * 1e3,
                        "speedup_N3_masked_over_fs": ms["fs"] / ms["N3_masked"],
                        "speedup_exact_over_fs": ms["fs"] / ms["exact"]}
        del sets, outs
        torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ c3 / c4: chunk forward

C3 = dict(B=4, H=16, T=8192, d_k=128, d_v=128, C=64)
C4 = dict(B=4, H=16, T=32768, d_k=128, d_v=128, C=64)


def chunk_bytes_flops(cfg, variant):
    B, H, T, dk, dv, C = (cfg[k] for k in ("B", "H", "T", "d_k", "d_v", "C"))
    tokens = B * H * T
    by = tokens * (2 * dk * 2 + dv * 2) + tokens * 2 * 4 + tokens * dv * 2 + B * H * dk * dv * 4
    n_chunks = tokens // C
    inv = (2 * (((C - 1).bit_length()) - 1) if variant[0] == "exact" else variant[1] - 1) * 2 * C ** 3
    per_chunk = (2 * C * C * dk          # K K^T
                 + inv                   # inverse products
                 + 2 * C * C * dk        # W = T diag(beta e^G) K
                 + 2 * C * C * dv        # U = T diag(beta) V
                 + 2 * C * dk * dv       # W S
                 + 2 * C * dk * dv       # Q S
                 + 2 * C * C * dk        # Q K^T
                 + 2 * C * C * dv        # P U'
                 + 2 * dk * C * dv)      # K^T U'
    return B * T, by, n_chunks * per_chunk


def bench_chunk(torch, tri, synth, cfg, variants, steps, warmup, n_sets=2, stats=False):
    B, H, T, dk, dv, C = (cfg[k] for k in ("B", "H", "T", "d_k", "d_v", "C"))
    sets = []
    for s in range(n_sets):
        x = synth.prefill(3 if s == 0 else 100 + s, B, H, T, dk, dv)
        sets.append({k: v.cuda() for k, v in x.items()})
        del x
    outs = [(torch.empty((B, H, T, dv), device="cuda", dtype=torch.bfloat16),
             torch.empty((B, H, dk, dv), device="cuda")) for _ in range(n_sets)]
    st = torch.zeros(4, dtype=torch.int64, device="cuda") if stats else None
    res = {}
    for v in variants:
        mode, N, mask, compute = v
        # one workspace for every launch: they run one after another on one stream
        need = tri.gdn_chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, mode, N, mask, compute)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None

        def launch(i):
            x = sets[i]
            tri.gdn_chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], C=C, scale=dk ** -0.5,
                              mode=mode, N=N, mask=mask, compute=compute, O=outs[i][0],
                              S_out=outs[i][1], stats=st, workspace=ws)
        ms, _ = time_launches(torch, launch, n_sets, steps, warmup)
        tok, by, fl = chunk_bytes_flops(cfg, v)
        name = ("exact" if mode == "exact" else "N%d_%s" % (N, "masked" if mask else "unmasked")) + "_" + compute
        res[name] = {"ms_per_step": ms, "tokens_per_s": tok / (ms * 1e-3),
                     "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "mfma_frac": fl / (ms * 1e-3) / 1e12 / (FP8_PEAK_TFLOPS if compute == "fp8" else BF16_PEAK_TFLOPS),
                     "bytes": by, "flops": fl}
        if stats:
            launch(0)
            torch.cuda.synchronize()
            res[name]["fp8_stats"] = dict(zip(tri.FP8_STATS_FIELDS, st.cpu().tolist()))
    del sets, outs
    torch.cuda.empty_cache()
    return res


def bench_wy(torch, tri, synth, steps, warmup):
    """Chunk-size sweep: A build + inverse + W = T diag(beta) K, U = T diag(beta) V at B=2,
    H=16, seq 16384, d_k = d_v = 128, for C = 64, 128, 256 (8192 / 4096 / 2048 blocks),
    with the masked N=3 sum (the method), the unmasked one and the exact doubling product.
    Bytes: K, V, beta, g read once, W and U (bf16) written once (1032 B per token-head,
    independent of C).  FLOPs: the method's dense count per block: gram + the inverse's
    C x C products (N-1 for the sum, 2(m-1) for doubling, m = ceil(log2 C)) + the two WY
    products (2 C^2 d each)."""
    B, H, T, dk, dv = 2, 16, 16384, 128, 128
    res = {}
    for C in (64, 128, 256):
        nb = B * H * T // C
        sets = [{k: v.cuda() for k, v in synth.blocks(2 if s == 0 else 200 + s, nb, C, dk, k_dtype="bf16",
                                                       d_v=dv).items()} for s in range(2)]
        outs = [(torch.empty((nb, C, dk), device="cuda", dtype=torch.bfloat16),
                 torch.empty((nb, C, dv), device="cuda", dtype=torch.bfloat16)) for _ in range(2)]
        for mode, N, mask in (("neumann", 3, True), ("neumann", 3, False), ("exact", 0, False)):
            def launch(i):
                x = sets[i]
                tri.gdn_wy(x["K"], x["beta"], x["g"], x["V"], C=C, mode=mode, N=max(N, 1), mask=mask,
                           W_out=outs[i][0], U_out=outs[i][1])
            ms, _ = time_launches(torch, launch, 2, steps, warmup)
            tokens = B * T
            by = B * H * T * (dk * 2 + dv * 2 + 8 + dk * 2 + dv * 2)
            prods = 2 * ((C - 1).bit_length() - 1) if mode == "exact" else N - 1
            fl = nb * (2 * C * C * dk + prods * 2 * C ** 3 + 2 * C * C * dk + 2 * C * C * dv)
            name = f"C{C}_" + ("exact" if mode == "exact" else f"N{N}_{'masked' if mask else 'unmasked'}")
            res[name] = {"ms_per_step": ms, "tokens_per_s": tokens / (ms * 1e-3),
                         "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "mfma_frac": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                         "bytes": by, "flops": fl, "n_blocks": nb}
        del sets, outs
        torch.cuda.empty_cache()
    return res


DEC = dict(H=32, d_k=128, d_v=128)


def decode_bytes(B, H, n, dk, dv):
    """Compulsory bytes of one decode call: the fp32 state read and written once, q, k,
    v (bf16), beta and g read and o (bf16) written once per token."""
    return B * H * (2 * dk * dv * 4 + n * (2 * dk * 2 + dv * 2 + 8 + dv * 2))


def bench_decode(torch, tri, synth, steps, warmup):
    """Gated delta rule token by token (the decode kernel), 32 heads, d_k = d_v = 128,
    bf16 q/k/v/o, fp32 state updated in place:
      batch64_step: one token for each of 64 sequences (B=64, n=1), four 128 MiB state
        sets rotating so that the state is not served from the 256 MB Infinity Cache;
      seq64: 64 tokens of one sequence per call, the state kept on chip (B=1, n=64);
      batch1_step: one token of one sequence (B=1, n=1), the latency of one step."""
    H, dk, dv = DEC["H"], DEC["d_k"], DEC["d_v"]
    res = {}
    for name, B, n, n_sets in (("batch64_step", 64, 1, 4), ("seq64", 1, 64, 4), ("batch1_step", 1, 1, 4)):
        sets = []
        for i in range(n_sets):
            x = {k: v.cuda() for k, v in synth.prefill(60 + i, B, H, n, dk, dv).items()}
            x["S"] = torch.zeros((B, H, dk, dv), device="cuda")
            x["O"] = torch.empty((B, H, n, dv), device="cuda", dtype=torch.bfloat16)
            sets.append(x)

        def launch(i):
            x = sets[i]
            tri.gdn_decode(x["Q"], x["K"], x["V"], x["beta"], x["g"], S=x["S"], S_out=x["S"], O=x["O"])
        ms, _ = time_launches(torch, launch, n_sets, steps, warmup)
        by = decode_bytes(B, H, n, dk, dv)
        res[name] = {"B": B, "H": H, "tokens_per_call": n, "ms_per_step": ms,
                     "us_per_token": ms * 1e3 / n, "tokens_per_s": B * n / (ms * 1e-3),
                     "bytes": by, "hbm_frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        del sets
        torch.cuda.empty_cache()
    return res


def replay_launches(torch, launch, n_sets, n):
    """One eager pass over the buffer sets, then n launches captured in a HIP graph and
    replayed once: the profiler sees the launches back to back, as the timed region of
    the benchmark runs them."""
    for i in range(n_sets):
        launch(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(n):
            launch(k % n_sets)
    graph.replay()
    torch.cuda.synchronize()
    del graph


def profile_c1(torch, tri, synth, n):
    """Headline launch n times on rotating buffer sets (graph-replayed), then a plain
    256 MiB copy n times: the copy's FETCH_SIZE / WRITE_SIZE per dispatch calibrate the
    counters."""
    C = C1["C"]
    n_blocks = C1["B"] * C1["H"] * C1["T"] // C
    sets = [{k: v.cuda() for k, v in synth.blocks(1 if s == 0 else 1000 + s, n_blocks, C, C1["d_k"],
                                                  k_dtype="bf16").items()} for s in range(N_SETS)]
    outs = [torch.empty((n_blocks, C, C), device="cuda") for _ in range(N_SETS)]

    def launch(i):
        x = sets[i]
        tri.gdn_tri_inverse_neumann(K=x["K"], beta=x["beta"], g=x["g"], C=C, N=3, mask=True,
                                    compute="bf16", out=outs[i])
    replay_launches(torch, launch, N_SETS, n)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()


def profile_c3(torch, tri, synth, n):
    """Prefill forward (B=4 H=16 seq 8192, N=3 masked) n times (graph-replayed), then the
    256 MiB copy."""
    cfg = C3
    x = {k: v.cuda() for k, v in synth.prefill(3, cfg["B"], cfg["H"], cfg["T"], cfg["d_k"],
                                                cfg["d_v"]).items()}
    O = torch.empty((cfg["B"], cfg["H"], cfg["T"], cfg["d_v"]), device="cuda", dtype=torch.bfloat16)
    S = torch.empty((cfg["B"], cfg["H"], cfg["d_k"], cfg["d_v"]), device="cuda")
    def launch(i):
        tri.gdn_chunk_fwd(x["Q"], x["K"], x["V"], x["beta"], x["g"], C=64, scale=cfg["d_k"] ** -0.5,
                          N=3, mask=True, O=O, S_out=S)
    replay_launches(torch, launch, 1, n)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()


def profile_decode(torch, tri, synth, n):
    """Decode step for 64 sequences (B=64 H=32 d=128, four rotating 128 MiB state sets)
    n times (graph-replayed), then the 256 MiB copy."""
    B, H, dk, dv = 64, DEC["H"], DEC["d_k"], DEC["d_v"]
    sets = []
    for i in range(4):
        x = {k: v.cuda() for k, v in synth.prefill(60 + i, B, H, 1, dk, dv).items()}
        x["S"] = torch.zeros((B, H, dk, dv), device="cuda")
        x["O"] = torch.empty((B, H, 1, dv), device="cuda", dtype=torch.bfloat16)
        sets.append(x)
    def launch(i):
        x = sets[i]
        tri.gdn_decode(x["Q"], x["K"], x["V"], x["beta"], x["g"], S=x["S"], S_out=x["S"], O=x["O"])
    replay_launches(torch, launch, 4, n)
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline_c1():
    import oracle
    import synth
    n_blocks = C1["B"] * C1["H"] * C1["T"] // C1["C"]
    inp = synth.blocks(1, n_blocks, C1["C"], C1["d_k"], k_dtype="bf16")
    K = inp["K"].double().numpy()
    beta = inp["beta"].double().numpy()
    g = inp["g"].double().numpy()
    reps = 0
    t0 = time.perf_counter()
    while True:
        A = oracle.build_A(K, beta, g)
        oracle.neumann(A, 3, True)
        reps += 1
        if time.perf_counter() - t0 > 10.0 or reps >= 400:
            break
    dt = time.perf_counter() - t0
    cores = oracle.max_threads()
    # one thread, on the first 256 blocks of the same workload (about 2 s)
    sub = slice(0, 256)
    oracle.set_threads(1)
    try:
        reps1 = 0
        t1 = time.perf_counter()
        while True:
            A = oracle.build_A(K[sub], beta[sub], g[sub])
            oracle.neumann(A, 3, True)
            reps1 += 1
            if time.perf_counter() - t1 > 2.0 or reps1 >= 100:
                break
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_threads(cores)
    return {"value": reps * n_blocks / dt, "unit": "blocks/s", "cores": cores,
            "kind": "oracle",
            "sample": "the full 2048-block workload (A build + N=3 masked Neumann, fp64), "
                      "%d pass(es), %.1f s" % (reps, dt),
            "single_thread": {"value": reps1 * 256 / dt1, "unit": "blocks/s",
                              "sample": "256 of the 2048 blocks, %d pass(es), %.1f s" % (reps1, dt1)}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only", default="all")
    ap.add_argument("--profile-launches", type=int, default=0,
                    help="profiling mode: run the headline launch this many times plus a "
                         "256 MiB device copy (counter calibration), print nothing else")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import tri_inverse_amd as tri

    torch.cuda.set_device(0)
    if args.profile_launches:
        if args.only == "c3":
            profile_c3(torch, tri, synth, args.profile_launches)
        elif args.only == "decode":
            profile_decode(torch, tri, synth, args.profile_launches)
        else:
            profile_c1(torch, tri, synth, args.profile_launches)
        return
    c1 = bench_c1(torch, tri, synth, args.steps, args.warmup)
    head = c1["N3_masked_Tf32"]
    traffic = load_traffic("inverse_kernel<4,1,128,1,0,1>")
    roofline = {
        "bound": "hbm",
        "achieved": head["bytes"] / (head["ms_kernel"] * 1e-3) / 1e9,
        "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": head["bytes"] / (head["ms_kernel"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "traffic": traffic,
    }
    out = {
        "metric": "64×64 tri-inverse blocks/s; GDN chunk-fwd tokens/s; % MFMA/HBM roofline",
        "value": head["blocks_per_s"],
        "unit": "blocks/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded unit-norm bf16 keys, U(0,1) beta, log-sigmoid gates)",
        "config": {"workload": "batched 64x64 tri-inverse, B=1 H=16 seq=8192 (2048 blocks), "
                               "d_k=128 bf16 K, A built in-kernel, truncated Neumann N=3 + band "
                               "mask, fp32 accumulate, T fp32",
                   "n_blocks": 2048, "C": 64, "d_k": 128, "N": 3, "mask": True},
        "roofline": roofline,
        "timing": "each leg: K launches captured in one HIP graph, replayed 7 times, each "
                  "replay timed with HIP events on its stream; ms_per_step is the median",
        "variants": c1,
        "source_digest": source_digest(),
    }
    if args.only in ("all", "c3"):
        c3 = bench_chunk(torch, tri, synth, C3,
                         [("neumann", 3, True, "bf16"), ("neumann", 3, False, "bf16"),
                          ("exact", 0, False, "bf16")], max(5, args.steps // 5), 2)
        h3 = c3["N3_masked_bf16"]
        out["chunk_fwd"] = {
            "workload": "chunk-wise GDN prefill forward, B=4 H=16 seq=8192 d_k=d_v=128 C=64, "
                        "N=3 band-masked inverse, bf16 Q/K/V/O, fp32 state",
            "tokens_per_s": h3["tokens_per_s"], "ms_per_step": h3["ms_per_step"],
            "roofline": {"bound": "hbm", "achieved": h3["bytes"] / (h3["ms_per_step"] * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": h3["hbm_frac"],
                         "traffic": load_traffic("chunk_fwd_kernel<128,16,1,1,true>")},
            "variants": c3}
    if args.only in ("all", "fs"):
        out["fs_speedup"] = bench_fs_speedup(torch, tri, synth, max(10, args.steps // 2), 3)
    if args.only in ("all", "decode"):
        dec = bench_decode(torch, tri, synth, max(20, args.steps), 5)
        hd = dec["batch64_step"]
        out["decode"] = {
            "workload": "GDN decode, 32 heads, d_k=d_v=128, bf16 q/k/v/o, fp32 state in place; "
                        "headline: one step for 64 sequences",
            "tokens_per_s": hd["tokens_per_s"], "ms_per_step": hd["ms_per_step"],
            "roofline": {"bound": "hbm", "achieved": hd["bytes"] / (hd["ms_per_step"] * 1e-3) / 1e9,
                         "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hd["hbm_frac"],
                         "traffic": load_traffic("decode_kernel<128,true,true>")},
            "variants": dec}
    if args.only in ("all", "c2"):
        out["wy"] = bench_wy(torch, tri, synth, max(5, args.steps // 5), 2)
    if args.only in ("all", "c4"):
        out["chunk_fwd_fp8"] = bench_chunk(torch, tri, synth, C4,
                                           [("neumann", 3, True, "fp8"), ("neumann", 3, False, "fp8")],
                                           3, 1, n_sets=1, stats=True)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_c1()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
