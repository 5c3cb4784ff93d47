#!/usr/bin/env python3
"""Benchmark of libkda on one MI355X.

The headline line times the KDA prefill at the K3 layer shape (B=1, H=96,
T=8192, dk=dv=128, bf16 q/k/v/z, fp32 g/beta, fp32 state, chunk 64, output
gate, final state emitted): `value` is tokens/s with the inputs resident in
HBM.  The other workloads of the method (varlen prefill, the KCP scan of a
1M-token sequence, the decode step) are timed in the same run and reported
under "workloads".  The fp64 CPU oracle is timed on a sample of the headline
workload on the host's cores ("cpu_baseline") and its outputs double as a
parity spot check ("parity_sample").

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads a,b]

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
WARMUP_POLICY = ("the device peaks are measured first (about 1 s of GPU work, skipped with "
                 "--no-measured-peaks); then every workload runs `warmup` untimed calls "
                 "(decode: `warmup` untimed steps) before its timed calls")
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
METRIC = "KDA prefill tokens/s @H=96,d=128 (% MFMA peak); decode state GB/s (% HBM)"
ALL_WORKLOADS = ("varlen_prefill", "kcp_long_sequence", "decode", "prefill_checkpoints",
                 "decode_replay", "prefill_fused_gates", "decode_fused_gates", "prefill_chunk32",
                 "prefill_bounded_workspace", "kcp_bounded_workspace")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------ work model
def prefill_bytes(tokens: int, H: int, dk: int, dv: int, elt: int, gated: bool,
                  nseq: int, reads_s0: bool, writes_sT: bool, gate_elt: int = 4) -> int:
    """Algorithmic HBM bytes: every input read once, every output written once.
    gate_elt: bytes of a g / beta element (fp32 4; the fused entry points'
    pre-activations a / b take the storage dtype)."""
    per_th = 2 * dk * elt + dv * elt + (dv * elt if gated else 0) + dv * elt + (dk + 1) * gate_elt
    states = nseq * H * dk * dv * 4 * (int(reads_s0) + int(writes_sT))
    return tokens * H * per_th + states


def prefill_flops(tokens: int, H: int, dk: int, dv: int, C: int) -> float:
    """Triangle-aware flops of the chunked form per token-head:
    2 [3 dk dv + C (3 dk + 2 dv) / 2] (state products + intra-chunk products)."""
    return float(tokens) * H * 2 * (3 * dk * dv + C * (3 * dk + 2 * dv) / 2)


def decode_bytes(N: int, H: int, dk: int, dv: int, elt: int, gated: bool, gate_elt: int = 4) -> int:
    state = 2 * N * H * dk * dv * 4
    inputs = N * H * (2 * dk * elt + dv * elt + (dv * elt if gated else 0) + (dk + 1) * gate_elt)
    return state + inputs + N * H * dv * elt


# ------------------------------------------------------------------ helpers
ROOT = os.path.dirname(os.path.abspath(__file__))


def counter_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (calibrated against a plain copy), or None when the kernel's sources have
    changed since the counters were taken."""
    import hashlib
    try:
        rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))[kernel]
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
    except (OSError, KeyError, ValueError):
        return None
    return rec["traffic_bytes"] if h.hexdigest() == rec["src_sha256"] else None


def time_steps(fn, steps: int, warmup: int, torch, per_call: bool = False):
    """Average ms per call of fn over `steps` calls, HIP events on the current
    stream, after `warmup` untimed calls.  per_call: also the time of each call
    (events between the calls), as a third value."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps - 1)] if per_call else []
    start.record()
    for i in range(steps):
        fn()
        if per_call and i < steps - 1:
            marks[i].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / steps
    if per_call:
        ev = [start] + marks + [end]
        return ms, wall, [a.elapsed_time(b) for a, b in zip(ev[:-1], ev[1:])]
    return ms, wall


def measured_peaks(torch, dev):
    """Achievable peaks on this GPU through torch: a streaming read-and-write
    pass over 2 GiB (an fp32 elementwise multiply into a second buffer, the
    fastest of torch's copy, multiply and fill here: ~6.2 TB/s read + write,
    against ~5.3 for copy_), and a bf16 GEMM of 8192^3 (hipBLASLt); best of 5."""
    n = 2 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    _, _, t_copy = time_steps(lambda: torch.mul(src, 2.0, out=dst), 5, 2, torch, per_call=True)
    del src, dst
    m = 8192
    a = torch.randn(m, m, device=dev).to(torch.bfloat16)
    b = torch.randn(m, m, device=dev).to(torch.bfloat16)
    c = torch.empty(m, m, dtype=torch.bfloat16, device=dev)
    _, _, t_mm = time_steps(lambda: torch.matmul(a, b, out=c), 5, 3, torch, per_call=True)
    del a, b, c
    torch.cuda.empty_cache()
    return {"hbm_stream_gbs": 2 * n / (min(t_copy) * 1e-3) / 1e9,
            "bf16_gemm_tflops": 2 * m ** 3 / (min(t_mm) * 1e-3) / 1e12,
            "how": "fp32 x 2.0 over 2 GiB into a second buffer (read + write bytes) and "
                   "torch.matmul bf16 8192^3 (hipBLASLt), best of 5 each"}


def device_info(torch, dev):
    p = torch.cuda.get_device_properties(dev)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2 ** 30, 1)}


def gpu_inputs(torch, lens, H, dk, dv, gated, s0_std, seed, dev):
    """The synthetic recipe drawn on the GPU (kda_inputs.draw_on_device)."""
    import kda_inputs
    inp = kda_inputs.draw_on_device(lens, H, dk, dv, gated, s0_std, seed, dev)
    return dict(q=inp.q, k=inp.k, v=inp.v, z=inp.z, beta=inp.beta, g=inp.g, s0=inp.S0,
                cu=inp.cu_seqlens.to(dev))


# ------------------------------------------------------------------ workloads
def bench_headline(args, torch, kda, kda_inputs, dev):
    w = kda_inputs.WORKLOADS[1]
    H, dk, dv, T, C = w["H"], w["dk"], w["dv"], w["lens"][0], w["chunk"]
    log(f"headline k3_layer_prefill: drawing inputs H={H} T={T} d={dk}")
    inp = kda_inputs.make_workload(1)
    d = {n: getattr(inp, n).to(dev) for n in ("q", "k", "v", "z", "g", "beta")}
    y = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_size(kda.KDA_BF16, H, dk, dv, C, 1, T),
                     dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], z=d["z"], chunk=C, y=y,
                      final_state=fs, workspace=ws)

    ms, wall, calls = time_steps(step, args.steps, args.warmup, torch, per_call=True)
    calls = sorted(calls)
    log(f"headline: {ms:.4f} ms per step ({args.steps} steps, wall {wall:.3f} s; "
        f"median {calls[len(calls) // 2]:.4f}, min {calls[0]:.4f})")
    nbytes = prefill_bytes(T, H, dk, dv, 2, True, 1, False, True)
    flops = prefill_flops(T, H, dk, dv, C)
    res = dict(ms=ms, ms_median=calls[len(calls) // 2], ms_min=calls[0], tokens_per_s=T / (ms * 1e-3),
               bytes=nbytes, flops=flops, gbs=nbytes / (ms * 1e-3) / 1e9,
               tflops=flops / (ms * 1e-3) / 1e12)
    return inp, res, (y, fs)


def bench_cpu_baseline(args, inp, gpu_out, torch):
    import numpy as np
    import oracle
    H, T = inp.H, inp.T
    nh = max(1, min(H, args.cpu_sample_heads))
    heads = list(range(0, H, max(1, H // nh)))[:nh]
    threads = oracle.default_threads()
    log(f"cpu baseline: fp64 oracle on {len(heads)} of {H} heads, T={T}, {threads} threads")
    # repeat the sample until about args.cpu_seconds of wall time have passed
    reps, t0 = 0, time.perf_counter()
    while True:
        yo, so = oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                                   chains=[(0, h) for h in heads], nthreads=threads)
        reps += 1
        total = time.perf_counter() - t0
        if total >= args.cpu_seconds or total / reps * (reps + 1) > 3 * args.cpu_seconds:
            break
    wall = total / reps
    log(f"cpu baseline: {reps} runs, {wall:.2f} s each")
    t1 = time.perf_counter()
    oracle.recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.cu_seqlens, z=inp.z,
                      chains=[(0, heads[0])], nthreads=1)
    one = time.perf_counter() - t1
    y, fs = gpu_out
    yg = y.cpu().double().numpy()[:, heads]
    sg = fs.cpu().double().numpy()[0, heads]
    ey = oracle.rel_l2(yg, yo[:, heads])
    es = oracle.rel_l2(sg, so)
    cpu = {"value": T / (wall * H / len(heads)), "unit": "tokens/s", "cores": threads,
           "kind": "oracle", "chains_per_s": len(heads) / wall,
           "single_thread_tokens_per_s": T / (one * H),
           "sample": (f"{len(heads)} of {H} heads of k3_layer_prefill (T={T}, full chains), fp64 "
                      f"sequential recurrence in C, run {reps} times ({total:.1f} s wall, "
                      f"{wall:.2f} s per run); value scaled to all {H} heads")}
    parity = {"heads": len(heads), "rel_l2_y": ey, "rel_l2_state": es, "tolerance": 2e-2}
    return cpu, parity


def bench_cpu_kcp(args):
    """The oracle's KCP-structured form (segment pairs, composition, outputs;
    OpenMP over segments and heads) on a bounded slice of the 1M-token KCP
    workload: its first 16 segments of 4096 tokens (the workload's segment
    length), all 4 heads."""
    import oracle
    import kda_inputs
    nseg, seg = 16, 4096
    inp = kda_inputs.make_workload(3, lens=[nseg * seg])
    threads = oracle.default_threads()
    bounds = [i * seg for i in range(nseg + 1)]
    t0 = time.perf_counter()
    oracle.kcp(inp.q, inp.k, inp.v, inp.g, inp.beta, bounds, z=inp.z, nthreads=threads)
    wall = time.perf_counter() - t0
    log(f"cpu kcp: {nseg} segments x {seg} tokens, H={inp.H}: {wall:.2f} s on {threads} threads")
    return {"value": nseg * seg / wall, "unit": "tokens/s", "cores": threads,
            "kind": "oracle, KCP-structured",
            "sample": (f"first {nseg} of the 256 segments ({seg} tokens each) of kcp_long_sequence, "
                       f"all {inp.H} heads, fp64, one run ({wall:.2f} s wall)")}


def bench_varlen(args, torch, kda, kda_inputs, dev):
    w = kda_inputs.WORKLOADS[2]
    lens = kda_inputs.varlen_lengths()
    H, dk, dv = w["H"], w["dk"], w["dv"]
    log(f"varlen_prefill: {len(lens)} sequences, {sum(lens)} tokens")
    d = gpu_inputs(torch, lens, H, dk, dv, True, w["s0_std"], kda_inputs.workload_seed(2), dev)
    T = sum(lens)
    y = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(len(lens), H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_size(kda.KDA_BF16, H, dk, dv, w["chunk"], len(lens), T),
                     dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_seqlens=d["cu"], z=d["z"],
                      initial_state=d["s0"], chunk=w["chunk"], y=y, final_state=fs, workspace=ws)

    ms, _ = time_steps(step, max(1, args.steps // 4), args.warmup, torch)
    nbytes = prefill_bytes(T, H, dk, dv, 2, True, len(lens), True, True)
    out = dict(ms=ms, tokens=T, tokens_per_s=T / (ms * 1e-3),
               gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               tflops=prefill_flops(T, H, dk, dv, w["chunk"]) / (ms * 1e-3) / 1e12)
    del d, y, fs, ws
    torch.cuda.empty_cache()
    return out


def bench_kcp(args, torch, kda, kda_inputs, dev):
    w = kda_inputs.WORKLOADS[3]
    H, dk, dv, T, S = w["H"], w["dk"], w["dv"], w["lens"][0], w["segments"]
    log(f"kcp_long_sequence: T={T} H={H} segments={S}")
    d = gpu_inputs(torch, [T], H, dk, dv, False, 0.0, kda_inputs.workload_seed(3), dev)
    ws = torch.empty(kda.kcp_workspace_size(kda.KDA_BF16, H, dk, dv, w["chunk"], T, S),
                     dtype=torch.uint8, device=dev)
    y = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)

    def step():
        kda.kcp_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], S, chunk=w["chunk"],
                     workspace=ws, y=y, final_state=fs)

    ms, _ = time_steps(step, max(1, args.steps // 4), args.warmup, torch)
    nbytes = prefill_bytes(T, H, dk, dv, 2, False, 1, False, True)
    out = dict(ms=ms, tokens_per_s=T / (ms * 1e-3), segments=S,
               gbs_single_pass=nbytes / (ms * 1e-3) / 1e9,
               hbm_frac_single_pass=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del d, ws, y, fs
    torch.cuda.empty_cache()
    return out


def bench_decode(args, torch, kda, kda_inputs, dev):
    w = kda_inputs.WORKLOADS[4]
    N, H, dk, dv, P = w["N"], w["H"], w["dk"], w["dv"], w["pool"]
    steps = args.decode_steps
    log(f"decode: N={N} H={H} pool={P} steps={steps}")
    gen = torch.Generator(device=dev).manual_seed(kda_inputs.workload_seed(4))

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    state = torch.randn(N, H, dk, dv, generator=gen, device=dev) * w["s0_std"]
    pool = []
    for _ in range(P):
        pool.append(dict(
            q=unit(torch.randn(N, H, dk, generator=gen, device=dev)).to(torch.bfloat16),
            k=unit(torch.randn(N, H, dk, generator=gen, device=dev)).to(torch.bfloat16),
            v=torch.randn(N, H, dv, generator=gen, device=dev).to(torch.bfloat16),
            z=torch.randn(N, H, dv, generator=gen, device=dev).to(torch.bfloat16),
            beta=torch.sigmoid(torch.randn(N, H, generator=gen, device=dev)),
            g=-5.0 * torch.sigmoid(torch.randn(N, H, dk, generator=gen, device=dev))))
    y = torch.empty(N, H, dv, dtype=torch.bfloat16, device=dev)

    def run_all(n=steps):
        for s in range(n):
            p = pool[s % P]
            kda.decode_step(p["q"], p["k"], p["v"], p["g"], p["beta"], state, z=p["z"], y=y)

    run_all(args.warmup)
    ms_all, _ = time_steps(run_all, 1, 0, torch)
    ms = ms_all / steps
    nbytes = decode_bytes(N, H, dk, dv, 2, True)
    out = dict(ms_per_step=ms, steps=steps, tokens_per_s=N / (ms * 1e-3),
               bytes_per_step=nbytes, gbs=nbytes / (ms * 1e-3) / 1e9,
               hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               traffic_per_step=counter_traffic("decode"))
    del state, pool, y
    torch.cuda.empty_cache()
    return out


def bench_checkpoints(args, torch, kda, kda_inputs, dev):
    """The K3 layer prefill saving the state every 512 tokens (the pages' prefix
    hash granularity): 16 extra fp32 states per head."""
    w = kda_inputs.WORKLOADS[1]
    H, dk, dv, T, C = w["H"], w["dk"], w["dv"], w["lens"][0], w["chunk"]
    interval = 512
    d = gpu_inputs(torch, [T], H, dk, dv, True, 0.0, kda_inputs.workload_seed(1), dev)
    ms, _ = time_steps(lambda: kda.chunk_fwd_checkpointed(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                                          interval, z=d["z"], chunk=C),
                       max(1, args.steps // 2), args.warmup, torch)
    nbytes = prefill_bytes(T, H, dk, dv, 2, True, 1, False, True) + (T // interval) * H * dk * dv * 4
    out = dict(ms=ms, tokens_per_s=T / (ms * 1e-3), interval=interval, checkpoints=T // interval,
               gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del d
    torch.cuda.empty_cache()
    return out


def bench_replay(args, torch, kda, kda_inputs, dev):
    """Speculative decoding at the decode workload's shape: 4 draft tokens per
    request, a verify pass (outputs of all drafts, state read only) and a commit
    pass (state after each request's accepted prefix written back)."""
    w = kda_inputs.WORKLOADS[4]
    N, H, dk, dv, Td = w["N"], w["H"], w["dk"], w["dv"], 4
    gen = torch.Generator(device=dev).manual_seed(kda_inputs.workload_seed(4) + 100)

    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)

    state = torch.randn(N, H, dk, dv, generator=gen, device=dev) * w["s0_std"]
    x = dict(q=unit(torch.randn(N, Td, H, dk, generator=gen, device=dev)).to(torch.bfloat16),
             k=unit(torch.randn(N, Td, H, dk, generator=gen, device=dev)).to(torch.bfloat16),
             v=torch.randn(N, Td, H, dv, generator=gen, device=dev).to(torch.bfloat16),
             z=torch.randn(N, Td, H, dv, generator=gen, device=dev).to(torch.bfloat16),
             beta=torch.sigmoid(torch.randn(N, Td, H, generator=gen, device=dev)),
             g=-5.0 * torch.sigmoid(torch.randn(N, Td, H, dk, generator=gen, device=dev)))
    acc = torch.randint(0, Td + 1, (N,), generator=gen, device=dev).to(torch.int32)
    y = torch.empty(N, Td, H, dv, dtype=torch.bfloat16, device=dev)
    ms_v, _ = time_steps(lambda: kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state,
                                                   z=x["z"], y=y), 20, args.warmup, torch)
    ms_c, _ = time_steps(lambda: kda.decode_replay(x["q"], x["k"], x["v"], x["g"], x["beta"], state,
                                                   accepted=acc, z=x["z"], want_y=False), 20, args.warmup, torch)
    st = H * dk * dv * 4                              # one request's states
    tok = H * (2 * dk * 2 + dv * 2 * 2 + dk * 4 + 4)   # one draft token's inputs
    a = [int(t) for t in acc.cpu().tolist()]
    verify_bytes = N * st + N * Td * tok + N * Td * H * dv * 2
    # a request that accepts nothing is skipped; the others read and write their states
    commit_bytes = sum(2 * st + an * tok for an in a if an > 0)
    out = dict(draft_tokens=Td, verify_ms=ms_v, commit_ms=ms_c,
               verify_gbs=verify_bytes / (ms_v * 1e-3) / 1e9,
               commit_gbs=commit_bytes / (ms_c * 1e-3) / 1e9,
               accepted_mean=sum(a) / N,
               draft_tokens_per_s=N * Td / (ms_v * 1e-3))
    del state, x, y
    torch.cuda.empty_cache()
    return out


def bench_prefill_bounded(args, torch, kda, kda_inputs, dev):
    """The K3 layer prefill in a 256 MiB workspace instead of its one-pass
    894 MB: time slabs with the state carried between them (the same results
    bit for bit); the workspace no longer grows with T."""
    w = kda_inputs.WORKLOADS[1]
    H, dk, dv, T, C = w["H"], w["dk"], w["dv"], w["lens"][0], w["chunk"]
    limit = 256 << 20
    d = gpu_inputs(torch, [T], H, dk, dv, True, 0.0, kda_inputs.workload_seed(1), dev)
    y = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(limit, dtype=torch.uint8, device=dev)
    ms, _ = time_steps(lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], z=d["z"], chunk=C,
                                             y=y, final_state=fs, workspace=ws), args.steps, args.warmup, torch)
    nbytes = prefill_bytes(T, H, dk, dv, 2, True, 1, False, True)
    full = kda.chunk_fwd_workspace_size(kda.KDA_BF16, H, dk, dv, C, 1, T)
    out = dict(ms=ms, workspace_bytes=limit, one_pass_workspace_bytes=full,
               min_workspace_bytes=kda.chunk_fwd_workspace_min(kda.KDA_BF16, H, dk, dv, C, 1, T),
               tokens_per_s=T / (ms * 1e-3), gbs=nbytes / (ms * 1e-3) / 1e9,
               hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del d, y, fs, ws
    torch.cuda.empty_cache()
    return out


def bench_kcp_bounded(args, torch, kda, kda_inputs, dev):
    """The 1M-token KCP scan in a 512 MiB workspace instead of its one-pass
    size (~4.3 GB): the chunk products in slabs, formed twice."""
    w = kda_inputs.WORKLOADS[3]
    H, dk, dv, T, S = w["H"], w["dk"], w["dv"], w["lens"][0], w["segments"]
    limit = 512 << 20
    d = gpu_inputs(torch, [T], H, dk, dv, False, 0.0, kda_inputs.workload_seed(3), dev)
    ws = torch.empty(limit, dtype=torch.uint8, device=dev)
    y = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    ms, _ = time_steps(lambda: kda.kcp_scan(d["q"], d["k"], d["v"], d["g"], d["beta"], S, chunk=w["chunk"],
                                            workspace=ws, y=y, final_state=fs),
                       max(1, args.steps // 4), args.warmup, torch)
    out = dict(ms=ms, tokens_per_s=T / (ms * 1e-3), segments=S, workspace_bytes=limit,
               one_pass_workspace_bytes=kda.kcp_workspace_size(kda.KDA_BF16, H, dk, dv, w["chunk"], T, S),
               min_workspace_bytes=kda.kcp_workspace_min(kda.KDA_BF16, H, dk, dv, w["chunk"], T, S))
    del d, ws, y, fs
    torch.cuda.empty_cache()
    return out


def bench_prefill_chunk32(args, torch, kda, kda_inputs, dev):
    """The K3 layer prefill with 32-token chunks (the headline fixes 64): the
    same result up to rounding, a smaller per-chunk triangular block."""
    w = kda_inputs.WORKLOADS[1]
    H, dk, dv, T = w["H"], w["dk"], w["dv"], w["lens"][0]
    C = 32
    d = gpu_inputs(torch, [T], H, dk, dv, True, 0.0, kda_inputs.workload_seed(1), dev)
    y = torch.empty(T, H, dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_size(kda.KDA_BF16, H, dk, dv, C, 1, T), dtype=torch.uint8,
                     device=dev)
    ms, _ = time_steps(lambda: kda.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], z=d["z"], chunk=C,
                                             y=y, final_state=fs, workspace=ws), args.steps, args.warmup, torch)
    nbytes = prefill_bytes(T, H, dk, dv, 2, True, 1, False, True)
    out = dict(ms=ms, chunk=C, tokens_per_s=T / (ms * 1e-3), gbs=nbytes / (ms * 1e-3) / 1e9,
               hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del d, y, fs, ws
    torch.cuda.empty_cache()
    return out


def bench_prefill_fused(args, torch, kda, kda_inputs, dev):
    """The K3 layer prefill from raw inputs (kda_chunk_fwd_fused): unnormalised
    q, k and the gate pre-activations a, b in bf16; the kernel forms unit q, k,
    g = -5 sigmoid(a) and beta = sigmoid(b)."""
    w = kda_inputs.WORKLOADS[1]
    H, dk, dv, T, C = w["H"], w["dk"], w["dv"], w["lens"][0], w["chunk"]
    gen = torch.Generator(device=dev).manual_seed(kda_inputs.workload_seed(1))
    bf = torch.bfloat16
    d = dict(q=torch.randn(T, H, dk, generator=gen, device=dev).to(bf),
             k=torch.randn(T, H, dk, generator=gen, device=dev).to(bf),
             v=torch.randn(T, H, dv, generator=gen, device=dev).to(bf),
             z=torch.randn(T, H, dv, generator=gen, device=dev).to(bf),
             b=torch.randn(T, H, generator=gen, device=dev).to(bf),
             a=torch.randn(T, H, dk, generator=gen, device=dev).to(bf))
    y = torch.empty(T, H, dv, dtype=bf, device=dev)
    fs = torch.empty(1, H, dk, dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_size(kda.KDA_BF16, H, dk, dv, C, 1, T),
                     dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_fwd_fused(d["q"], d["k"], d["v"], d["a"], d["b"], z=d["z"], chunk=C, y=y,
                            final_state=fs, workspace=ws)

    ms, _ = time_steps(step, args.steps, args.warmup, torch)
    nbytes = prefill_bytes(T, H, dk, dv, 2, True, 1, False, True, gate_elt=2)
    out = dict(ms=ms, tokens_per_s=T / (ms * 1e-3), bytes=nbytes,
               gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
               tflops=prefill_flops(T, H, dk, dv, C) / (ms * 1e-3) / 1e12)
    del d, y, fs, ws
    torch.cuda.empty_cache()
    return out


def bench_decode_fused(args, torch, kda, kda_inputs, dev):
    """The decode workload from raw inputs (kda_decode_step_fused)."""
    w = kda_inputs.WORKLOADS[4]
    N, H, dk, dv, P = w["N"], w["H"], w["dk"], w["dv"], w["pool"]
    steps = args.decode_steps
    gen = torch.Generator(device=dev).manual_seed(kda_inputs.workload_seed(4))
    bf = torch.bfloat16
    state = torch.randn(N, H, dk, dv, generator=gen, device=dev) * w["s0_std"]
    pool = [dict(q=torch.randn(N, H, dk, generator=gen, device=dev).to(bf),
                 k=torch.randn(N, H, dk, generator=gen, device=dev).to(bf),
                 v=torch.randn(N, H, dv, generator=gen, device=dev).to(bf),
                 z=torch.randn(N, H, dv, generator=gen, device=dev).to(bf),
                 b=torch.randn(N, H, generator=gen, device=dev).to(bf),
                 a=torch.randn(N, H, dk, generator=gen, device=dev).to(bf)) for _ in range(P)]
    y = torch.empty(N, H, dv, dtype=bf, device=dev)

    def run_all(n=steps):
        for s in range(n):
            p = pool[s % P]
            kda.decode_step_fused(p["q"], p["k"], p["v"], p["a"], p["b"], state, z=p["z"], y=y)

    run_all(args.warmup)
    ms_all, _ = time_steps(run_all, 1, 0, torch)
    ms = ms_all / steps
    nbytes = decode_bytes(N, H, dk, dv, 2, True, gate_elt=2)
    out = dict(ms_per_step=ms, steps=steps, tokens_per_s=N / (ms * 1e-3), bytes_per_step=nbytes,
               gbs=nbytes / (ms * 1e-3) / 1e9, hbm_frac=nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS)
    del state, pool, y
    torch.cuda.empty_cache()
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workloads", default="all",
                    help="comma list of extra workloads (%s), 'all' or 'none'" % ",".join(ALL_WORKLOADS))
    ap.add_argument("--cpu-sample-heads", type=int, default=96)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-measured-peaks", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall time over which the CPU oracle sample is repeated")
    ap.add_argument("--decode-steps", type=int, default=1000,
                    help="decode steps timed as one loop (the workload runs 1000)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the KDA path here has no multi-GPU leg "
              "(heads and requests shard with no exchange; see the design notes).",
              file=sys.stderr)
        return 2
    import torch
    import gated_delta_rule_75_amd as kda
    import kda_inputs
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    kda.lib()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        ms, _ = time_steps(lambda: dst.copy_(src), 5, 1, torch)
        print(json.dumps({"calibrate_copy_bytes": n, "ms": ms, "gbs": 2 * n / (ms * 1e-3) / 1e9}))
        return 0

    peaks = measured_peaks(torch, dev) if not args.no_measured_peaks else None
    if peaks:
        log(f"measured peaks: {json.dumps(peaks)}")
    inp, head, gpu_out = bench_headline(args, torch, kda, kda_inputs, dev)
    extras = ALL_WORKLOADS if args.workloads == "all" else tuple(
        x for x in args.workloads.split(",") if x and x != "none")
    workloads = {}
    for name in extras:
        fn = {"varlen_prefill": bench_varlen, "kcp_long_sequence": bench_kcp,
              "decode": bench_decode, "prefill_checkpoints": bench_checkpoints,
              "decode_replay": bench_replay, "prefill_fused_gates": bench_prefill_fused,
              "decode_fused_gates": bench_decode_fused, "prefill_chunk32": bench_prefill_chunk32,
              "prefill_bounded_workspace": bench_prefill_bounded,
              "kcp_bounded_workspace": bench_kcp_bounded}[name]
        workloads[name] = fn(args, torch, kda, kda_inputs, dev)
        log(f"{name}: {json.dumps(workloads[name])}")
    cpu, parity = (None, None)
    if not args.no_cpu_baseline:
        cpu, parity = bench_cpu_baseline(args, inp, gpu_out, torch)
        if "kcp_long_sequence" in workloads:
            workloads["kcp_long_sequence"]["cpu_baseline"] = bench_cpu_kcp(args)

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_policy": WARMUP_POLICY,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "k3_layer_prefill", "B": 1, "H": 96, "T": 8192, "dk": 128,
                   "dv": 128, "chunk": 64, "gated": True, "state": "fp32"},
        "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": head["gbs"] / HBM_PEAK_GBS,
                     "traffic": counter_traffic("prefill"),
                     "kernel": ("kda_chunk_fwd = chunk_prep_kernel + chunk_state_kernel "
                                "(bf16, dk=dv=128, chunk 64); time of the whole call"),
                     "bytes_per_launch": head["bytes"],
                     "frac_of_measured": head["gbs"] / peaks["hbm_stream_gbs"] if peaks else None},
        "mfma": {"achieved": head["tflops"], "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": head["tflops"] / BF16_MFMA_PEAK_TFLOPS,
                 "flops_per_launch": head["flops"],
                 "frac_of_measured": head["tflops"] / peaks["bf16_gemm_tflops"] if peaks else None},
        "attainable_frac": max(head["gbs"] / HBM_PEAK_GBS, head["tflops"] / BF16_MFMA_PEAK_TFLOPS),
        "ms_median": head["ms_median"],
        "ms_min": head["ms_min"],
        "measured_peaks": peaks,
        "device": device_info(torch, dev),
        "cpu_baseline": cpu,
        "parity_sample": parity,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
