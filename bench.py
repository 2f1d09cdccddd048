#!/usr/bin/env python3
"""Benchmark of the packed varlen KDA forward on one MI355X.

A step is one pass of the whole path over one synthetic packed batch:
segment_ids -> cu_seqlens (pkv_segment_ids_to_cu_seqlens), the masked short
conv when the workload has one, and chunk_kda_varlen. Inputs are resident in
HBM before the timed region. Prints ONE JSON line on stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Modes used for profiling (no JSON line): --mode kernel (only chunk_kda_varlen,
for rocprofv3 counters) and --mode copy (a plain device copy of known size,
the calibration of the HBM byte counters). --mode backward times the reverse
pass (chunk_kda_varlen_backward) on the same workload and prints its own JSON
line (not the headline metric).
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed tokens/sec for chunk_kda_varlen fwd at H=32,D=128; % MFMA/HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
DOMINANT_KERNEL = "chunk_kda_varlen"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="flat_microbatch")
    p.add_argument("--final-state", choices=["auto", "on", "off"], default="auto")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="oracle sample size in tokens (0: sized for ~15 s of CPU work)")
    p.add_argument("--mode", choices=["bench", "kernel", "copy", "backward"], default="bench")
    p.add_argument("--entry", choices=["cu_seqlens", "segment_ids"], default="cu_seqlens",
                   help="segment_ids: the step is one pkv_chunk_kda_segment_ids call on the [B, T] ids "
                        "(no conversion, no phantom slots) instead of the conversion + chunk_kda_varlen")
    return p.parse_args()


def kernel_source_hash():
    """Hash of the sources the dominant kernel is built from (ties a counter
    summary to its code): kda_chunk.hip and the common header."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "packed_varlen_gated_amd", "csrc")
    for f in ("common.h", "kda_chunk.hip"):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(cfg, cu, final_state):
    """Bytes the dominant kernel must move at least once: q, k, g, v, beta read
    and o written for tokens inside segments; o written for uncovered tokens;
    cu_seqlens read; final states written when requested."""
    E = 4 if cfg.dtype == "f32" else 2
    N, H = cfg.B * cfg.T, cfg.H
    covered = int(cu[-1])
    per_tok_head = E * (3 * cfg.Dk + 2 * cfg.Dv + 1)
    total = covered * H * per_tok_head + (N - covered) * H * E * cfg.Dv + 4 * len(cu)
    if final_state:
        total += 4 * (len(cu) - 1) * H * cfg.Dk * cfg.Dv
    return total


def backward_bytes(cfg, cu):
    """Bytes the reverse pass must move at least once: q, k, g, v, beta and do
    read, dq, dk, dg, dv and dbeta written, for every position (uncovered ones
    get zero gradients, written), and cu_seqlens read."""
    E = 4 if cfg.dtype == "f32" else 2
    N, H = cfg.B * cfg.T, cfg.H
    covered = int(cu[-1])
    per_tok_head = E * (6 * cfg.Dk + 3 * cfg.Dv + 2)
    return covered * H * per_tok_head + (N - covered) * H * E * (3 * cfg.Dk + cfg.Dv + 1) + 4 * len(cu)


def algorithmic_flops(cfg, cu):
    """Chunked method (C = 64): 2*Dk*Dv each for Q.S and K^T V, and the causal
    halves of the intra-chunk Q K^T and A V, per token and head."""
    covered = int(cu[-1])
    C = 64
    return covered * cfg.H * (4 * cfg.Dk * cfg.Dv + C * (cfg.Dk + cfg.Dv))


def read_traffic(workload):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"{DOMINANT_KERNEL}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(wl, cu, sample_tokens, target_s=15.0):
    """The oracle, as it stands, on the first S tokens of the workload
    (segments clipped there), all heads, split by head over a process pool.
    S = sample_tokens if given, else sized from a short timed prefix so the
    measured run takes about target_s seconds. Returns a dict for the JSON line."""
    import multiprocessing as mp
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor

    cfg = wl.cfg
    ncores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, ncores, cfg.H))
    groups = np.array_split(np.arange(cfg.H), workers)

    def jobs(S):
        cu_s = np.minimum(cu, S)
        arrs = [t[:S].float().numpy() for t in (wl.q, wl.k, wl.v, wl.g, wl.beta)]  # exact for bf16
        return [tuple(a[:, gidx] for a in arrs) + (cu_s,) for gidx in groups]

    ctx = mp.get_context("spawn")  # workers never touch the GPU
    os.environ["OMP_NUM_THREADS"] = "1"
    with ProcessPoolExecutor(workers, mp_context=ctx) as ex:
        list(ex.map(_warm, range(workers)))  # spawn and import outside the timed runs
        if sample_tokens:
            S = min(sample_tokens, wl.N)
        else:
            S0 = min(512, wl.N)
            rate = S0 / max(ex.map(_oracle_job, jobs(S0)))
            S = int(min(wl.N, max(S0, rate * target_s)) // 64 * 64) or S0
        dt = max(ex.map(_oracle_job, jobs(S)))  # workers run in parallel: the slowest one
    return {"value": S / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"first {S} of {wl.N} tokens ({cfg.name}), all {cfg.H} heads, "
                      f"fp64 token recurrence, {workers} processes split by head, {dt:.1f} s "
                      f"(slowest process, compute only)"}


def _warm(_):
    import oracle  # noqa: F401
    return True


def _oracle_job(args):
    """Runs the oracle on one head group; returns its own run time (the data
    transfer and the fp64 conversion are not timed)."""
    import numpy as np
    import oracle
    q, k, v, g, beta = (a.astype(np.float64) for a in args[:5])
    t0 = time.perf_counter()
    oracle.chunk_kda_varlen(q, k, v, g, beta, args[5])
    return time.perf_counter() - t0


def main():
    args = parse()
    if args.gpus != 1:
        log("bench.py runs on one GPU only: this build has no multi-GPU path "
            "(the sharding design is described in DESIGN.md). Use --gpus 1.")
        sys.exit(2)
    import numpy as np
    import torch
    import workloads
    import packed_varlen_gated_amd as pkv

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)

    if args.mode == "copy":
        nbytes = 1 << 30
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {nbytes} bytes")
        return

    t0 = time.perf_counter()
    wl = workloads.make_workload(args.workload)
    cfg = wl.cfg
    log(f"workload {cfg.name}: {cfg.description}; generated in {time.perf_counter() - t0:.1f} s")
    final_state = cfg.final_state if args.final_state == "auto" else args.final_state == "on"
    N, H = wl.N, cfg.H
    seg = torch.from_numpy(wl.segment_ids).to(dev)
    q = wl.q.reshape(1, N, H, cfg.Dk).to(dev)
    k = wl.k.reshape(1, N, H, cfg.Dk).to(dev)
    v = wl.v.reshape(1, N, H, cfg.Dv).to(dev)
    g = wl.g.reshape(1, N, H, cfg.Dk).to(dev)
    beta = wl.beta.reshape(1, N, H).to(dev)
    conv_x = wl.conv_x.to(dev) if wl.conv_x is not None else None
    conv_w = wl.conv_w.to(dev) if wl.conv_w is not None else None

    # Outputs allocated once, outside the timed region.
    o = torch.empty(1, N, H, cfg.Dv, dtype=q.dtype, device=dev)
    conv_y = torch.empty_like(conv_x) if conv_x is not None else None
    ws_bytes = pkv.chunk_kda_varlen_workspace_size(N, H, cfg.Dk, cfg.Dv, cfg.max_segs, q.dtype)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)

    res = pkv.segment_ids_to_cu_seqlens(seg, cfg.max_segs)
    cu_host = res.cu_seqlens.cpu().numpy()
    n_segs = int(res.n_segs.item())

    if args.mode == "kernel":
        for _ in range(args.warmup + args.steps):
            pkv.chunk_kda_varlen(q, k, v, g, beta, res.cu_seqlens, output_final_state=final_state,
                                 flags=flags, out=o, workspace=ws)
        torch.cuda.synchronize()
        log(f"kernel mode: {args.warmup + args.steps} launches of {DOMINANT_KERNEL}")
        return

    if args.mode == "backward":
        gen = torch.Generator(device=dev).manual_seed(2024)
        do = torch.randn(1, N, H, cfg.Dv, generator=gen, device=dev, dtype=torch.float32).to(q.dtype)
        bws = torch.empty(max(pkv.chunk_kda_varlen_backward_workspace_size(N, H, cfg.Dk, cfg.Dv, cfg.max_segs,
                                                                          q.dtype), 1),
                          dtype=torch.uint8, device=dev)
        cu_dev = res.cu_seqlens
        for _ in range(args.warmup):
            pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, cu_dev, flags=flags, workspace=bws)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        t0 = time.perf_counter()
        for a_ev, b_ev in evs:
            a_ev.record()
            pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, cu_dev, flags=flags, workspace=bws)
            b_ev.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1000.0 / args.steps
        call_s = sum(a.elapsed_time(b) for a, b in evs) / len(evs) / 1000.0
        bb = backward_bytes(cfg, cu_host)
        achieved = bb / call_s / 1e9
        log(f"backward: {call_s * 1e3:.3f} ms per call; {achieved:.0f} GB/s = "
            f"{achieved / HBM_PEAK_GBS:.3f} of HBM peak; flags {int(flags.item())}")
        print(json.dumps({
            "metric": f"packed tokens/sec for chunk_kda_varlen bwd at H={H},D={cfg.Dk}",
            "value": N / call_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
            "config": {"workload": cfg.name, "N": N, "H": H, "Dk": cfg.Dk, "Dv": cfg.Dv,
                       "max_segs": cfg.max_segs, "n_segs": n_segs, "step": "chunk_kda_varlen_backward"},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "chunk_kda_varlen_backward", "kernel_avg_us": call_s * 1e6,
                         "algorithmic_bytes_per_launch": bb},
            "cpu_baseline": None}), flush=True)
        return

    if args.entry == "segment_ids":
        B, T = cfg.B, cfg.T
        qb, kb, gb = (t.view(B, T, H, cfg.Dk) for t in (q, k, g))
        vb, ob, betab = v.view(B, T, H, cfg.Dv), o.view(B, T, H, cfg.Dv), beta.view(B, T, H)
        ws_ids = torch.empty(pkv.chunk_kda_segment_ids_workspace_size(B, T, H, cfg.Dk, cfg.Dv, q.dtype),
                             dtype=torch.uint8, device=dev)

    def step(ev=None):
        if args.entry == "segment_ids":
            if conv_x is not None:
                pkv.short_conv_segmask(conv_x, conv_w, seg, out=conv_y)
            if ev is not None:
                ev[0].record()
            out = pkv.chunk_kda_segment_ids(qb, kb, vb, gb, betab, seg, output_final_state=final_state,
                                            flags=flags, out=ob, workspace=ws_ids)
            if ev is not None:
                ev[1].record()
            return out
        r = pkv.segment_ids_to_cu_seqlens(seg, cfg.max_segs)
        if conv_x is not None:
            pkv.short_conv_segmask(conv_x, conv_w, seg, out=conv_y)
        if ev is not None:
            ev[0].record()
        out = pkv.chunk_kda_varlen(q, k, v, g, beta, r.cu_seqlens, output_final_state=final_state,
                                   flags=flags, out=o, workspace=ws)
        if ev is not None:
            ev[1].record()
        return out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if int(flags.item()) != 0:
        log(f"warning: flags = {int(flags.item())}")
    ms = (t1 - t0) * 1000.0 / args.steps
    kc_ms = [a.elapsed_time(b) for a, b in events]
    kc_avg_s = sum(kc_ms) / len(kc_ms) / 1000.0
    value = N / (ms / 1000.0)

    alg_bytes = algorithmic_bytes(cfg, cu_host, final_state)
    achieved = alg_bytes / kc_avg_s / 1e9
    flops = algorithmic_flops(cfg, cu_host)
    mfma_frac = flops / kc_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS
    traffic = read_traffic(cfg.name) if args.entry == "cu_seqlens" else None
    log(f"step {ms:.3f} ms; {DOMINANT_KERNEL} {kc_avg_s * 1e6:.1f} us avg "
        f"(min {min(kc_ms) * 1e3:.1f} max {max(kc_ms) * 1e3:.1f}); {achieved:.0f} GB/s "
        f"= {achieved / HBM_PEAK_GBS:.3f} of HBM peak; MFMA {mfma_frac:.4f} of bf16 peak; "
        f"n_segs {n_segs}")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle ...")
        cpu = cpu_baseline(wl, cu_host, args.cpu_sample_tokens)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} cores")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "N": N, "H": H, "Dk": cfg.Dk,
                   "Dv": cfg.Dv, "max_segs": cfg.max_segs, "n_segs": n_segs,
                   "output_final_state": final_state, "short_conv": conv_x is not None,
                   "step": ("chunk_kda_segment_ids" if args.entry == "segment_ids" else
                            "segment_ids_to_cu_seqlens" + (" + short_conv_segmask" if conv_x is not None else "")
                            + " + chunk_kda_varlen")},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "kernel": DOMINANT_KERNEL if args.entry == "cu_seqlens" else "chunk_kda_segment_ids",
                     "kernel_avg_us": kc_avg_s * 1e6,
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "mfma_frac_bf16": mfma_frac},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
