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
line (not the headline metric); with --bwd-states the reverse pass reads the
per-chunk states a forward call saved (chunk_kda_varlen(..., chunk_states=...))
instead of recomputing them. The default run also reports both, measured after
the headline steps, under "legs" (backward; backward_saved_states, with the
saving forward call beside it).
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
    p.add_argument("--no-legs", dest="legs", action="store_false",
                   help="skip the extra timed legs (final states toggled, q/k L2 norm, device copy)")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="oracle sample size in tokens (0: sized for ~15 s of CPU work)")
    p.add_argument("--mode", choices=["bench", "kernel", "copy", "backward"], default="bench")
    p.add_argument("--bwd-states", action="store_true",
                   help="--mode backward: the reverse pass reads the states a forward call saved")
    p.add_argument("--fwd-states", action="store_true",
                   help="--mode kernel: the forward call also saves the per-chunk states")
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


def cpu_model():
    """The host CPU's model name (lscpu's "Model name"), or None."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, cu, sample_tokens, target_s=15.0):
    """The oracle, as it stands, on the first S tokens of the workload
    (segments clipped there), every (segment, head) unit: the heads are split
    into one group per worker process (one per available core, at most 16,
    the GPU host's CPU share), each worker running the oracle over every
    segment of its heads. The inputs are written once to memory-mapped files
    before the timed run (as the GPU's inputs are resident before its timed
    region); the timed run is the pool's wall time. S = sample_tokens if
    given, else sized from a short timed prefix so the measured run takes
    about target_s seconds (capped at the whole workload). Returns a dict for
    the JSON line."""
    import multiprocessing as mp
    import shutil
    import tempfile
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor

    cfg = wl.cfg
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host_cores, cfg.H))
    groups = [g.tolist() for g in np.array_split(np.arange(cfg.H), workers)]
    tmp = tempfile.mkdtemp(prefix="pkv_oracle_")
    try:
        paths = []
        for name, t in zip(("q", "k", "v", "g", "beta"), (wl.q, wl.k, wl.v, wl.g, wl.beta)):
            path = os.path.join(tmp, name + ".npy")
            np.save(path, t.float().numpy())  # exact for bf16
            paths.append(path)

        def run(ex, S):
            cu_s = np.minimum(cu, S)
            t0 = time.perf_counter()
            list(ex.map(_oracle_job, [(paths, hs, S, cu_s) for hs in groups]))
            return time.perf_counter() - t0

        ctx = mp.get_context("spawn")  # workers never touch the GPU
        os.environ["OMP_NUM_THREADS"] = "1"
        with ProcessPoolExecutor(workers, mp_context=ctx) as ex:
            list(ex.map(_warm, range(workers)))  # spawn and import outside the timed runs
            if sample_tokens:
                S = min(sample_tokens, wl.N)
            else:
                S0 = min(1024, wl.N)
                rate = S0 / run(ex, S0)
                S = int(min(wl.N, max(S0, rate * target_s)) // 64 * 64) or S0
            dt = run(ex, S)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return {"value": S / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "host_cores": host_cores, "cpu_model": cpu_model(),
            "sample": f"first {S} of {wl.N} tokens ({cfg.name}): every (segment, head) unit, "
                      f"fp64 token recurrence, heads split over {workers} processes, {dt:.1f} s wall"}


def _warm(_):
    import oracle  # noqa: F401
    return True


def _oracle_job(args):
    """Runs the oracle on every (segment, head) unit of a group of heads."""
    import numpy as np
    import oracle
    paths, heads, S, cu_s = args
    q, k, v, g, beta = (np.load(p, mmap_mode="r")[:S, heads[0]:heads[-1] + 1].astype(np.float64)
                        for p in paths)
    oracle.chunk_kda_varlen(q, k, v, g, beta, cu_s)
    return True


def pct(xs):
    """Average, median, p10 and p90 of a list of durations."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"avg": float(a.mean()), "median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90))}


def copy_bandwidth(dev, nbytes=1 << 30, reps=10):
    """Measured device-to-device copy rate (bytes read + written per second)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    dt = a.elapsed_time(b) / 1000.0 / reps
    del src, dst
    return 2 * nbytes / dt / 1e9


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
        kst = pkv.new_chunk_states(N, H, cfg.Dk, cfg.Dv, cfg.max_segs, dev) if args.fwd_states else None
        for _ in range(args.warmup + args.steps):
            pkv.chunk_kda_varlen(q, k, v, g, beta, res.cu_seqlens, output_final_state=final_state,
                                 flags=flags, out=o, workspace=ws, chunk_states=kst)
        torch.cuda.synchronize()
        log(f"kernel mode: {args.warmup + args.steps} launches of {DOMINANT_KERNEL}")
        return

    def time_calls(call, warmup, steps):
        """warmup untimed calls, then steps calls: wall ms per call and each
        call's seconds by HIP events on the launch stream."""
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        t0 = time.perf_counter()
        for a_ev, b_ev in evs:
            a_ev.record()
            call()
            b_ev.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return (t1 - t0) * 1000.0 / steps, [a.elapsed_time(b) / 1000.0 for a, b in evs]

    chunk_states = None

    def saving_forward():
        """The forward call that also keeps the state before every chunk."""
        return pkv.chunk_kda_varlen(q, k, v, g, beta, res.cu_seqlens, output_final_state=False, flags=flags,
                                    out=o, workspace=ws, chunk_states=chunk_states)

    def time_backward(warmup, steps, with_states=False):
        """One chunk_kda_varlen_backward call per step (seeded do, no initial
        or final state), recomputing the states or (with_states) reading the ones
        a saving forward call left: wall ms per step and each call's seconds."""
        nonlocal chunk_states
        gen = torch.Generator(device=dev).manual_seed(2024)
        do = torch.randn(1, N, H, cfg.Dv, generator=gen, device=dev, dtype=torch.float32).to(q.dtype)
        size_fn = (pkv.chunk_kda_varlen_backward_states_workspace_size if with_states
                   else pkv.chunk_kda_varlen_backward_workspace_size)
        bws = torch.empty(max(size_fn(N, H, cfg.Dk, cfg.Dv, cfg.max_segs, q.dtype), 1),
                          dtype=torch.uint8, device=dev)
        cu_dev = res.cu_seqlens
        st = None
        if with_states:
            if chunk_states is None:
                chunk_states = pkv.new_chunk_states(N, H, cfg.Dk, cfg.Dv, cfg.max_segs, dev)
            saving_forward()
            st = chunk_states
        call = lambda: pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, cu_dev, flags=flags, workspace=bws,
                                                     chunk_states=st)
        return time_calls(call, warmup, steps)

    def states_read_bytes():
        """bf16 states the reverse pass reads when they are given: one per chunk
        but a segment's first (zero without an initial state)."""
        import numpy as np
        lens = np.diff(cu_host.astype(np.int64))
        chunks = int(np.sum((lens + 63) // 64)) - int(np.sum(lens > 0))
        return chunks * H * cfg.Dk * cfg.Dv * 2

    if args.mode == "backward":
        ms, calls = time_backward(args.warmup, args.steps, args.bwd_states)
        call_s = sum(calls) / len(calls)
        cp = pct(calls)
        # with saved states they are one more input
        bb = backward_bytes(cfg, cu_host) + (states_read_bytes() if args.bwd_states else 0)
        achieved = bb / call_s / 1e9
        log(f"backward: {call_s * 1e3:.3f} ms per call (median {cp['median'] * 1e3:.3f}, p10 "
            f"{cp['p10'] * 1e3:.3f}, p90 {cp['p90'] * 1e3:.3f}); {achieved:.0f} GB/s = "
            f"{achieved / HBM_PEAK_GBS:.3f} of HBM peak; flags {int(flags.item())}")
        print(json.dumps({
            "metric": f"packed tokens/sec for chunk_kda_varlen bwd at H={H},D={cfg.Dk}",
            "value": N / call_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
            "config": {"workload": cfg.name, "N": N, "H": H, "Dk": cfg.Dk, "Dv": cfg.Dv,
                       "max_segs": cfg.max_segs, "n_segs": n_segs,
                       "step": "chunk_kda_varlen_backward" + (" (states saved by the forward call)"
                                                              if args.bwd_states else "")},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "chunk_kda_varlen_backward", "kernel_avg_us": call_s * 1e6,
                         "algorithmic_bytes_per_launch": bb},
            "timing": {"call_us": {k2: x * 1e6 for k2, x in cp.items()}},
            "cpu_baseline": None}), flush=True)
        return

    if args.entry == "segment_ids":
        B, T = cfg.B, cfg.T
        qb, kb, gb = (t.view(B, T, H, cfg.Dk) for t in (q, k, g))
        vb, ob, betab = v.view(B, T, H, cfg.Dv), o.view(B, T, H, cfg.Dv), beta.view(B, T, H)
        ws_ids = torch.empty(pkv.chunk_kda_segment_ids_workspace_size(B, T, H, cfg.Dk, cfg.Dv, q.dtype),
                             dtype=torch.uint8, device=dev)

    def step(ev=None, fstate=None, l2=False):
        """One pass of the path; ev = (step start, call start, call end, step end) events."""
        fst = final_state if fstate is None else fstate
        if ev is not None:
            ev[0].record()
        if args.entry == "segment_ids":
            if conv_x is not None:
                pkv.short_conv_segmask(conv_x, conv_w, seg, out=conv_y)
            if ev is not None:
                ev[1].record()
            out = pkv.chunk_kda_segment_ids(qb, kb, vb, gb, betab, seg, output_final_state=fst,
                                            flags=flags, out=ob, workspace=ws_ids, use_qk_l2norm_in_kernel=l2)
        else:
            r = pkv.segment_ids_to_cu_seqlens(seg, cfg.max_segs)
            if conv_x is not None:
                pkv.short_conv_segmask(conv_x, conv_w, seg, out=conv_y)
            if ev is not None:
                ev[1].record()
            out = pkv.chunk_kda_varlen(q, k, v, g, beta, r.cu_seqlens, output_final_state=fst,
                                       flags=flags, out=o, workspace=ws, use_qk_l2norm_in_kernel=l2)
        if ev is not None:
            ev[2].record()
            ev[3].record()
        return out

    def timed(nsteps, **kw):
        """nsteps steps bracketed by synchronisations: (wall ms per step, call
        durations in s, step durations in s) from HIP events on the launch stream."""
        evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(nsteps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(nsteps):
            step(evs[i], **kw)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        calls = [e[1].elapsed_time(e[2]) / 1000.0 for e in evs]
        steps = [e[0].elapsed_time(e[3]) / 1000.0 for e in evs]
        return (t1 - t0) * 1000.0 / nsteps, calls, steps

    # Extra legs, measured before the headline steps and not part of `value`:
    # a plain 1 GiB device copy (the measured bandwidth beside the published
    # peak), then the same workload with the final states toggled and with q, k
    # normalised inside the call (each after its own W warm-up steps). They run
    # first, the copy first of all, so the headline steps follow compute-bound
    # calls and find the GPU at the clocks of sustained work (clocks rise over
    # the first ~15 ms of work, and a memory-bound copy lets them drop). The
    # reverse pass on the same inputs is timed after the headline steps, so its
    # heavier load cannot change their clocks.
    legs = {}
    if args.legs:
        legs["copy_gbs"] = copy_bandwidth(dev)
        for name, kw, with_fs in (("output_final_state_" + ("off" if final_state else "on"),
                                   {"fstate": not final_state}, not final_state),
                                  ("qk_l2norm", {"l2": True}, final_state)):
            for _ in range(args.warmup):
                step(**kw)
            lm, lk, ls = timed(args.steps, **kw)
            b = algorithmic_bytes(cfg, cu_host, with_fs)
            lp = pct(lk)
            legs[name] = {"call_us": {k2: x * 1e6 for k2, x in lp.items()}, "ms_per_step": lm,
                          "tokens_per_s": N / (lm / 1000.0), "algorithmic_bytes": b,
                          "hbm_frac": b / lp["avg"] / 1e9 / HBM_PEAK_GBS}
            log(f"leg {name}: call {lp['avg'] * 1e6:.1f} us avg (median {lp['median'] * 1e6:.1f}); "
                f"{b / lp['avg'] / 1e9 / HBM_PEAK_GBS:.3f} of HBM peak")
        log(f"device copy of 1 GiB: {legs['copy_gbs']:.0f} GB/s (read + written) against the "
            f"{HBM_PEAK_GBS:.0f} GB/s published peak")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms, kc, st = timed(args.steps)
    if int(flags.item()) != 0:
        log(f"warning: flags = {int(flags.item())}")
    kc_avg_s = sum(kc) / len(kc)
    value = N / (ms / 1000.0)

    alg_bytes = algorithmic_bytes(cfg, cu_host, final_state)
    achieved = alg_bytes / kc_avg_s / 1e9
    flops = algorithmic_flops(cfg, cu_host)
    mfma_frac = flops / kc_avg_s / 1e12 / MFMA_BF16_PEAK_TFLOPS
    traffic = read_traffic(cfg.name) if args.entry == "cu_seqlens" else None
    kp, sp = pct(kc), pct(st)
    log(f"step {ms:.3f} ms (events: median {sp['median'] * 1e3:.3f}, p10 {sp['p10'] * 1e3:.3f}, "
        f"p90 {sp['p90'] * 1e3:.3f}); {DOMINANT_KERNEL} {kc_avg_s * 1e6:.1f} us avg, median "
        f"{kp['median'] * 1e6:.1f}, p10 {kp['p10'] * 1e6:.1f}, p90 {kp['p90'] * 1e6:.1f} "
        f"(min {min(kc) * 1e6:.1f} max {max(kc) * 1e6:.1f}); {achieved:.0f} GB/s "
        f"= {achieved / HBM_PEAK_GBS:.3f} of HBM peak; MFMA {mfma_frac:.4f} of bf16 peak; "
        f"n_segs {n_segs}")
    log("calls in order (us): " + " ".join(f"{x * 1e6:.0f}" for x in kc))
    if args.legs:
        # the reverse pass on the same inputs (one chunk_kda_varlen_backward call per step)
        bm, bc = time_backward(args.warmup, args.steps)
        bp = pct(bc)
        bb = backward_bytes(cfg, cu_host)
        legs["backward"] = {"call_us": {k2: x * 1e6 for k2, x in bp.items()}, "ms_per_step": bm,
                            "tokens_per_s": N / bp["avg"], "algorithmic_bytes": bb,
                            "hbm_frac": bb / bp["avg"] / 1e9 / HBM_PEAK_GBS}
        log(f"leg backward: call {bp['avg'] * 1e6:.1f} us avg (median {bp['median'] * 1e6:.1f}); "
            f"{bb / bp['avg'] / 1e9 / HBM_PEAK_GBS:.3f} of HBM peak")
        # the training pair with the states kept by the forward call: that call,
        # then the reverse pass reading them
        if pkv.chunk_kda_states_size(N, H, cfg.Dk, cfg.Dv, cfg.max_segs, q.dtype) > 0:
            sm, sc = time_backward(args.warmup, args.steps, with_states=True)
            fm, fc = time_calls(saving_forward, args.warmup, args.steps)
            spp, fpp = pct(sc), pct(fc)
            sb = bb + states_read_bytes()
            legs["backward_saved_states"] = {
                "call_us": {k2: x * 1e6 for k2, x in spp.items()}, "ms_per_step": sm,
                "tokens_per_s": N / spp["avg"], "algorithmic_bytes": sb,
                "hbm_frac": sb / spp["avg"] / 1e9 / HBM_PEAK_GBS,
                "saving_forward_call_us": {k2: x * 1e6 for k2, x in fpp.items()},
                "pair_us": (spp["avg"] + fpp["avg"]) * 1e6,
                "pair_us_recomputing": (bp["avg"] + kc_avg_s) * 1e6}
            log(f"leg backward_saved_states: call {spp['avg'] * 1e6:.1f} us avg (median "
                f"{spp['median'] * 1e6:.1f}); the saving forward call {fpp['avg'] * 1e6:.1f} us avg; "
                f"forward + reverse {(spp['avg'] + fpp['avg']) * 1e6:.0f} us against "
                f"{(bp['avg'] + kc_avg_s) * 1e6:.0f} us recomputing")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the oracle ...")
        cpu = cpu_baseline(wl, cu_host, args.cpu_sample_tokens)
        log(f"cpu baseline: {cpu['value']:.1f} tokens/s on {cpu['cores']} processes "
            f"({cpu['host_cores']} host cores available, {cpu['cpu_model']})")

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
        "timing": {"call_us": {k2: x * 1e6 for k2, x in kp.items()},
                   "step_ms": {k2: x * 1e3 for k2, x in sp.items()}},
        "legs": legs or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
