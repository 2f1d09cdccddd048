"""Full-size parity: the fp64 oracle over every (segment, head) pair of a
workload, run in a pool of processes on the host's cores, compared with the
GPU's outputs element by element.

The inputs and the GPU's outputs are written once to a temporary directory as
.npy files (bf16 tensors as their raw 16-bit patterns, which the workers widen
exactly to fp32) and memory-mapped by the workers, so nothing large is
pickled. Each job takes one head and every segment; it returns, per
(segment, head) and per compared tensor, the squared error, the squared
reference, the largest absolute error and reference and whether every value
is finite. The caller sums them into per-tensor and per-segment relative L2
errors.

Test infrastructure: only the GPU tests use it.
"""

import multiprocessing as mp
import os
import shutil
import tempfile
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import torch


def workers():
    """Worker processes: the host's cores, at most 16 (the GPU machine's CPU share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


class Store:
    """Arrays written once, memory-mapped read-only by the workers."""

    def __init__(self):
        self.dir = tempfile.mkdtemp(prefix="pkv_fullsize_")
        self.paths = {}

    def put(self, name, t):
        """t: a CPU or GPU torch tensor (bf16 or fp32) or a numpy array."""
        if isinstance(t, torch.Tensor):
            t = t.detach().cpu().contiguous()
            if t.dtype == torch.bfloat16:
                arr, kind = t.view(torch.int16).numpy(), "bf16"
            else:
                arr, kind = t.to(torch.float32).numpy(), "f32"
        else:
            arr, kind = np.ascontiguousarray(t), "np"
        path = os.path.join(self.dir, f"{name}.{kind}.npy")
        np.save(path, arr)
        self.paths[name] = path

    def close(self):
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _load(path):
    return np.load(path, mmap_mode="r")


def _f64(a, path, idx):
    """Rows idx of a stored array as float64 (bf16 bit patterns widened exactly)."""
    x = np.asarray(a[idx])
    if path.endswith(".bf16.npy"):
        x = (x.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return x.astype(np.float64)


def _stats(got, ref):
    d = got - ref
    return (float(np.sum(d * d)), float(np.sum(ref * ref)),
            float(np.max(np.abs(d))) if d.size else 0.0,
            float(np.max(np.abs(ref))) if ref.size else 0.0,
            bool(np.all(np.isfinite(got))))


def _fwd_job(args):
    paths, h, cu, scale = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import oracle
    arr = {n: _load(p) for n, p in paths.items()}
    out = []
    for i in range(len(cu) - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        if e <= a:
            continue
        sl = (slice(a, e), slice(h, h + 1))
        ins = [_f64(arr[n], paths[n], sl) for n in ("q", "k", "v", "g")]
        beta = _f64(arr["beta"], paths["beta"], sl)
        s0 = None
        if "s0" in paths:
            s0 = _f64(arr["s0"], paths["s0"], (slice(i, i + 1), slice(h, h + 1)))
        ro, rfs = oracle.chunk_kda_varlen(*ins, beta, None, scale, s0)
        rec = {"o": _stats(_f64(arr["o"], paths["o"], sl)[:, 0], ro[:, 0])}
        if "fs" in paths:
            rec["fs"] = _stats(_f64(arr["fs"], paths["fs"], (i, h)), rfs[0, 0])
        out.append((i, h, rec))
    return out


def _bwd_job(args):
    paths, h, cu, scale = args
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import oracle
    arr = {n: _load(p) for n, p in paths.items()}
    out = []
    for i in range(len(cu) - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        if e <= a:
            continue
        sl = (slice(a, e), slice(h, h + 1))
        ins = [_f64(arr[n], paths[n], sl) for n in ("q", "k", "v", "g", "beta", "do")]
        dF = _f64(arr["dF"], paths["dF"], (slice(i, i + 1), slice(h, h + 1))) if "dF" in paths else None
        ref = oracle.chunk_kda_varlen_backward(*ins, None, scale, None, dF)
        rec = {}
        for n, r in zip(("dq", "dk", "dv", "dg", "dbeta"), ref[:5]):
            rec[n] = _stats(_f64(arr[n], paths[n], sl)[:, 0], r[:, 0])
        if "dS0" in paths:
            rec["dS0"] = _stats(_f64(arr["dS0"], paths["dS0"], (i, h)), ref[5][0, 0])
        out.append((i, h, rec))
    return out


def run_pairs(job, paths, H, cu, scale=1.0, heads=None, nproc=None):
    """Runs job over heads (default: all H) on a spawned process pool; returns
    the list of (segment, head, {tensor: stats}) records."""
    heads = list(range(H)) if heads is None else list(heads)
    ctx = mp.get_context("spawn")  # the workers never touch the GPU
    recs = []
    with ProcessPoolExecutor(nproc or workers(), mp_context=ctx) as ex:
        for r in ex.map(job, [(paths, h, np.asarray(cu), scale) for h in heads]):
            recs.extend(r)
    return recs


def summarize(recs):
    """Per tensor: global rel-L2, max abs error, max |ref|, the worst
    per-segment rel-L2 (over all heads of the segment) and all-finite."""
    tensors = sorted({n for _, _, rec in recs for n in rec})
    out = {}
    for n in tensors:
        se = sr = 0.0
        me = mr = 0.0
        fin = True
        seg = {}
        for i, _, rec in recs:
            if n not in rec:
                continue
            a, b, c, d, f = rec[n]
            se += a; sr += b
            me = max(me, c); mr = max(mr, d)
            fin = fin and f
            s = seg.setdefault(i, [0.0, 0.0])
            s[0] += a; s[1] += b
        worst = max((np.sqrt(a / b) if b > 0 else (0.0 if a == 0 else np.inf)) for a, b in seg.values())
        out[n] = {"rel_l2": float(np.sqrt(se / sr)) if sr > 0 else (0.0 if se == 0 else float("inf")),
                  "max_abs": me, "max_ref": mr, "worst_segment_rel_l2": float(worst), "finite": fin,
                  "pairs": sum(1 for _, _, rec in recs if n in rec)}
    return out
