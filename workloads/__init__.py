"""Seeded synthetic workloads for the packed varlen KDA path.

This module only draws inputs; it holds none of the method's arithmetic (no
boundary detection, no cu_seqlens, no recurrence, no convolution). Tests and
``bench.py`` hand the same arrays to the HIP library and to the oracle.

The pages measure on Ling3-tiny Megatron-packed pretraining data (8193-token
samples, EOD-separated documents; RFC-0026 Background). That dataset is not
available, so seeded draws with the shapes and document-length mixes below
stand in for it.

Recipe: document lengths come from ``numpy.random.default_rng(seed)``; every
tensor is drawn in fixed blocks of 4096 tokens, block j of tensor i
(q=0, k=1, v=2, g=3, beta=4, conv x=5, conv w=6) from its own
``numpy.random.default_rng([seed, i, j])``, so blocks can be drawn in parallel
and the result does not depend on scheduling. Values are drawn in float64 and
rounded to the workload dtype by torch (round to nearest even). q and k are N(0, 1) normalised to unit L2 norm
over the head dimension per (token, head); v ~ N(0, 1); g = -U(lo, hi) per
key channel; beta = sigmoid(N(0, 1)) per (token, head); conv x ~ N(0, 1),
conv w ~ N(0, 1/Kc) in float32. Rows are filled by appending documents until
the row (minus any trailing padding) is full, truncating the last one; ids
restart at 1 in every row; 0 marks padding.
"""

from dataclasses import dataclass, field
import math
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

# Token block used for the blocked tensor draws (keeps float64 temporaries small).
_BLOCK_TOKENS = 4096


@dataclass(frozen=True)
class Config:
    name: str
    dtype: str            # "f32" or "bf16"
    B: int
    T: int
    lengths: tuple        # ("uniform", lo, hi) | ("lognormal", median, sigma, lo, hi) | ("dirichlet", n)
    max_segs: int
    H: int
    Dk: int
    Dv: int
    g_range: tuple        # g = -U(lo, hi)
    seed: int
    pad: tuple = ()       # ("row_tail", row, count) | ("every_row_tail", count)
    conv: tuple = ()      # (F, Kc) or () for none
    final_state: bool = False
    description: str = ""


CONFIGS = {
    "tiny_f32": Config(
        "tiny_f32", "f32", 2, 256, ("uniform", 16, 96), 16, 2, 32, 32, (0.01, 0.3), 0,
        pad=("row_tail", 1, 20), conv=(64, 4), final_state=True,
        description="tiny packed batch, fp32, B=2 T=256, padding at the end of row 1"),
    "tiny_f32_midpad": Config(
        "tiny_f32_midpad", "f32", 2, 256, ("uniform", 16, 96), 16, 2, 32, 32, (0.01, 0.3), 0,
        pad=("row_tail", 0, 20), conv=(64, 4), final_state=True,
        description="as tiny_f32 with the padding at the end of row 0 (between documents)"),
    "ling3_tiny_sample": Config(
        "ling3_tiny_sample", "bf16", 1, 8192, ("lognormal", 800.0, 1.0, 32, 8192), 128, 16, 128, 128,
        (0.01, 0.3), 1, conv=(3 * 16 * 128, 4), final_state=True,
        description="Ling3-tiny-like single sample, bf16, T=8192, H=16, D=128"),
    "flat_microbatch": Config(
        "flat_microbatch", "bf16", 8, 8192, ("lognormal", 1500.0, 1.0, 32, 8192), 256, 32, 128, 128,
        (0.001, 0.2), 2,
        description="flattened micro-batch, bf16, B=8 x T=8192 -> 65536 tokens, H=32, D=128"),
    "many_short_docs": Config(
        "many_short_docs", "bf16", 4, 8192, ("uniform", 8, 200), 1024, 32, 64, 64, (0.01, 0.3), 3,
        pad=("every_row_tail", 410),
        description="many short documents, bf16, B=4 x T=8192, 5% trailing padding per row, H=32, D=64"),
    "long_context": Config(
        "long_context", "bf16", 1, 131072, ("dirichlet", 6), 8, 32, 128, 128, (0.0005, 0.05), 4,
        final_state=True,
        description="long context, bf16, T=131072, 6 documents, H=32, D=128, final states"),
}


@dataclass
class Doc:
    row: int
    start: int     # position inside the row
    length: int    # real (non-padding) tokens


@dataclass
class Workload:
    cfg: Config
    segment_ids: np.ndarray            # int32 [B, T]
    docs: list                         # [Doc] in flattened order
    q: torch.Tensor = None             # [N, H, Dk] in cfg dtype (CPU)
    k: torch.Tensor = None
    v: torch.Tensor = None             # [N, H, Dv]
    g: torch.Tensor = None             # [N, H, Dk]
    beta: torch.Tensor = None          # [N, H]
    conv_x: torch.Tensor = None        # [B, T, F]
    conv_w: torch.Tensor = None        # [F, Kc] float32
    extra: dict = field(default_factory=dict)

    @property
    def N(self):
        return self.cfg.B * self.cfg.T


def torch_dtype(name):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _draw_lengths(cfg, rng, room):
    kind = cfg.lengths[0]
    if kind == "uniform":
        _, lo, hi = cfg.lengths
        return int(rng.integers(lo, hi + 1))
    if kind == "lognormal":
        _, median, sigma, lo, hi = cfg.lengths
        x = int(round(float(rng.lognormal(math.log(median), sigma))))
        return int(min(max(x, lo), hi))
    raise ValueError(kind)


def _dirichlet_lengths(rng, n, total):
    """n positive lengths summing to total: Dirichlet(1,...,1) shares, largest-remainder rounding."""
    shares = rng.dirichlet(np.ones(n)) * total
    base = np.floor(shares).astype(np.int64)
    rest = total - int(base.sum())
    order = np.argsort(-(shares - base), kind="stable")
    base[order[:rest]] += 1
    # every document keeps at least one token
    for i in range(n):
        if base[i] < 1:
            j = int(np.argmax(base))
            base[j] -= 1
            base[i] += 1
    return [int(x) for x in base]


def make_segments(cfg, rng):
    """Pack documents into rows; return (segment_ids int32 [B, T], docs)."""
    B, T = cfg.B, cfg.T
    seg = np.zeros((B, T), dtype=np.int32)
    docs = []
    fill = [T] * B
    if cfg.pad and cfg.pad[0] == "every_row_tail":
        fill = [T - cfg.pad[1]] * B
    for b in range(B):
        pos = 0
        if cfg.lengths[0] == "dirichlet":
            lens = _dirichlet_lengths(rng, cfg.lengths[1], fill[b])
        else:
            lens = []
            while pos < fill[b]:
                L = min(_draw_lengths(cfg, rng, fill[b] - pos), fill[b] - pos)
                lens.append(L)
                pos += L
            pos = 0
        for L in lens:
            docs.append(Doc(b, pos, L))
            pos += L
    if cfg.pad and cfg.pad[0] == "row_tail":
        _, prow, count = cfg.pad
        cut = T - count
        kept = []
        for d in docs:
            if d.row == prow:
                L = min(d.length, cut - d.start)
                if L <= 0:
                    continue
                d = Doc(d.row, d.start, L)
            kept.append(d)
        docs = kept
    ids = [0] * B
    for d in docs:
        ids[d.row] += 1
        seg[d.row, d.start:d.start + d.length] = ids[d.row]
    n_real = len(docs)
    if n_real > cfg.max_segs:
        raise RuntimeError(f"{cfg.name}: {n_real} documents exceed max_segs={cfg.max_segs} for seed {cfg.seed}")
    return seg, docs


def _blocked(seed, tensor_id, shape, draw, to_dtype, post=None):
    """Draw ``shape`` = [N, ...] in token blocks, block j from rng([seed, tensor_id, j])."""
    N = shape[0]
    out = torch.empty(shape, dtype=to_dtype)
    starts = list(range(0, N, _BLOCK_TOKENS))

    def one(j):
        s = starts[j]
        e = min(N, s + _BLOCK_TOKENS)
        rng = np.random.default_rng([seed, tensor_id, j])
        a = torch.from_numpy(draw(rng, (e - s,) + tuple(shape[1:])))
        if post is not None:
            a = post(a)
        out[s:e] = a.to(to_dtype)

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(workers) as ex:
        list(ex.map(one, range(len(starts))))
    return out


def _unit_rows(a):
    return a / torch.linalg.vector_norm(a, dim=-1, keepdim=True)


def make_workload(name, tensors=True, conv=True):
    """Build the named workload. ``tensors=False`` stops after the segment ids."""
    cfg = CONFIGS[name]
    rng = np.random.default_rng(cfg.seed)
    seg, docs = make_segments(cfg, rng)
    wl = Workload(cfg, seg, docs)
    if not tensors:
        return wl
    N, H = cfg.B * cfg.T, cfg.H
    dt = torch_dtype(cfg.dtype)
    normal = lambda r, s: r.standard_normal(s)
    lo, hi = cfg.g_range
    sd = cfg.seed
    wl.q = _blocked(sd, 0, (N, H, cfg.Dk), normal, dt, _unit_rows)
    wl.k = _blocked(sd, 1, (N, H, cfg.Dk), normal, dt, _unit_rows)
    wl.v = _blocked(sd, 2, (N, H, cfg.Dv), normal, dt)
    wl.g = _blocked(sd, 3, (N, H, cfg.Dk), lambda r, s: -r.uniform(lo, hi, s), dt)
    wl.beta = _blocked(sd, 4, (N, H), normal, dt, torch.sigmoid)
    if conv and cfg.conv:
        F, Kc = cfg.conv
        xs = _blocked(sd, 5, (cfg.B * cfg.T, F), normal, dt)
        wl.conv_x = xs.reshape(cfg.B, cfg.T, F)
        wrng = np.random.default_rng([sd, 6, 0])
        wl.conv_w = torch.from_numpy(wrng.normal(0.0, math.sqrt(1.0 / Kc), (F, Kc))).to(torch.float32)
    return wl


def random_segment_ids(rng, B, T, max_len, pad_prob=0.0, lead_pad=False, mid_pad=False):
    """Small random [B, T] segment ids for fuzzing (documents, optional padding runs)."""
    seg = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        pos = 0
        if lead_pad and rng.random() < 0.5:
            pos = int(rng.integers(1, max(2, T // 4)))
        nid = 0
        while pos < T:
            L = int(rng.integers(1, max_len + 1))
            nid += 1
            seg[b, pos:pos + L] = nid
            pos += L
            if mid_pad and rng.random() < pad_prob:
                pos += int(rng.integers(1, max_len + 1))
        if pad_prob > 0 and rng.random() < pad_prob:
            cut = int(rng.integers(0, T))
            seg[b, cut:] = 0
    return seg
