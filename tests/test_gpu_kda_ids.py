"""GPU parity of pkv_chunk_kda_segment_ids (RFC-0026 section 3.1.1's [B, T]
contract, with section 3.4's padding id 0 ignored) against the oracle, and
against the cu_seqlens entry on the same documents."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from parity import check_close, device, f64

pytestmark = pytest.mark.gpu


def _pkv():
    import packed_varlen_gated_amd as pkv
    return pkv


def _inputs(rng, B, T, H, Dk, Dv, dtype, gl=0.01, gh=0.3):
    q = rng.standard_normal((B, T, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, Dv))
    g = -rng.uniform(gl, gh, (B, T, H, Dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    return [torch.from_numpy(a).to(dtype) for a in (q, k, v, g, beta)]


def _ids(rng, B, T):
    """Documents of varied length, padding runs (id 0), single-token segments,
    and equal ids across a row boundary (still two segments)."""
    seg = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        t, d = 0, 1 if b % 2 else 2
        while t < T:
            n = int(rng.choice([1, 1, 5, 63, 64, 65, 130, 300]))
            seg[b, t:t + n] = d if rng.random() > 0.15 else 0
            t += n
            d += 1
    seg[1, 0] = seg[0, -1]
    return seg


def _run(ts, seg, S0=None, scale=1.0):
    pkv = _pkv()
    q, k, v, g, beta = [t.to(device()) for t in ts]
    s0 = None if S0 is None else torch.from_numpy(S0).float().to(device())
    o, fs = pkv.chunk_kda_segment_ids(q, k, v, g, beta, torch.from_numpy(seg).to(device()), scale=scale,
                                      initial_state=s0)
    torch.cuda.synchronize()
    return o, fs


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Dk,Dv", [(32, 32), (64, 64), (128, 128), (64, 128), (128, 64)])
def test_small_shapes(dtype, Dk, Dv):
    rng = np.random.default_rng(Dk + 3 * Dv)
    B, T, H = 3, 700, 2
    ts = _inputs(rng, B, T, H, Dk, Dv, dtype)
    seg = _ids(rng, B, T)
    S0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    print(f"ids dtype {dtype} Dk {Dk} Dv {Dv}", flush=True)
    o, fs = _run(ts, seg, S0, scale=0.9)
    ro, rfs = oracle.chunk_kda_segment_ids(*[f64(t) for t in ts], seg, scale=0.9, initial_state=S0)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o), ro, dt, "o")
    check_close(f64(fs), rfs, dt, "final states")


def test_long_row_cut_into_runs_with_initial_state():
    """A 12000-token row with two segments: the long one (172 chunks) is cut
    into 3 runs and folds the row's initial state in through the composition."""
    rng = np.random.default_rng(3)
    B, T, H, D = 1, 12000, 2, 64
    ts = _inputs(rng, B, T, H, D, D, torch.bfloat16, gl=0.00001, gh=0.0005)
    seg = np.ones((B, T), dtype=np.int32)
    seg[0, 11000:] = 2
    S0 = rng.standard_normal((B, H, D, D)) * 2.0
    o, fs = _run(ts, seg, S0)
    ro, rfs = oracle.chunk_kda_segment_ids(*[f64(t) for t in ts], seg, initial_state=S0)
    check_close(f64(o), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final state")
    check_close(f64(o)[0, 7296:11000], ro[0, 7296:11000], "bf16", "last run of the first segment")


@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.float32, 64, 64), (torch.bfloat16, 64, 64),
                                         (torch.bfloat16, 128, 128), (torch.bfloat16, 128, 64)])
def test_padding_is_ignored(dtype, Dk, Dv):
    """RFC-0026 section 3.4: rows padded with id 0 (to a multiple of 64, as the
    module does, at the front, everywhere, and between two runs of one id),
    with non-zero initial states. Padding outputs are exactly 0; a row's final
    state is the state after its last real token (a row of padding only keeps
    its initial state bit for bit); the outputs of a padded row equal those of
    the same row with the trailing padding cut off."""
    rng = np.random.default_rng(Dk + Dv + (dtype == torch.float32))
    B, T, H = 4, 640, 2
    ts = _inputs(rng, B, T, H, Dk, Dv, dtype)
    seg = np.zeros((B, T), dtype=np.int32)
    seg[0, :250] = 1
    seg[0, 250:603] = 2                     # 37 trailing padding positions
    seg[1, 100:400] = 1                     # leading and trailing padding
    seg[1, 400:] = 2
    seg[3, :200] = 4
    seg[3, 300:500] = 4                     # the same id on both sides of padding
    S0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    print(f"padding dtype {dtype} Dk {Dk} Dv {Dv}", flush=True)
    o, fs = _run(ts, seg, S0, scale=0.7)
    ro, rfs = oracle.chunk_kda_segment_ids(*[f64(t) for t in ts], seg, scale=0.7, initial_state=S0)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o), ro, dt, "o")
    for b in range(B):
        check_close(f64(fs[b]), rfs[b], dt, f"final state of row {b}")
    pad = torch.from_numpy(seg == 0).to(device())
    assert torch.count_nonzero(o[pad]).item() == 0
    assert torch.equal(fs[2], torch.from_numpy(S0[2]).float().to(device()))
    # row 0 without its trailing padding: the same bits
    o0, f0 = _run([t[:1, :603].contiguous() for t in ts], seg[:1, :603].copy(), S0[:1], scale=0.7)
    assert torch.equal(o0[0], o[0, :603]) and torch.equal(f0[0], fs[0])


def test_every_token_its_own_segment():
    """T segments per row: more slots than the plan keeps in LDS."""
    rng = np.random.default_rng(9)
    B, T, H, D = 2, 5000, 1, 64
    ts = _inputs(rng, B, T, H, D, D, torch.bfloat16)
    seg = np.tile(np.arange(1, T + 1, dtype=np.int32), (B, 1))
    o, fs = _run(ts, seg)
    ro, rfs = oracle.chunk_kda_segment_ids(*[f64(t) for t in ts], seg)
    check_close(f64(o), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final states")


def test_matches_cu_seqlens_entry_on_flat_microbatch():
    """On the flattened micro-batch (no padding) the documents are the same in
    both entries, so every (segment, head) runs the same computation: the
    outputs agree bit for bit; a sampled segment is checked against the oracle."""
    pkv = _pkv()
    wl = workloads.make_workload("flat_microbatch", conv=False)
    cfg = wl.cfg
    B, T, H = cfg.B, cfg.T, cfg.H
    dev = device()
    q, k, g = [t.reshape(B, T, H, cfg.Dk).to(dev) for t in (wl.q, wl.k, wl.g)]
    v = wl.v.reshape(B, T, H, cfg.Dv).to(dev)
    beta = wl.beta.reshape(B, T, H).to(dev)
    seg = torch.from_numpy(np.ascontiguousarray(wl.segment_ids).astype(np.int32)).to(dev)
    o1, _ = pkv.chunk_kda_segment_ids(q, k, v, g, beta, seg, output_final_state=False)
    cu = pkv.segment_ids_to_cu_seqlens(seg, cfg.max_segs).cu_seqlens
    o2, _ = pkv.chunk_kda_varlen(q, k, v, g, beta, cu, output_final_state=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("dtype,Dk,Dv", [(torch.float32, 64, 32), (torch.bfloat16, 64, 64),
                                         (torch.bfloat16, 128, 128)])
def test_qk_l2norm(dtype, Dk, Dv):
    """RFC-0026 section 3.3's use_qk_l2norm_in_kernel on the [B, T] entry, with
    padding and unnormalised q and k."""
    pkv = _pkv()
    rng = np.random.default_rng(Dk + 5 * Dv)
    B, T, H = 3, 500, 2
    ts = _inputs(rng, B, T, H, Dk, Dv, dtype)
    ts[0] = (ts[0] * torch.from_numpy(rng.uniform(0.3, 4.0, (B, T, H, 1))).to(dtype)).to(dtype)
    ts[1] = (ts[1] * torch.from_numpy(rng.uniform(0.3, 4.0, (B, T, H, 1))).to(dtype)).to(dtype)
    seg = _ids(rng, B, T)
    S0 = rng.standard_normal((B, H, Dk, Dv)) * 0.5
    q, k, v, g, beta = [t.to(device()) for t in ts]
    o, fs = pkv.chunk_kda_segment_ids(q, k, v, g, beta, torch.from_numpy(seg).to(device()),
                                      initial_state=torch.from_numpy(S0).float().to(device()),
                                      use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_segment_ids(*[f64(t) for t in ts], seg, initial_state=S0, use_qk_l2norm=True)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o), ro, dt, "o")
    check_close(f64(fs), rfs, dt, "final states")
