"""GPU parity of pkv_chunk_kda_varlen against the fp64 oracle, plus the
invariants the pages require (reset, isolation, determinism)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import fullsize
from parity import check_close, device, f64, kda_inputs_to_device

pytestmark = pytest.mark.gpu


def _pkv():
    import packed_varlen_gated_amd as pkv
    return pkv


def _cu(wl):
    cu, _, _ = oracle.segment_ids_to_cu_seqlens(wl.segment_ids, wl.cfg.max_segs)
    return cu


def _run_wl(wl, final_state=True, cu=None):
    pkv = _pkv()
    q, k, v, g, beta = kda_inputs_to_device(wl)
    cu = _cu(wl) if cu is None else cu
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    flags = torch.zeros(1, dtype=torch.int32, device=device())
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, output_final_state=final_state, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    return o[0], fs, cu


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_midpad"])
def test_tiny_full_oracle(name):
    wl = workloads.make_workload(name)
    o, fs, cu = _run_wl(wl)
    ro, rfs = oracle.chunk_kda_varlen(f64(wl.q), f64(wl.k), f64(wl.v), f64(wl.g), f64(wl.beta), cu)
    check_close(f64(o), ro, "f32", "o")
    check_close(f64(fs), rfs, "f32", "final_state")
    assert np.all(f64(o)[cu[-1]:] == 0)


def test_ling3_tiny_sample_full_oracle():
    wl = workloads.make_workload("ling3_tiny_sample", conv=False)
    o, fs, cu = _run_wl(wl)
    ro, rfs = oracle.chunk_kda_varlen(f64(wl.q), f64(wl.k), f64(wl.v), f64(wl.g), f64(wl.beta), cu)
    check_close(f64(o), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final_state")
    for i in range(len(cu) - 1):
        if cu[i + 1] > cu[i]:
            check_close(f64(o)[cu[i]:cu[i + 1]], ro[cu[i]:cu[i + 1]], "bf16", f"o segment {i}")


@pytest.mark.parametrize("name", ["flat_microbatch", "many_short_docs", "long_context"])
def test_full_size_every_pair(name):
    """Every (segment, head) pair of the full-size workload against the oracle
    (run over the host's cores): o and final states, rel-L2 over the whole
    tensor and per segment; the uncovered tail and phantom slots exactly 0."""
    wl = workloads.make_workload(name)
    o, fs, cu = _run_wl(wl, final_state=True)
    dt = wl.cfg.dtype
    with fullsize.Store() as st:
        for n, t in zip(("q", "k", "v", "g", "beta"), (wl.q, wl.k, wl.v, wl.g, wl.beta)):
            st.put(n, t)
        st.put("o", o)
        st.put("fs", fs)
        print(f"  {name}: oracle over {len(cu) - 1} slots x {wl.cfg.H} heads on "
              f"{fullsize.workers()} processes", flush=True)
        summ = fullsize.summarize(fullsize.run_pairs(fullsize._fwd_job, st.paths, wl.cfg.H, cu))
    for n, r in summ.items():
        print(f"  {name} {n}: rel-L2 {r['rel_l2']:.3e} (worst segment {r['worst_segment_rel_l2']:.3e}), "
              f"max abs err {r['max_abs']:.3e} of max |ref| {r['max_ref']:.3e}, {r['pairs']} pairs", flush=True)
        assert r["finite"], f"{n}: non-finite output"
        assert r["pairs"] == int(np.sum(np.diff(cu) > 0)) * wl.cfg.H
        if dt == "f32":
            assert r["max_abs"] <= 1e-4 * r["max_ref"], n
        else:
            assert r["rel_l2"] <= 2e-2 and r["worst_segment_rel_l2"] <= 2e-2, n
    lens = np.diff(cu)
    assert torch.count_nonzero(o[int(cu[-1]):]).item() == 0
    for i in range(len(lens)):
        if lens[i] == 0:
            assert torch.count_nonzero(fs[i]).item() == 0


def _small_case(rng, N, H, Dk, Dv, dtype, cu):
    q = rng.standard_normal((N, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((N, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, Dv))
    g = -rng.uniform(0.01, 0.3, (N, H, Dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, H))))
    ts = [torch.from_numpy(a).to(dtype) for a in (q, k, v, g, beta)]
    return ts


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Dk,Dv", [(32, 32), (64, 64), (128, 128), (32, 128), (128, 64), (64, 32)])
def test_small_shapes(dtype, Dk, Dv):
    pkv = _pkv()
    rng = np.random.default_rng(Dk * 7 + Dv)
    H = 3
    lens = [1, 63, 64, 65, 2, 127, 128, 129, 16, 17, 200]
    cu = np.concatenate([[0], np.cumsum(lens), [sum(lens)] * 2])      # two phantom slots
    N = sum(lens) + 37                                                 # uncovered tail
    ts = _small_case(rng, N, H, Dk, Dv, dtype, cu)
    q, k, v, g, beta = [t.to(device()) for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    o, fs = pkv.chunk_kda_varlen(q[None], k[None], v[None], g[None], beta[None], cud, scale=0.5)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu, scale=0.5)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o[0]), ro, dt, "o")
    check_close(f64(fs), rfs, dt, "final_state")
    for i in range(len(cu) - 1):
        if cu[i + 1] > cu[i]:
            check_close(f64(o[0])[cu[i]:cu[i + 1]], ro[cu[i]:cu[i + 1]], dt, f"segment {i}")
    assert torch.count_nonzero(o[0, cu[-1]:]).item() == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_no_cu_seqlens_is_one_segment(dtype):
    pkv = _pkv()
    rng = np.random.default_rng(5)
    N, H, D = 301, 2, 64
    ts = _small_case(rng, N, H, D, D, dtype, None)
    q, k, v, g, beta = [t.to(device())[None] for t in ts]
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, None)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], None)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o[0]), ro, dt, "o")
    check_close(f64(fs), rfs, dt, "state")


def test_leakage_row_independence_determinism():
    pkv = _pkv()
    wl = workloads.make_workload("many_short_docs")
    q, k, v, g, beta = kda_inputs_to_device(wl)
    cu = _cu(wl)
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    o1, f1 = pkv.chunk_kda_varlen(q, k, v, g, beta, cud)
    o2, f2 = pkv.chunk_kda_varlen(q, k, v, g, beta, cud)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2), "not deterministic"
    # perturb document 5 only: every other document is bit-identical
    a, e = int(cu[5]), int(cu[6])
    v2, q2, g2 = v.clone(), q.clone(), g.clone()
    v2[0, a:e] *= -3
    q2[0, a:e] += 1
    g2[0, a:e] -= 0.5
    o3, f3 = pkv.chunk_kda_varlen(q2, k, v2, g2, beta, cud)
    torch.cuda.synchronize()
    keep = torch.ones(wl.N, dtype=torch.bool, device=device())
    keep[a:e] = False
    assert torch.equal(o1[0, keep], o3[0, keep])
    assert torch.equal(torch.cat([f1[:5], f1[6:]]), torch.cat([f3[:5], f3[6:]]))
    assert not torch.equal(o1[0, a:e], o3[0, a:e])
    # row independence: change the segment ids of row 3 only; rows 0..2 keep their bits
    seg = wl.segment_ids.copy()
    seg[3] = np.where(seg[3] > 0, (seg[3] + 1) // 2, 0)     # merge pairs of documents in row 3
    cu_b = torch.from_numpy(oracle.segment_ids_to_cu_seqlens(seg, wl.cfg.max_segs)[0].astype(np.int32)).to(device())
    o4, _ = pkv.chunk_kda_varlen(q, k, v, g, beta, cu_b)
    torch.cuda.synchronize()
    T = wl.cfg.T
    assert torch.equal(o1[0, :3 * T], o4[0, :3 * T])
    assert not torch.equal(o1[0, 3 * T:], o4[0, 3 * T:])


def test_packed_equals_each_document_alone():
    pkv = _pkv()
    wl = workloads.make_workload("ling3_tiny_sample", conv=False)
    q, k, v, g, beta = kda_inputs_to_device(wl)
    cu = _cu(wl)
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud)
    for i in range(len(cu) - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        if e <= a:
            continue
        oi, fi = pkv.chunk_kda_varlen(q[:, a:e].contiguous(), k[:, a:e].contiguous(), v[:, a:e].contiguous(),
                                      g[:, a:e].contiguous(), beta[:, a:e].contiguous(), None)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:e], oi), f"segment {i}"
        assert torch.equal(fs[i], fi[0]), f"segment {i}"


def test_bad_cu_seqlens_sets_flag():
    pkv = _pkv()
    rng = np.random.default_rng(1)
    N, H, D = 200, 2, 32
    ts = _small_case(rng, N, H, D, D, torch.float32, None)
    q, k, v, g, beta = [t.to(device())[None] for t in ts]
    for bad in ([0, 50, 40, 120], [3, 50, 90, 120], [0, 50, 90, 250]):
        cud = torch.tensor(bad, dtype=torch.int32, device=device())
        flags = torch.zeros(1, dtype=torch.int32, device=device())
        pkv.chunk_kda_varlen(q, k, v, g, beta, cud, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) & pkv.FLAG_BAD_CU_SEQLENS, bad


@pytest.mark.parametrize("n_slots", [37, 2100])
def test_slot_order_ties_phantoms(n_slots):
    """The longest-first processing order gives the oracle's per-segment
    results: lengths with ties, empty slots between real ones, and phantom
    slots at the end (37 slots, and 2100, more than the plan's 2048 length
    bins and two tiles of its slot scan)."""
    pkv = _pkv()
    rng = np.random.default_rng(n_slots)
    H, D = 2, 64
    lens = [int(x) for x in rng.choice([0, 1, 64, 65, 130, 130, 7, 64, 0, 300], size=30)]
    real = np.concatenate([[0], np.cumsum(lens)])
    cu = np.concatenate([real, [real[-1]] * (n_slots + 1 - len(real))])
    N = int(real[-1]) + 5
    ts = _small_case(rng, N, H, D, D, torch.bfloat16, cu)
    q, k, v, g, beta = [t.to(device()) for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    print(f"slots {n_slots}: workspace {pkv.chunk_kda_varlen_workspace_size(N, H, D, D, n_slots, torch.bfloat16)} bytes",
          flush=True)
    o, fs = pkv.chunk_kda_varlen(q[None], k[None], v[None], g[None], beta[None], cud)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu)
    check_close(f64(o[0]), ro, "bf16", "o")
    for i in range(len(cu) - 1):
        if cu[i + 1] > cu[i]:
            check_close(f64(o[0])[cu[i]:cu[i + 1]], ro[cu[i]:cu[i + 1]], "bf16", f"segment {i}")
            check_close(f64(fs[i]), rfs[i], "bf16", f"state {i}")
        else:
            assert torch.count_nonzero(fs[i]).item() == 0
    assert torch.count_nonzero(o[0, cu[-1]:]).item() == 0


# Segments longer than 128 chunks (8192 tokens) are cut into
# m = min(16, ceil(n / 64)) nearly equal runs (run j = chunks
# [n j / m, n (j + 1) / m)), whatever else the launch holds; a run starts from
# the state composed of the earlier runs' states and decay products. Empty
# slots get no run. Slow gates keep the carried state large, so a wrong
# composition shows.
def _runs_of(n):
    return 1 if n <= 128 else min(16, -(-n // 64))


@pytest.mark.parametrize("case,H,Dk,Dv,lens,slots,runs,pieces", [
    # 313 chunks -> 5 runs
    ("one_segment", 2, 64, 64, [20000], None, 5, 4),
    # 141, 2, 0, 266, 128, 129, 1 chunks: 3 + 1 + 5 + 1 + 3 + 1 runs; the
    # empty slot and the 3 phantoms get none; 128 chunks is not cut
    ("mixed", 2, 128, 128, [9000, 100, 0, 17000, 8192, 8193, 1], 10, 14, 8),
    # 1100 chunks: the 16-run cap
    ("sixteen_runs", 1, 128, 64, [64 * 1100 - 17], 2, 16, 15),
    # 31, 17 and 8 chunks (a Ling3-like sample at H = 32): never cut
    ("short_docs", 32, 128, 128, [1984, 1050, 512], 3, 3, 0),
])
def test_long_segments_cut_into_runs(case, H, Dk, Dv, lens, slots, runs, pieces):
    pkv = _pkv()
    rng = np.random.default_rng(len(case))
    if slots is None:
        cu = None
        N = lens[0]
    else:
        real = np.concatenate([[0], np.cumsum(lens)])
        cu = np.concatenate([real, [real[-1]] * (slots + 1 - len(real))])
        N = int(real[-1]) + 3
    q = rng.standard_normal((N, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((N, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, Dv))
    g = -rng.uniform(0.0001, 0.003, (N, H, Dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, H))))
    ts = [torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v, g, beta)]
    dq, dk, dv, dg, db = [t.to(device())[None] for t in ts]
    max_segs = 1 if cu is None else len(cu) - 1
    ws = torch.empty(pkv.chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, torch.bfloat16),
                     dtype=torch.uint8, device=device())
    cud = None if cu is None else torch.from_numpy(cu.astype(np.int32)).to(device())
    print(f"{case}: N {N} H {H} Dk {Dk} Dv {Dv} slots {max_segs} workspace {ws.numel()} bytes", flush=True)
    o, fs = pkv.chunk_kda_varlen(dq, dk, dv, dg, db, cud, workspace=ws)
    torch.cuda.synchronize()
    head = ws[:8].view(torch.int32).cpu().tolist()
    assert (head[0], head[1]) == (runs, pieces)
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu)
    go = f64(o[0])
    check_close(go, ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final states")
    bounds = np.array([0, N]) if cu is None else cu
    for i in range(len(bounds) - 1):
        a, e = int(bounds[i]), int(bounds[i + 1])
        n = (e - a + 63) // 64
        m = _runs_of(n)
        if m == 1:
            continue
        for j in range(m):
            ra, re = a + 64 * (n * j // m), min(e, a + 64 * (n * (j + 1) // m))
            check_close(go[ra:re], ro[ra:re], "bf16", f"segment {i} run {j}")
        # the carried state matters: the last run alone from zero is far off
        alone, _ = oracle.chunk_kda_varlen(*[f64(t)[ra:re] for t in ts], None)
        assert np.linalg.norm(alone - ro[ra:re]) > 0.2 * np.linalg.norm(ro[ra:re])
    if cu is not None:
        assert torch.count_nonzero(o[0, int(cu[-1]):]).item() == 0


def test_row_independence_with_cut_segments():
    """RFC-0026 Tests (row independence): two rows, row 0 holding documents
    long enough to be cut into runs; changing only row 1's segment ids (which
    changes the launch's chunk count and its number of runs) leaves row 0's
    outputs and final states bit-identical."""
    pkv = _pkv()
    rng = np.random.default_rng(123)
    B, T, H, D = 2, 20480, 16, 128
    N = B * T
    seg = np.zeros((B, T), dtype=np.int32)
    seg[0, :12000] = 1
    seg[0, 12000:] = 2                      # 188 and 133 chunks: cut into 3 runs each
    variants = {
        "seven documents": [700, 1500, 300, 4000, 9000, 2500, 2480],
        "one document": [20480],
        "205 short documents": [100] * 204 + [80],   # 410 chunks
        "padding only": None,                        # row 1 all id 0
    }
    ts = _small_case(rng, N, H, D, D, torch.bfloat16, None)
    q, k, v, g, beta = [t.to(device())[None] for t in ts]
    max_segs = 256
    ws = torch.empty(pkv.chunk_kda_varlen_workspace_size(N, H, D, D, max_segs, torch.bfloat16),
                     dtype=torch.uint8, device=device())
    outs = []
    for name, lens in variants.items():
        s = seg.copy()
        s[1] = 0 if lens is None else np.repeat(np.arange(1, len(lens) + 1), lens)
        cu = oracle.segment_ids_to_cu_seqlens(s, max_segs)[0]
        cud = torch.from_numpy(cu.astype(np.int32)).to(device())
        o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, workspace=ws)
        torch.cuda.synchronize()
        head = ws[:8].view(torch.int32).cpu().tolist()
        print(f"  row 1 {name}: runs {head[0]}, saved pieces {head[1]}", flush=True)
        outs.append((name, o, fs, head))
    assert len({tuple(x[3][:2]) for x in outs}) == len(outs)  # every launch differs
    _, o0, f0, _ = outs[0]
    for name, o, fs, _ in outs[1:]:
        assert torch.equal(o0[0, :T], o[0, :T]), name
        assert torch.equal(f0[:2], fs[:2]), name  # row 0's two documents are slots 0 and 1
        assert not torch.equal(o0[0, T:], o[0, T:]), name


def test_packed_equals_each_document_alone_long_context():
    """RFC-0026 Tests (packed equivalence with per-document runs), bit-exact,
    on long_context, whose long documents are cut into runs: each document run
    alone (cu_seqlens = None) gives the packed call's outputs and final state
    bit for bit."""
    pkv = _pkv()
    wl = workloads.make_workload("long_context")
    q, k, v, g, beta = kda_inputs_to_device(wl)
    cu = _cu(wl)
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    ws = torch.empty(pkv.chunk_kda_varlen_workspace_size(wl.N, wl.cfg.H, 128, 128, len(cu) - 1, torch.bfloat16),
                     dtype=torch.uint8, device=device())
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, workspace=ws)
    torch.cuda.synchronize()
    print(f"  long_context packed: runs {ws[:8].view(torch.int32).cpu().tolist()[:2]}", flush=True)
    cut = 0
    for i in range(len(cu) - 1):
        a, e = int(cu[i]), int(cu[i + 1])
        if e <= a:
            continue
        cut += (e - a + 63) // 64 > 128
        oi, fi = pkv.chunk_kda_varlen(q[:, a:e].contiguous(), k[:, a:e].contiguous(), v[:, a:e].contiguous(),
                                      g[:, a:e].contiguous(), beta[:, a:e].contiguous(), None)
        torch.cuda.synchronize()
        print(f"  document {i}: {e - a} tokens", flush=True)
        assert torch.equal(o[:, a:e], oi), f"segment {i}"
        assert torch.equal(fs[i], fi[0]), f"segment {i}"
    assert cut >= 3  # the invariant is tested where cuts happen


def _plan_items(lens, grouped):
    """Items of the forward plan for segments of these token counts (slot order):
    a segment of n chunks is _runs_of(n) runs; when grouped (a call without
    initial and final states), short segments (1..4 chunks) in consecutive slots
    whose first chunks fall in the same 12-chunk window of the global chunk order
    share one item."""
    n = [-(-int(L) // 64) for L in lens]
    cb = np.concatenate([[0], np.cumsum(n)])
    items, span = 0, 0
    for i, ni in enumerate(n):
        if ni == 0:
            continue
        short = grouped and ni <= 4
        if short and i > 0 and 1 <= n[i - 1] <= 4 and cb[i - 1] // 12 == cb[i] // 12:
            span += ni
            assert span <= 15
            continue
        span = ni
        items += _runs_of(ni)
    return items


def _group_lens(rng):
    """Short documents of 1..300 tokens (1..5 chunks) with exact multiples of 64,
    single tokens, empty slots and a document cut into runs among them."""
    lens = list(rng.integers(1, 301, 70))
    lens[3:9] = [64, 1, 128, 0, 65, 256]
    lens[20:23] = [9000, 0, 320]   # 141 chunks (3 runs), an empty slot, 5 chunks
    lens[40:44] = [1, 1, 1, 63]
    return lens


@pytest.mark.parametrize("Dk,Dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_grouped_short_documents(Dk, Dv):
    """Without initial and final states, short documents share an item and each
    starts from the zero state inside it: the outputs, and the states kept
    before every chunk, are bit-identical to those of the call that runs every
    document as its own item (the same call with final states), and the outputs
    match the oracle; the plan holds the expected number of items."""
    pkv = _pkv()
    rng = np.random.default_rng(Dk + 3 * Dv)
    lens = _group_lens(rng)
    slots = len(lens) + 3
    real = np.concatenate([[0], np.cumsum(lens)])
    cu = np.concatenate([real, [real[-1]] * (slots + 1 - len(real))]).astype(np.int64)
    N, H = int(real[-1]) + 5, 2
    print(f"  grouped Dk={Dk} Dv={Dv}: N {N}, {slots} slots, items {_plan_items(lens, True)} "
          f"grouped / {_plan_items(lens, False)}", flush=True)
    ts = _small_case(rng, N, H, Dk, Dv, torch.bfloat16, None)
    q, k, v, g, beta = [t.to(device())[None] for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    ws = torch.empty(pkv.chunk_kda_varlen_workspace_size(N, H, Dk, Dv, slots, torch.bfloat16),
                     dtype=torch.uint8, device=device())
    nst = pkv.chunk_kda_states_size(N, H, Dk, Dv, slots)
    st_g = torch.zeros(nst, dtype=torch.uint8, device=device())
    st_u = torch.zeros(nst, dtype=torch.uint8, device=device())
    o_g, none = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, output_final_state=False, workspace=ws)
    torch.cuda.synchronize()
    items_g = ws[:8].view(torch.int32).cpu().tolist()[0]
    o_u, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, workspace=ws)
    torch.cuda.synchronize()
    items_u = ws[:8].view(torch.int32).cpu().tolist()[0]
    assert none is None
    assert (items_g, items_u) == (_plan_items(lens, True), _plan_items(lens, False))
    assert items_g < items_u
    assert torch.equal(o_g, o_u)
    o_gs, _ = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, output_final_state=False, chunk_states=st_g)
    o_us, _ = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, chunk_states=st_u)
    torch.cuda.synchronize()
    assert torch.equal(o_gs, o_g) and torch.equal(o_us, o_g)
    assert torch.equal(st_g, st_u)
    assert torch.count_nonzero(st_g).item() > 0
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu)
    check_close(f64(o_g[0]), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final states")


# RFC-0026 section 3.3's initial_state, one per segment slot: every segment
# starts from its slot's state; empty slots keep it as their final state.
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Dk,Dv", [(32, 32), (64, 64), (128, 128), (64, 128), (128, 64)])
def test_initial_state(dtype, Dk, Dv):
    pkv = _pkv()
    rng = np.random.default_rng(Dk * 7 + Dv)
    lens = [70, 0, 1, 200, 64]
    real = np.concatenate([[0], np.cumsum(lens)])
    cu = np.concatenate([real, [real[-1]] * 2])  # two phantom slots
    N, H = int(real[-1]) + 9, 2
    ts = _small_case(rng, N, H, Dk, Dv, dtype, cu)
    S0 = rng.standard_normal((len(cu) - 1, H, Dk, Dv)) * 0.5
    q, k, v, g, beta = [t.to(device())[None] for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    s0 = torch.from_numpy(S0).to(torch.float32).to(device())
    print(f"initial_state dtype {dtype} Dk {Dk} Dv {Dv}", flush=True)
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, initial_state=s0, scale=0.8)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu, scale=0.8, initial_state=S0)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o[0]), ro, dt, "o")
    for i in range(len(cu) - 1):
        check_close(f64(fs[i]), rfs[i], dt, f"state {i}")
    assert torch.equal(fs[1], s0[1]) and torch.equal(fs[-1], s0[-1])  # empty slots keep it
    assert torch.count_nonzero(o[0, int(cu[-1]):]).item() == 0


def test_initial_state_with_cut_segments():
    """A long segment cut into runs: the first run starts from the initial
    state and the later ones fold it in through the composition."""
    pkv = _pkv()
    rng = np.random.default_rng(77)
    N, H, D = 9000, 2, 64
    q = rng.standard_normal((N, H, D)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((N, H, D)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, D))
    g = -rng.uniform(0.00001, 0.0005, (N, H, D))  # slow: the initial state lasts the whole segment
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, H))))
    ts = [torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v, g, beta)]
    S0 = rng.standard_normal((1, H, D, D)) * 2.0
    dq, dk, dv, dg, db = [t.to(device())[None] for t in ts]
    ws = torch.empty(pkv.chunk_kda_varlen_workspace_size(N, H, D, D, 1, torch.bfloat16),
                     dtype=torch.uint8, device=device())
    o, fs = pkv.chunk_kda_varlen(dq, dk, dv, dg, db, None, workspace=ws,
                                 initial_state=torch.from_numpy(S0).float().to(device()))
    torch.cuda.synchronize()
    assert ws[:8].view(torch.int32).cpu().tolist()[1] == 2  # 141 chunks: 3 runs, 2 saved pieces
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], None, initial_state=S0)
    check_close(f64(o[0]), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final state")
    # the initial state matters for the last run's outputs (chunks 94..140):
    # five times the bf16 tolerance, so dropping it from the composition fails above
    r0, _ = oracle.chunk_kda_varlen(*[f64(t) for t in ts], None)
    assert np.linalg.norm(ro[6016:] - r0[6016:]) > 0.1 * np.linalg.norm(ro[6016:])


# RFC-0026 section 3.3's use_qk_l2norm_in_kernel: q and k are normalised
# inside the call, so the inputs here are not unit-norm (random positive
# per-(token, head) scales); the oracle normalises in fp64.
def _unnormalised(ts, rng):
    q, k = ts[0], ts[1]
    N, H = q.shape[0], q.shape[1]
    sq = torch.from_numpy(rng.uniform(0.3, 4.0, (N, H, 1))).to(q.dtype)
    sk = torch.from_numpy(rng.uniform(0.3, 4.0, (N, H, 1))).to(k.dtype)
    return [(q * sq).to(q.dtype), (k * sk).to(k.dtype)] + list(ts[2:])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Dk,Dv", [(32, 32), (64, 64), (128, 128), (64, 128), (128, 64)])
def test_qk_l2norm_small_shapes(dtype, Dk, Dv):
    pkv = _pkv()
    rng = np.random.default_rng(Dk * 11 + Dv)
    H = 3
    lens = [1, 63, 64, 65, 2, 127, 129, 16, 200]
    cu = np.concatenate([[0], np.cumsum(lens), [sum(lens)]])
    N = sum(lens) + 21
    ts = _unnormalised(_small_case(rng, N, H, Dk, Dv, dtype, cu), rng)
    q, k, v, g, beta = [t.to(device()) for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    print(f"qk_l2norm dtype {dtype} Dk {Dk} Dv {Dv}", flush=True)
    o, fs = pkv.chunk_kda_varlen(q[None], k[None], v[None], g[None], beta[None], cud, scale=0.6,
                                 use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu, scale=0.6, use_qk_l2norm=True)
    dt = "f32" if dtype == torch.float32 else "bf16"
    check_close(f64(o[0]), ro, dt, "o")
    check_close(f64(fs), rfs, dt, "final_state")
    for i in range(len(cu) - 1):
        if cu[i + 1] > cu[i]:
            check_close(f64(o[0])[cu[i]:cu[i + 1]], ro[cu[i]:cu[i + 1]], dt, f"segment {i}")
    # the unnormalised inputs give a different result without the option
    o2, _ = pkv.chunk_kda_varlen(q[None], k[None], v[None], g[None], beta[None], cud, scale=0.6)
    torch.cuda.synchronize()
    assert np.linalg.norm(f64(o2[0]) - ro) > 0.1 * np.linalg.norm(ro)


def test_qk_l2norm_cut_segment_and_ling3_sample():
    """The option through the state pass of a cut segment (141 chunks, 3 runs,
    with an initial state) and on the whole Ling3-like sample."""
    pkv = _pkv()
    rng = np.random.default_rng(91)
    N, H, D = 9000, 2, 128
    ts = _unnormalised(_small_case(rng, N, H, D, D, torch.bfloat16, None), rng)
    S0 = rng.standard_normal((1, H, D, D))
    dq, dk, dv, dg, db = [t.to(device())[None] for t in ts]
    ws = torch.empty(pkv.chunk_kda_varlen_workspace_size(N, H, D, D, 1, torch.bfloat16),
                     dtype=torch.uint8, device=device())
    o, fs = pkv.chunk_kda_varlen(dq, dk, dv, dg, db, None, workspace=ws, use_qk_l2norm_in_kernel=True,
                                 initial_state=torch.from_numpy(S0).float().to(device()))
    torch.cuda.synchronize()
    assert ws[:8].view(torch.int32).cpu().tolist()[:2] == [3, 2]
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], None, initial_state=S0, use_qk_l2norm=True)
    check_close(f64(o[0]), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final state")
    check_close(f64(o[0])[6016:], ro[6016:], "bf16", "last run")

    wl = workloads.make_workload("ling3_tiny_sample", conv=False)
    cu = _cu(wl)
    ts = _unnormalised([wl.q, wl.k, wl.v, wl.g, wl.beta], rng)
    q, k, v, g, beta = [t.to(device())[None] for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, use_qk_l2norm_in_kernel=True)
    torch.cuda.synchronize()
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in ts], cu, use_qk_l2norm=True)
    check_close(f64(o[0]), ro, "bf16", "ling3 o")
    check_close(f64(fs), rfs, "bf16", "ling3 final states")


def _gate_case(rng, N, H, Dk, Dv, glo, ghi):
    q = rng.standard_normal((N, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((N, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, Dv))
    g = -rng.uniform(glo, ghi, (N, H, Dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, H))))
    return [q, k, v, g, beta]


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128)])
def test_gate_range_edge_and_flag(Dk, Dv):
    """RFC-0026 Background recurrence with strong forgetting on the chunked
    bf16 path. Gates of -4.3 .. -4.7 per token keep every 16-token sub-chunk
    sum above the path's limit (-83): forward and reverse match the oracle and
    no flag is set. One key channel of one head at g = -7 (a 16-token sum of
    -112) sets PKV_FLAG_GATE_RANGE on both passes."""
    pkv = _pkv()
    rng = np.random.default_rng(Dk + 11)
    H = 2
    lens = [200, 64, 77]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = int(cu[-1])
    arrs = _gate_case(rng, N, H, Dk, Dv, 4.3, 4.7)
    do = rng.standard_normal((N, H, Dv))
    ts = [torch.from_numpy(a).to(torch.bfloat16) for a in arrs]
    dot = torch.from_numpy(do).to(torch.bfloat16)
    dev = device()
    q, k, v, g, beta = [t.to(dev)[None] for t in ts]
    cud = torch.from_numpy(cu).to(dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, flags=flags)
    gr = pkv.chunk_kda_varlen_backward(q, k, v, g, beta, dot.to(dev)[None], cud, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    x64 = [f64(t) for t in ts]
    ro, rfs = oracle.chunk_kda_varlen(*x64, cu)
    check_close(f64(o[0]), ro, "bf16", "o")
    check_close(f64(fs), rfs, "bf16", "final_state")
    ref = oracle.chunk_kda_varlen_backward(*x64, f64(dot), cu)
    for n, got, r in zip(("dq", "dk", "dv", "dg", "dbeta"), gr[:5], ref[:5]):
        check_close(f64(got[0]), r, "bf16", n)
    # one channel beyond the limit
    g2 = g.clone()
    g2[0, :, 1, 3] = -7.0
    for backward in (False, True):
        flags.zero_()
        if backward:
            pkv.chunk_kda_varlen_backward(q, k, v, g2, beta, dot.to(dev)[None], cud, flags=flags)
        else:
            pkv.chunk_kda_varlen(q, k, v, g2, beta, cud, flags=flags)
        torch.cuda.synchronize()
        assert int(flags.item()) & pkv.FLAG_GATE_RANGE, ("backward" if backward else "forward")
