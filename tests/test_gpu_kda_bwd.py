"""GPU parity of pkv_chunk_kda_varlen_backward (the reverse pass of the packed
KDA recurrence, RFC-0026 Background and section 3.3) against the fp64 oracle's
reverse mode, which keeps every state and takes dg per step, while the kernel
recomputes the states and takes dg as a reverse running sum."""

import numpy as np
import pytest
import torch

import oracle
import workloads
import fullsize
from parity import check_close, device, f64

pytestmark = pytest.mark.gpu


def _pkv():
    import packed_varlen_gated_amd as pkv
    return pkv


def _inputs(rng, N, H, Dk, Dv, dtype, gl=0.01, gh=0.3):
    q = rng.standard_normal((1, N, H, Dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((1, N, H, Dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((1, N, H, Dv))
    g = -rng.uniform(gl, gh, (1, N, H, Dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal((1, N, H))))
    do = rng.standard_normal((1, N, H, Dv))
    return [torch.from_numpy(a).to(dtype) for a in (q, k, v, g, beta, do)]


def _oracle(ts, cu, scale, S0, dF):
    q, k, v, g, beta, do = [f64(t)[0] for t in ts]
    return oracle.chunk_kda_varlen_backward(q, k, v, g, beta, do, cu, scale, S0, dF)


def _run(ts, cu, scale, S0, dF, flags=None, want_dinit=True):
    pkv = _pkv()
    dev = device()
    q, k, v, g, beta, do = [t.to(dev) for t in ts]
    cud = torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(dev)
    s0 = None if S0 is None else torch.from_numpy(S0).float().to(dev)
    df = None if dF is None else torch.from_numpy(dF).float().to(dev)
    r = pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, cud, scale=scale, initial_state=s0,
                                      dfinal_state=df, output_d_initial_state=want_dinit, flags=flags)
    torch.cuda.synchronize()
    return r


def _compare(r, ref, tol, what):
    names = ["dq", "dk", "dv", "dg", "dbeta"]
    for name, got, exp in zip(names, r[:5], ref[:5]):
        check_close(f64(got)[0], exp, tol, f"{what} {name}")
    if r.d_initial_state is not None:
        check_close(f64(r.d_initial_state), ref[5], tol, f"{what} d_initial_state")


CU_RAGGED = [0, 1, 66, 66, 200, 263, 264, 330]  # single tokens, an empty slot, tails past 64


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Dk,Dv", [(32, 32), (64, 64), (128, 128), (64, 128), (128, 32)])
def test_small_shapes_full_oracle(dtype, Dk, Dv):
    """Every output against the oracle, with initial states, a final-state
    cotangent and scale != 1; ragged segments, an empty slot and positions
    past cu[max_segs] (zero gradients)."""
    print(f"  bwd small dtype={dtype} Dk={Dk} Dv={Dv}", flush=True)
    rng = np.random.default_rng(7 * Dk + Dv + (dtype == torch.bfloat16))
    N, H = 345, 2
    cu = np.array(CU_RAGGED, dtype=np.int64)
    ts = _inputs(rng, N, H, Dk, Dv, dtype)
    S = len(cu) - 1
    S0 = rng.standard_normal((S, H, Dk, Dv)) * 0.5
    dF = rng.standard_normal((S, H, Dk, Dv)) * 0.5
    scale = Dk ** -0.5
    tol = "f32" if dtype == torch.float32 else "bf16"
    r = _run(ts, cu, scale, S0, dF)
    ref = _oracle(ts, cu, scale, S0, dF)
    _compare(r, ref, tol, f"{Dk}x{Dv}")
    for t in r[:5]:
        assert np.all(f64(t)[0, cu[-1]:] == 0)
    # the empty slot passes the cotangent straight through to its initial state
    assert np.array_equal(f64(r.d_initial_state)[2], dF[2].astype(np.float32).astype(np.float64))


@pytest.mark.parametrize("with_s0,with_dF", [(False, False), (True, False), (False, True)])
def test_optional_states(with_s0, with_dF):
    print(f"  bwd optional states s0={with_s0} dF={with_dF}", flush=True)
    rng = np.random.default_rng(11 + 2 * with_s0 + with_dF)
    N, H, D = 300, 3, 64
    cu = np.array([0, 100, 170, 300], dtype=np.int64)
    ts = _inputs(rng, N, H, D, D, torch.float32)
    S0 = rng.standard_normal((3, H, D, D)) if with_s0 else None
    dF = rng.standard_normal((3, H, D, D)) if with_dF else None
    r = _run(ts, cu, 1.0, S0, dF, want_dinit=True)
    ref = _oracle(ts, cu, 1.0, S0, dF)
    _compare(r, ref, "f32", "optional")


def test_no_cu_seqlens_is_one_segment():
    print("  bwd cu_seqlens=None", flush=True)
    pkv = _pkv()
    rng = np.random.default_rng(5)
    N, H, D = 200, 2, 32
    ts = _inputs(rng, N, H, D, D, torch.float32)
    q, k, v, g, beta, do = [t.to(device()) for t in ts]
    r = pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, None, scale=0.5)
    torch.cuda.synchronize()
    ref = _oracle(ts, None, 0.5, None, None)
    _compare(r, ref, "f32", "one segment")


def test_grads_are_segment_local():
    """The reset makes each segment's gradients depend on that segment alone:
    changing every input of segment 1 leaves segments 0 and 2 bit-identical."""
    print("  bwd segment isolation", flush=True)
    rng = np.random.default_rng(21)
    N, H, D = 256, 2, 64
    cu = np.array([0, 90, 180, 256], dtype=np.int64)
    ts = _inputs(rng, N, H, D, D, torch.bfloat16)
    r1 = _run(ts, cu, 1.0, None, None)
    ts2 = [t.clone() for t in ts]
    alt = _inputs(np.random.default_rng(22), N, H, D, D, torch.bfloat16)
    for t, a in zip(ts2, alt):
        t[0, 90:180] = a[0, 90:180]
    r2 = _run(ts2, cu, 1.0, None, None)
    for a, b in zip(r1[:5], r2[:5]):
        a, b = a.cpu(), b.cpu()
        assert torch.equal(a[0, :90], b[0, :90]) and torch.equal(a[0, 180:], b[0, 180:])
        assert not torch.equal(a[0, 90:180], b[0, 90:180])


def test_gate_identity_with_hip_forward():
    """At a segment's last token dg is q dq - k dk there plus the row sums of
    dF * S_end; S_end here is the HIP forward's final state, so the backward
    and forward entries agree on the state they both imply. (At the first
    token the same sum cancels to round-off and tests nothing.)"""
    print("  bwd gate identity with the HIP forward", flush=True)
    pkv = _pkv()
    rng = np.random.default_rng(31)
    N, H, D = 180, 2, 64
    cu = np.array([0, 70, 180], dtype=np.int64)
    ts = _inputs(rng, N, H, D, D, torch.float32, gl=0.001, gh=0.02)
    dF = rng.standard_normal((2, H, D, D))
    r = _run(ts, cu, 1.0, None, dF, want_dinit=False)
    q, k, v, g, beta, do = [t.to(device()) for t in ts]
    cud = torch.from_numpy(cu.astype(np.int32)).to(device())
    _, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, cud)
    torch.cuda.synchronize()
    qn, kn = f64(ts[0])[0], f64(ts[1])[0]
    dq, dk, dg = f64(r.dq)[0], f64(r.dk)[0], f64(r.dg)[0]
    for i in range(2):
        t = cu[i + 1] - 1
        end_term = (dF[i] * f64(fs)[i]).sum(-1)              # [H, Dk]
        assert np.abs(end_term).max() > 0.1
        rhs = qn[t] * dq[t] - kn[t] * dk[t] + end_term
        np.testing.assert_allclose(dg[t], rhs, rtol=0, atol=1e-4 * np.abs(end_term).max())


def test_bad_cu_seqlens_sets_flag():
    print("  bwd bad cu_seqlens", flush=True)
    rng = np.random.default_rng(3)
    N, H, D = 64, 1, 32
    ts = _inputs(rng, N, H, D, D, torch.float32)
    flags = torch.zeros(1, dtype=torch.int32, device=device())
    _run(ts, np.array([0, 40, 30, 64]), 1.0, None, None, flags=flags, want_dinit=False)
    assert int(flags.item()) & _pkv().FLAG_BAD_CU_SEQLENS


@pytest.mark.parametrize("lens,Dk,Dv", [((9000,), 64, 64), ((70, 20000, 33), 64, 64), ((8300,), 128, 128)])
def test_long_segments_cut_into_pieces(lens, Dk, Dv):
    """One head and long documents: the plan cuts every segment over 128 chunks
    into pieces of about 64 (141 chunks -> 3, 313 -> 5, 130 -> 3), so the state
    kernel composes the pieces' summaries; with an initial state and a
    final-state cotangent on every slot."""
    print(f"  bwd cut pieces lens={lens} Dk={Dk} Dv={Dv}", flush=True)
    rng = np.random.default_rng(sum(lens) + Dk)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, H = int(cu[-1]), 1
    ts = _inputs(rng, N, H, Dk, Dv, torch.bfloat16, gl=0.0005, gh=0.02)
    S = len(lens)
    S0 = rng.standard_normal((S, H, Dk, Dv)) * 0.3
    dF = rng.standard_normal((S, H, Dk, Dv)) * 0.3
    r = _run(ts, cu, Dk ** -0.5, S0, dF)
    ref = _oracle(ts, cu, Dk ** -0.5, S0, dF)
    _compare(r, ref, "bf16", "cut pieces")
    for i in range(S):
        a, e = cu[i], cu[i + 1]
        for name, got, exp in zip(["dq", "dk", "dv", "dg"], r[:4], ref[:4]):
            check_close(f64(got)[0, a:e], exp[a:e], "bf16", f"segment {i} {name}")


# The reverse-mode oracle keeps every state of a segment (Dk x Dv fp64 per
# token): 6.8 GB per head for long_context's 53274-token document, so there it
# runs on every segment of one head in four, on half the processes.
@pytest.mark.parametrize("name,head_step,procs", [("flat_microbatch", 1, None),
                                                  ("many_short_docs", 1, None),
                                                  ("long_context", 4, 8)])
def test_full_size_every_pair(name, head_step, procs):
    """Every gradient of every (segment, head) pair (long_context: every
    segment of every fourth head) against the oracle's reverse mode, with a
    final-state cotangent on every slot; rel-L2 per gradient over the whole
    tensor and per segment, and zero gradients past cu[max_segs]."""
    pkv = _pkv()
    print(f"  bwd {name}: building inputs", flush=True)
    wl = workloads.make_workload(name, conv=False)
    cu, _, _ = oracle.segment_ids_to_cu_seqlens(wl.segment_ids, wl.cfg.max_segs)
    N, H, Dk, Dv = wl.N, wl.cfg.H, wl.cfg.Dk, wl.cfg.Dv
    gen = torch.Generator().manual_seed(11)
    do = torch.randn((N, H, Dv), generator=gen).to(torch.bfloat16)
    S = len(cu) - 1
    dF = torch.randn((S, H, Dk, Dv), generator=gen) * 0.05
    dev = device()
    args = [t.reshape(1, N, H, -1).to(dev) for t in (wl.q, wl.k, wl.v, wl.g)]
    beta = wl.beta.reshape(1, N, H).to(dev)
    cud = torch.from_numpy(cu.astype(np.int32)).to(dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    print(f"  bwd {name}: launch", flush=True)
    r = pkv.chunk_kda_varlen_backward(*args, beta, do.reshape(1, N, H, Dv).to(dev), cud,
                                      dfinal_state=dF.to(dev), output_d_initial_state=True, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    for t in r[:5]:
        assert torch.count_nonzero(t[0, int(cu[-1]):]).item() == 0
    heads = list(range(0, H, head_step))
    with fullsize.Store() as st:
        for n, t in zip(("q", "k", "v", "g", "beta", "do"), (wl.q, wl.k, wl.v, wl.g, wl.beta, do)):
            st.put(n, t)
        st.put("dF", dF.numpy().astype(np.float64))
        for n, t in zip(("dq", "dk", "dv", "dg", "dbeta"), r[:5]):
            st.put(n, t[0])
        st.put("dS0", r.d_initial_state)
        del r
        print(f"  bwd {name}: oracle over {S} slots x {len(heads)} heads", flush=True)
        summ = fullsize.summarize(fullsize.run_pairs(fullsize._bwd_job, st.paths, H, cu, heads=heads,
                                                     nproc=procs))
    real = int(np.sum(np.diff(cu) > 0))
    for n, x in summ.items():
        print(f"  bwd {name} {n}: rel-L2 {x['rel_l2']:.3e} (worst segment {x['worst_segment_rel_l2']:.3e}), "
              f"max abs err {x['max_abs']:.3e} of max |ref| {x['max_ref']:.3e}, {x['pairs']} pairs", flush=True)
        assert x["finite"], n
        assert x["pairs"] == real * len(heads), n
        assert x["rel_l2"] <= 2e-2 and x["worst_segment_rel_l2"] <= 2e-2, n


def test_bad_cu_seqlens_sets_flag_chunked():
    """The chunked path (bf16, D = 64): a decreasing cu_seqlens entry sets the flag; the
    plan keeps every index inside the workspace (overlapping slots only race)."""
    print("  bwd bad cu_seqlens (chunked)", flush=True)
    rng = np.random.default_rng(4)
    N, H, D = 64, 2, 64
    ts = _inputs(rng, N, H, D, D, torch.bfloat16)
    flags = torch.zeros(1, dtype=torch.int32, device=device())
    _run(ts, np.array([0, 40, 30, 64]), 1.0, None, None, flags=flags, want_dinit=True)
    assert int(flags.item()) & _pkv().FLAG_BAD_CU_SEQLENS


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 128)])
def test_backward_deterministic(Dk, Dv):
    """No atomics on the data path: two calls give the same bits."""
    print(f"  bwd determinism Dk={Dk} Dv={Dv}", flush=True)
    rng = np.random.default_rng(9)
    cu = np.array(CU_RAGGED, dtype=np.int64)
    N, H = 345, 3
    ts = _inputs(rng, N, H, Dk, Dv, torch.bfloat16)
    S = len(cu) - 1
    dF = rng.standard_normal((S, H, Dk, Dv))
    r1 = _run(ts, cu, 0.5, None, dF)
    r2 = _run(ts, cu, 0.5, None, dF)
    for a, b in zip(r1, r2):
        assert torch.equal(a.cpu(), b.cpu())


# ---- the forward call that keeps the state before every chunk, and the reverse
# pass that reads those states instead of recomputing them

def _oracle_prefix_state(ts, cu, i, c, S0):
    """The oracle's state of segment i after its first 64 c tokens (the state
    before its chunk c), [H, Dk, Dv]."""
    q, k, v, g, beta, _ = [f64(t)[0] for t in ts]
    a = int(cu[i])
    e = a + 64 * c
    init = None if S0 is None else S0[i:i + 1]
    _, fs = oracle.chunk_kda_varlen(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], [0, e - a], 1.0, init)
    return fs[0]


def _saved_states_case(ts, cu, scale, S0, dF, what, check_states=True):
    pkv = _pkv()
    dev = device()
    q, k, v, g, beta, do = [t.to(dev) for t in ts]
    N, H, Dk, Dv = q.shape[1], q.shape[2], q.shape[3], v.shape[3]
    S = len(cu) - 1
    cud = torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(dev)
    s0 = None if S0 is None else torch.from_numpy(S0).float().to(dev)
    df = None if dF is None else torch.from_numpy(dF).float().to(dev)
    o0, f0 = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, scale=scale, initial_state=s0)
    st = pkv.new_chunk_states(N, H, Dk, Dv, S, dev)
    o1, f1 = pkv.chunk_kda_varlen(q, k, v, g, beta, cud, scale=scale, initial_state=s0, chunk_states=st)
    torch.cuda.synchronize()
    # the outputs do not depend on whether the states are kept
    assert torch.equal(o0, o1) and torch.equal(f0, f1), what
    if check_states:
        sv = st.view(torch.bfloat16).view(-1, H, Dk, Dv)
        nch = [int((cu[i + 1] - cu[i] + 63) // 64) for i in range(S)]
        b = np.concatenate([[0], np.cumsum(nch)]).astype(np.int64)
        for i in range(S):
            for c in range(nch[i]):
                if c == 0 and S0 is None:
                    continue  # zero, not stored
                check_close(f64(sv[b[i] + c]), _oracle_prefix_state(ts, cu, i, c, S0), "bf16",
                            f"{what} state slot {i} chunk {c}")
    r = pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, cud, scale=scale, initial_state=s0,
                                      dfinal_state=df, output_d_initial_state=True, chunk_states=st)
    r0 = pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, cud, scale=scale, initial_state=s0,
                                       dfinal_state=df, output_d_initial_state=True)
    torch.cuda.synchronize()
    ref = _oracle(ts, cu, scale, S0, dF)
    _compare(r, ref, "bf16", f"{what} from saved states")
    # and close to the reverse pass that recomputes the states (both round them to bf16)
    for name, a_, b_ in zip(["dq", "dk", "dv", "dg", "dbeta", "dinit"], r, r0):
        a64, b64 = f64(a_), f64(b_)
        rel = np.linalg.norm(a64 - b64) / max(np.linalg.norm(b64), 1e-30)
        print(f"    {what} {name}: saved vs recomputed rel-L2 {rel:.2e}", flush=True)
        assert rel <= 1e-2, (what, name, rel)


@pytest.mark.parametrize("Dk,Dv,with_s0,with_dF", [(128, 128, False, True), (64, 64, True, True),
                                                   (128, 64, True, False), (64, 128, False, False)])
def test_saved_chunk_states(Dk, Dv, with_s0, with_dF):
    """pkv_chunk_kda_varlen_states gives o and final states bit-identical to the
    plain call, every stored state matches the oracle's state at that chunk
    boundary (layout: entry b_i + c, rows d, columns e), and the reverse pass that
    reads them matches the oracle's reverse mode and the recomputing pass; ragged
    segments, single tokens and an empty slot."""
    print(f"  saved states Dk={Dk} Dv={Dv} s0={with_s0} dF={with_dF}", flush=True)
    rng = np.random.default_rng(100 + Dk + Dv + 2 * with_s0 + with_dF)
    N, H = 345, 2
    cu = np.array(CU_RAGGED, dtype=np.int64)
    ts = _inputs(rng, N, H, Dk, Dv, torch.bfloat16)
    S = len(cu) - 1
    S0 = rng.standard_normal((S, H, Dk, Dv)) * 0.5 if with_s0 else None
    dF = rng.standard_normal((S, H, Dk, Dv)) * 0.5 if with_dF else None
    _saved_states_case(ts, cu, Dk ** -0.5, S0, dF, f"{Dk}x{Dv}")


@pytest.mark.parametrize("lens,Dk,Dv", [((70, 20000, 33), 64, 64), ((8300,), 128, 128)])
def test_saved_chunk_states_cut_segments(lens, Dk, Dv):
    """Documents long enough that the forward pass cuts them into runs (each run
    after the first starts from a composed state) and the reverse pass into
    pieces; initial states and a final-state cotangent on every slot."""
    print(f"  saved states cut lens={lens} Dk={Dk} Dv={Dv}", flush=True)
    rng = np.random.default_rng(sum(lens) + 3 * Dk)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N, H = int(cu[-1]), 1
    ts = _inputs(rng, N, H, Dk, Dv, torch.bfloat16, gl=0.0005, gh=0.02)
    S = len(lens)
    S0 = rng.standard_normal((S, H, Dk, Dv)) * 0.3
    dF = rng.standard_normal((S, H, Dk, Dv)) * 0.3
    _saved_states_case(ts, cu, Dk ** -0.5, S0, dF, f"cut {lens}", check_states=False)
