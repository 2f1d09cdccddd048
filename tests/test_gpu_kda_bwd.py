"""GPU parity of pkv_chunk_kda_varlen_backward (the reverse pass of the packed
KDA recurrence, RFC-0026 Background and section 3.3) against the fp64 oracle's
reverse mode, which keeps every state and takes dg per step, while the kernel
recomputes the states and takes dg as a reverse running sum."""

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


def test_flat_microbatch_sampled():
    """The full-size packed batch (bf16, 65536 tokens, H = 32, D = 128): the
    oracle's reverse mode on the shortest, a middle and the longest segment,
    one head each, with a final-state cotangent."""
    print("  bwd flat_microbatch: building inputs", flush=True)
    pkv = _pkv()
    wl = workloads.make_workload("flat_microbatch")
    cu, _, _ = oracle.segment_ids_to_cu_seqlens(wl.segment_ids, wl.cfg.max_segs)
    N, H, D = wl.N, wl.cfg.H, wl.cfg.Dk
    gen = torch.Generator().manual_seed(2024)
    do = torch.randn((N, H, D), generator=gen).to(torch.bfloat16)
    S = len(cu) - 1
    dF = torch.randn((S, H, D, D), generator=gen) * 0.1
    dev = device()
    args = [t.reshape(1, N, H, -1).to(dev) for t in (wl.q, wl.k, wl.v, wl.g)]
    beta = wl.beta.reshape(1, N, H).to(dev)
    cud = torch.from_numpy(cu.astype(np.int32)).to(dev)
    dod = do.reshape(1, N, H, D).to(dev)
    dfd = dF.to(dev)
    print("  bwd flat_microbatch: launch", flush=True)
    r = pkv.chunk_kda_varlen_backward(*args, beta, dod, cud, dfinal_state=dfd)
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    pkv.chunk_kda_varlen_backward(*args, beta, dod, cud, dfinal_state=dfd)
    t1.record()
    torch.cuda.synchronize()
    print(f"  bwd flat_microbatch: {t0.elapsed_time(t1):.3f} ms", flush=True)
    lens = np.diff(cu)
    real = [i for i in range(S) if lens[i] > 0]
    picks = sorted({min(real, key=lambda i: lens[i]), real[len(real) // 2], max(real, key=lambda i: lens[i])})
    for n, i in enumerate(picks):
        a, e = int(cu[i]), int(cu[i + 1])
        h = (5 * n + 3) % H
        print(f"  oracle bwd segment {i} [{a},{e}) head {h}", flush=True)
        sl, hs = slice(a, e), slice(h, h + 1)
        ref = oracle.chunk_kda_varlen_backward(
            f64(wl.q[sl, hs]), f64(wl.k[sl, hs]), f64(wl.v[sl, hs]), f64(wl.g[sl, hs]),
            f64(wl.beta[sl, hs]), f64(do[sl, hs]), None, 1.0, None, f64(dF[i:i + 1, hs]))
        for name, got, exp in zip(["dq", "dk", "dv", "dg", "dbeta"], r[:5], ref[:5]):
            check_close(f64(got[0, sl, h]), exp[:, 0], "bf16", f"segment {i} head {h} {name}")


@pytest.mark.parametrize("lens,Dk,Dv", [((3000,), 64, 64), ((70, 5000, 33), 64, 64), ((4100,), 128, 128)])
def test_long_segments_cut_into_pieces(lens, Dk, Dv):
    """One head and long documents: the plan cuts every segment over 32 chunks into
    pieces (the per-CU share is tiny), so the state kernel composes the pieces'
    summaries; with an initial state and a final-state cotangent on every slot."""
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


def _full_size_sampled(name, pick, dF_scale=0.1):
    pkv = _pkv()
    print(f"  bwd {name}: building inputs", flush=True)
    wl = workloads.make_workload(name, conv=False)
    cu, _, _ = oracle.segment_ids_to_cu_seqlens(wl.segment_ids, wl.cfg.max_segs)
    N, H, Dk, Dv = wl.N, wl.cfg.H, wl.cfg.Dk, wl.cfg.Dv
    gen = torch.Generator().manual_seed(11)
    do = torch.randn((N, H, Dv), generator=gen).to(torch.bfloat16)
    S = len(cu) - 1
    dF = torch.randn((S, H, Dk, Dv), generator=gen) * dF_scale
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
    lens = np.diff(cu)
    for n, i in enumerate(pick(lens)):
        a, e = int(cu[i]), int(cu[i + 1])
        h = (7 * n + 5) % H
        print(f"  oracle bwd {name} segment {i} [{a},{e}) head {h}", flush=True)
        sl, hs = slice(a, e), slice(h, h + 1)
        ref = oracle.chunk_kda_varlen_backward(
            f64(wl.q[sl, hs]), f64(wl.k[sl, hs]), f64(wl.v[sl, hs]), f64(wl.g[sl, hs]),
            f64(wl.beta[sl, hs]), f64(do[sl, hs]), None, 1.0, None, f64(dF[i:i + 1, hs]))
        for nm, got, exp in zip(["dq", "dk", "dv", "dg", "dbeta"], r[:5], ref[:5]):
            check_close(f64(got[0, sl, h]), exp[:, 0], "bf16", f"{name} segment {i} head {h} {nm}")
        check_close(f64(r.d_initial_state[i, h]), ref[5][0, 0], "bf16", f"{name} segment {i} head {h} dS0")


def test_many_short_docs_sampled():
    """D = 64, hundreds of short documents, phantom slots and trailing padding."""
    def pick(lens):
        real = [i for i in range(len(lens)) if lens[i] > 0]
        return sorted({min(real, key=lambda i: lens[i]), real[len(real) // 2], max(real, key=lambda i: lens[i])})
    _full_size_sampled("many_short_docs", pick)


def test_long_context_sampled():
    """H = 32, six documents over 131072 tokens: the long ones are cut into pieces at
    full size (the per-CU share is 257 chunks); the shortest and the longest."""
    def pick(lens):
        real = [i for i in range(len(lens)) if lens[i] > 0]
        return sorted({min(real, key=lambda i: lens[i]), max(real, key=lambda i: lens[i])})
    _full_size_sampled("long_context", pick, dF_scale=0.05)


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
