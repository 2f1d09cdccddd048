"""Pins for the oracle's packed KDA recurrence.

None of these re-types the oracle's update rule: each compares it with an
independent statement of the same result (unrolled closed form, a masked
matrix product, a geometric series, single-token algebra, gate injection) or
checks an invariant the pages require (reset, isolation, phantoms).
"""

import math

import numpy as np
import pytest

import oracle


def _rand_inputs(rng, N, H, Dk, Dv, gmax=0.5, gpos=False):
    q = rng.standard_normal((N, H, Dk))
    k = rng.standard_normal((N, H, Dk))
    v = rng.standard_normal((N, H, Dv))
    g = -rng.uniform(0.0, gmax, (N, H, Dk))
    if gpos:
        g = rng.uniform(-gmax, gmax, (N, H, Dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((N, H))))
    return q, k, v, g, beta


def _closed_form(q, k, v, g, beta, cu, scale):
    """Unrolled recurrence: with b the in-segment inclusive cumsum of g,
    o_t = scale * sum_{s<=t} beta_s (sum_i q_t[i] k_s[i] e^{b_t[i]-b_s[i]}) v_s and
    S_end = sum_s diag(e^{b_end - b_s}) beta_s k_s v_s^T."""
    N, H, Dk = q.shape
    Dv = v.shape[2]
    M = len(cu) - 1
    o = np.zeros((N, H, Dv))
    fs = np.zeros((M, H, Dk, Dv))
    for i in range(M):
        a, e = cu[i], cu[i + 1]
        if e <= a:
            continue
        for h in range(H):
            b = np.cumsum(g[a:e, h, :], axis=0)          # b[t - a] = sum_{u=a..t} g_u
            for t in range(a, e):
                acc = np.zeros(Dv)
                for s in range(a, t + 1):
                    w = sum(q[t, h, d] * k[s, h, d] * math.exp(b[t - a, d] - b[s - a, d]) for d in range(Dk))
                    acc += beta[s, h] * w * v[s, h, :]
                o[t, h] = scale * acc
            for s in range(a, e):
                fs[i, h] += np.outer(np.exp(b[e - 1 - a] - b[s - a]) * beta[s, h] * k[s, h], v[s, h])
    return o, fs


@pytest.mark.parametrize("gpos", [False, True])
def test_unrolled_closed_form(gpos):
    rng = np.random.default_rng(1)
    N, H, Dk, Dv = 40, 2, 3, 2       # Dk != Dv catches a transposed state
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv, gpos=gpos)
    cu = np.array([0, 7, 7, 19, 20, 33, 33])      # phantom slots, tail [33, 40) uncovered
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale=0.75)
    o2, fs2 = _closed_form(q, k, v, g, beta, cu, 0.75)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(fs, fs2, rtol=1e-12, atol=1e-13)
    assert np.all(o[33:] == 0)


def test_zero_gate_is_block_diagonal_masked_matmul():
    # g = 0, beta = 1: o = (M * Q K^T) V with M the block-diagonal causal mask
    # of "Drill: Sequence Packing", The math.
    rng = np.random.default_rng(2)
    N, H, Dk, Dv = 50, 3, 5, 4
    q, k, v, _, _ = _rand_inputs(rng, N, H, Dk, Dv)
    g = np.zeros((N, H, Dk))
    beta = np.ones((N, H))
    cu = np.array([0, 11, 12, 30, 45, 45])
    o, _ = oracle.chunk_kda_varlen(q, k, v, g, beta, cu)
    doc = np.full(N, -1)
    for i in range(len(cu) - 1):
        doc[cu[i]:cu[i + 1]] = i
    s = np.arange(N)
    M = (doc[:, None] == doc[None, :]) & (doc[:, None] >= 0) & (s[:, None] >= s[None, :])
    for h in range(H):
        ref = (M * (q[:, h] @ k[:, h].T)) @ v[:, h]
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-11, atol=1e-12)


def test_geometric_series():
    # Dk = Dv = 1 with constant g, k, v, beta: S_t = beta k v (1 - e^{g(t+1)}) / (1 - e^g).
    L, gval, kv, bval, qv = 57, -0.137, (0.8, -1.3), 0.6, 0.9
    q = np.full((L, 1, 1), qv)
    k = np.full((L, 1, 1), kv[0])
    v = np.full((L, 1, 1), kv[1])
    g = np.full((L, 1, 1), gval)
    beta = np.full((L, 1), bval)
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, None)
    t = np.arange(L)
    S = bval * kv[0] * kv[1] * (1 - np.exp(gval * (t + 1))) / (1 - np.exp(gval))
    np.testing.assert_allclose(o[:, 0, 0], qv * S, rtol=1e-12)
    np.testing.assert_allclose(fs[0, 0, 0, 0], S[-1], rtol=1e-12)


def test_single_token_segments():
    # segment_ids [1, 2, 3, 4] (RFC-0025 Design section 1, fourth example):
    # every segment is one token, so o_t = beta_t (q_t . k_t) v_t, S = beta k v^T.
    seg = np.array([[1, 2, 3, 4]], dtype=np.int32)
    cu, _, _ = oracle.segment_ids_to_cu_seqlens(seg, 4)
    rng = np.random.default_rng(3)
    q, k, v, g, beta = _rand_inputs(rng, 4, 2, 3, 5)
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu)
    for t in range(4):
        for h in range(2):
            np.testing.assert_allclose(o[t, h], beta[t, h] * np.dot(q[t, h], k[t, h]) * v[t, h], rtol=1e-13)
            np.testing.assert_allclose(fs[t, h], beta[t, h] * np.outer(k[t, h], v[t, h]), rtol=1e-13)


def test_hard_forgetting_leaves_only_the_current_token():
    # RFC-0026 Background recurrence with g = -50 on every channel: e^{-50} is
    # below 2e-22, so every earlier token's weight in S_t vanishes and
    # o_t = scale beta_t (q_t . k_t) v_t, S_end = beta_last k_last v_last^T, to
    # fp64 rounding (the strong-forgetting regime the chunked GPU path flags).
    rng = np.random.default_rng(8)
    N, H, Dk, Dv = 40, 2, 5, 3
    q, k, v, _, beta = _rand_inputs(rng, N, H, Dk, Dv)
    g = np.full((N, H, Dk), -50.0)
    cu = np.array([0, 17, 40])
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale=0.7)
    for t in range(N):
        for h in range(H):
            np.testing.assert_allclose(o[t, h], 0.7 * beta[t, h] * np.dot(q[t, h], k[t, h]) * v[t, h],
                                       rtol=1e-12, atol=1e-14)
    for i, t in enumerate((16, 39)):
        for h in range(H):
            np.testing.assert_allclose(fs[i, h], beta[t, h] * np.outer(k[t, h], v[t, h]), rtol=1e-12, atol=1e-14)


def test_gate_injection_equivalence():
    # RFC-0026 Alternatives, gate injection: one continuous segment with
    # g = -inf at every document's first token gives the segmented result.
    rng = np.random.default_rng(4)
    N, H, Dk, Dv = 60, 2, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    cu = np.array([0, 9, 25, 26, 60])
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu)
    g2 = g.copy()
    for i in range(1, len(cu) - 1):
        g2[cu[i]] = -np.inf
    o2, fs2 = oracle.chunk_kda_varlen(q, k, v, g2, beta, None)
    assert np.array_equal(o, o2)
    assert np.array_equal(fs[-1], fs2[0])


def test_first_token_gate_has_no_effect():
    rng = np.random.default_rng(5)
    N, H, Dk, Dv = 30, 2, 3, 3
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    cu = np.array([0, 4, 17, 30])
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu)
    g2 = g.copy()
    g2[cu[:-1]] = rng.uniform(-3, 3, g2[cu[:-1]].shape)
    o2, fs2 = oracle.chunk_kda_varlen(q, k, v, g2, beta, cu)
    assert np.array_equal(o, o2) and np.array_equal(fs, fs2)


def test_packed_equals_each_document_alone_and_no_leakage():
    # RFC-0026 Tests: packed output equals running each document on its own
    # from a zero state; perturbing one document changes no other.
    rng = np.random.default_rng(6)
    N, H, Dk, Dv = 64, 2, 4, 4
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    cu = np.array([0, 13, 40, 41, 64, 64])
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu)
    for i in range(len(cu) - 1):
        a, e = cu[i], cu[i + 1]
        if e <= a:
            assert np.all(fs[i] == 0)
            continue
        oi, fsi = oracle.chunk_kda_varlen(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], None)
        assert np.array_equal(o[a:e], oi) and np.array_equal(fs[i], fsi[0])
    # leakage: perturb document 1 only
    q2, v2, g2 = q.copy(), v.copy(), g.copy()
    q2[13:40] += 1.0
    v2[13:40] *= -2.0
    g2[13:40] -= 0.3
    o2, fs2 = oracle.chunk_kda_varlen(q2, k, v2, g2, beta, cu)
    other = np.r_[0:13, 40:64]
    assert np.array_equal(o[other], o2[other])
    assert np.array_equal(fs[[0, 2, 3]], fs2[[0, 2, 3]])
    assert not np.allclose(o[13:40], o2[13:40])


def test_linearity_and_phantoms():
    rng = np.random.default_rng(8)
    N, H, Dk, Dv = 33, 2, 3, 4
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    cu = np.array([0, 10, 10, 10, 30])
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu)
    assert np.all(fs[1] == 0) and np.all(fs[2] == 0)
    assert np.all(o[30:] == 0)
    o2, _ = oracle.chunk_kda_varlen(q, k, 2.0 * v, g, beta, cu)
    assert np.array_equal(o2, 2.0 * o)
    q3 = rng.standard_normal(q.shape)
    o3, _ = oracle.chunk_kda_varlen(q3, k, v, g, beta, cu)
    o4, _ = oracle.chunk_kda_varlen(q + q3, k, v, g, beta, cu)
    np.testing.assert_allclose(o4, o + o3, rtol=1e-12, atol=1e-12)


def test_decay_acts_on_key_axis():
    # One key channel with a strong decay and one without: only the state row
    # of the decaying key channel fades (the gate has Dk entries).
    L = 5
    q = np.zeros((L, 1, 2)); q[-1, 0] = [1.0, 0.0]
    k = np.zeros((L, 1, 2)); k[0, 0] = [1.0, 1.0]
    v = np.zeros((L, 1, 3)); v[0, 0] = [1.0, 2.0, 3.0]
    g = np.zeros((L, 1, 2)); g[:, 0, 0] = math.log(0.5)
    beta = np.ones((L, 1))
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, None)
    # row 0 decays by 0.5 per step after the first token, row 1 keeps its value
    np.testing.assert_allclose(fs[0, 0, 0], 0.5 ** (L - 1) * np.array([1.0, 2.0, 3.0]), rtol=1e-14)
    np.testing.assert_allclose(fs[0, 0, 1], np.array([1.0, 2.0, 3.0]), rtol=1e-14)
    np.testing.assert_allclose(o[-1, 0], 0.5 ** (L - 1) * np.array([1.0, 2.0, 3.0]), rtol=1e-14)


def test_initial_state_adds_its_decayed_readout():
    """RFC-0026 section 3.3's initial_state (one per segment slot): the state a
    segment starts from decays with the running product of exp(g) and is read
    out by q, on top of the zero-start result (linearity in S0):
    delta o_t = scale * (exp(sum_{u=a..t} g_u) * S0)^T q_t,
    delta final = exp(sum_{u=a..e-1} g_u) * S0 (per key channel)."""
    rng = np.random.default_rng(31)
    N, H, Dk, Dv = 23, 2, 3, 4
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    cu = np.array([0, 9, 9, 23])
    S0 = rng.standard_normal((3, H, Dk, Dv))
    scale = 0.7
    o0, f0 = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale)
    o1, f1 = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale, initial_state=S0)
    for i in range(3):
        a, e = cu[i], cu[i + 1]
        G = np.cumsum(g[a:e], axis=0)                          # [L, H, Dk]
        for t in range(a, e):
            dS = np.exp(G[t - a])[:, :, None] * S0[i]            # [H, Dk, Dv]
            want = scale * np.einsum("hd,hde->he", q[t], dS)
            np.testing.assert_allclose(o1[t] - o0[t], want, rtol=1e-10, atol=1e-12)
        decay = np.exp(G[-1]) if e > a else np.ones((H, Dk))
        np.testing.assert_allclose(f1[i] - f0[i], decay[:, :, None] * S0[i], rtol=1e-10, atol=1e-12)
    assert np.array_equal(f1[1], S0[1])  # the empty slot keeps its initial state


def test_split_and_resume_equals_whole_segment():
    """Running [a, c) as [a, b) and then [b, c) started from the first part's
    final state gives the whole segment's outputs and final state."""
    rng = np.random.default_rng(32)
    N, H, Dk, Dv = 40, 2, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    ow, fw = oracle.chunk_kda_varlen(q, k, v, g, beta, np.array([0, N]))
    for b in (1, 17, 39):
        oa, fa = oracle.chunk_kda_varlen(q[:b], k[:b], v[:b], g[:b], beta[:b], np.array([0, b]))
        ob, fb = oracle.chunk_kda_varlen(q[b:], k[b:], v[b:], g[b:], beta[b:], np.array([0, N - b]),
                                         initial_state=fa)
        np.testing.assert_allclose(np.concatenate([oa, ob]), ow, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(fb, fw, rtol=1e-12, atol=1e-12)


def test_segment_ids_contract_is_gate_injection_per_row():
    """RFC-0026 section 3.1.1's [B, T] contract with section 3.4's padding
    (id 0, ignored by the kernel) equals, row by row, one continuous run over
    the row's real positions only, with g = -inf (RFC-0026 Alternatives, gate
    injection) at every real position whose id differs from the position
    before it in the row, except the row's first real position; the run starts
    from the row's initial state. Padding positions get exactly o = 0 and the
    row's final state is the run's."""
    rng = np.random.default_rng(41)
    B, T, H, Dk, Dv = 5, 40, 2, 3, 4
    q, k, v, g, beta = [a.reshape((B, T) + a.shape[1:]) for a in _rand_inputs(rng, B * T, H, Dk, Dv)]
    seg = np.array([[1] * 10 + [2] * 5 + [0] * 3 + [3] * 22,   # padding between documents
                    [0] * 4 + [1] * 36,                        # leading padding
                    [5] * 40,                                  # one document
                    [1] * 7 + [0] * 2 + [1] * 20 + [0] * 11,   # the same id on both sides of padding
                    [0] * 40])                                 # padding only
    S0 = rng.standard_normal((B, H, Dk, Dv))
    o, fs = oracle.chunk_kda_segment_ids(q, k, v, g, beta, seg, scale=0.9, initial_state=S0)
    for b in range(B):
        real = [t for t in range(T) if seg[b, t] != 0]
        pad = [t for t in range(T) if seg[b, t] == 0]
        assert np.all(o[b, pad] == 0)
        if not real:
            assert np.array_equal(fs[b], S0[b])
            continue
        g2 = g[b, real].copy()
        for j, t in enumerate(real):
            if j > 0 and seg[b, t] != seg[b, t - 1]:
                g2[j] = -np.inf
        o2, f2 = oracle.chunk_kda_varlen(q[b, real], k[b, real], v[b, real], g2, beta[b, real], None,
                                         scale=0.9, initial_state=S0[b:b + 1])
        assert np.array_equal(o[b, real], o2)
        assert np.array_equal(fs[b], f2[0])


def test_segment_ids_trailing_padding_is_ignored():
    """A row padded with zeros to a longer length (RFC-0026 section 3.4: the
    module pads T up to a multiple of 64 with id 0) gives the unpadded row's
    outputs and final state, and zeros at the padding."""
    rng = np.random.default_rng(43)
    T0, T, H, Dk, Dv = 45, 64, 2, 3, 2
    q, k, v, g, beta = [a.reshape((1, T) + a.shape[1:]) for a in _rand_inputs(rng, T, H, Dk, Dv)]
    seg = np.array([[1] * 20 + [2] * 25 + [0] * (T - T0)])
    S0 = rng.standard_normal((1, H, Dk, Dv))
    o, fs = oracle.chunk_kda_segment_ids(q, k, v, g, beta, seg, initial_state=S0)
    o0, f0 = oracle.chunk_kda_segment_ids(q[:, :T0], k[:, :T0], v[:, :T0], g[:, :T0], beta[:, :T0],
                                          seg[:, :T0], initial_state=S0)
    assert np.array_equal(o[:, :T0], o0) and np.array_equal(fs, f0)
    assert np.all(o[:, T0:] == 0)


def test_segment_ids_contract_hand_case():
    """Dk = Dv = 1, q = k = v = beta = 1, g = 0: the state counts the tokens of
    the current segment (plus the row's initial state in its first segment);
    padding positions read 0 and change nothing."""
    seg = np.array([[1, 1, 2, 2, 2], [0, 0, 3, 3, 0], [1, 0, 1, 1, 0], [0, 0, 0, 0, 0]])
    one = np.ones((4, 5, 1, 1))
    S0 = np.array([5.0, 4.0, 5.0, 7.0]).reshape(4, 1, 1, 1)
    o, fs = oracle.chunk_kda_segment_ids(one, one, one, np.zeros((4, 5, 1, 1)), np.ones((4, 5, 1)), seg,
                                         initial_state=S0)
    assert o[0, :, 0, 0].tolist() == [6, 7, 1, 2, 3]
    assert o[1, :, 0, 0].tolist() == [0, 0, 5, 6, 0]
    assert o[2, :, 0, 0].tolist() == [6, 0, 1, 2, 0]
    assert o[3, :, 0, 0].tolist() == [0, 0, 0, 0, 0]
    assert fs[:, 0, 0, 0].tolist() == [3, 6, 2, 7]


def test_backward_matches_finite_differences():
    """Every gradient of the reverse-mode oracle against central finite
    differences of L = sum(do * o) + sum(dF * final_state), on a tiny packed
    batch with an empty slot, an initial state and a final-state cotangent."""
    rng = np.random.default_rng(51)
    N, H, Dk, Dv = 13, 2, 3, 2
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv, gmax=0.6, gpos=True)
    cu = np.array([0, 5, 5, 13])
    S0 = rng.standard_normal((3, H, Dk, Dv))
    do = rng.standard_normal((N, H, Dv))
    dF = rng.standard_normal((3, H, Dk, Dv))
    scale = 0.7

    def loss(q, k, v, g, beta, S0):
        o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale, initial_state=S0)
        return np.sum(do * o) + np.sum(dF * fs)

    grads = oracle.chunk_kda_varlen_backward(q, k, v, g, beta, do, cu, scale, initial_state=S0,
                                             dfinal_state=dF)
    args = [q, k, v, g, beta, S0]
    eps = 1e-6
    for a_idx, grad in enumerate(grads):
        x = args[a_idx]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            ap, am = list(args), list(args)
            ap[a_idx], am[a_idx] = xp, xm
            fd[idx] = (loss(*ap) - loss(*am)) / (2 * eps)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-7, err_msg=f"input {a_idx}")


def test_backward_gate_gradient_identity():
    """g enters only through b_t = cumsum(g) in exp(b_t - b_s) and exp(b_end):
    dL/db_u = q_u * dq_u - k_u * dk_u (plus sum_e dF * S_end at the segment's
    end), so dg_t is its reverse cumulative sum over the segment. The GPU
    backward computes dg this way; here the identity is checked on the oracle."""
    rng = np.random.default_rng(52)
    N, H, Dk, Dv = 30, 2, 4, 3
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    cu = np.array([0, 11, 30])
    S0 = rng.standard_normal((2, H, Dk, Dv))
    do = rng.standard_normal((N, H, Dv))
    dF = rng.standard_normal((2, H, Dk, Dv))
    _, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, initial_state=S0)
    dq, dk, _, dg, _, _ = oracle.chunk_kda_varlen_backward(q, k, v, g, beta, do, cu, initial_state=S0,
                                                           dfinal_state=dF)
    for i in range(2):
        a, e = cu[i], cu[i + 1]
        db = q[a:e] * dq[a:e] - k[a:e] * dk[a:e]
        want = np.cumsum(db[::-1], axis=0)[::-1] + np.einsum("hde,hde->hd", dF[i], fs[i])[None]
        np.testing.assert_allclose(dg[a:e], want, rtol=1e-10, atol=1e-10)


def test_qk_l2norm_hand_case():
    """One token, Dk = 2, Dv = 1, beta = 1, v = 1: q = (3, 4) and k = (0, 2)
    normalise to (0.6, 0.8) and (0, 1), so S = (0, 1)^T and o = 0.8; the
    squared norms 25 and 4 each carry eps = 1e-6."""
    q = np.array([[[3.0, 4.0]]])
    k = np.array([[[0.0, 2.0]]])
    o, fs = oracle.chunk_kda_varlen(q, k, np.ones((1, 1, 1)), np.zeros((1, 1, 2)), np.ones((1, 1)), None,
                                    use_qk_l2norm=True)
    expect = 0.8 * 5 / math.sqrt(25 + 1e-6) * 2 / math.sqrt(4 + 1e-6)
    assert o[0, 0, 0] == pytest.approx(expect, rel=1e-15)
    assert fs[0, 0, :, 0] == pytest.approx([0.0, 2 / math.sqrt(4 + 1e-6)], rel=1e-15)


def test_qk_l2norm_scale_invariance_and_unit_rows():
    """The norm is taken per (token, head) over the head dimension: positive
    per-(token, head) scales of q and k leave the result unchanged (to the
    eps term); already unit-norm q and k give the plain recurrence (to the
    same term); v is not normalised, so o scales with it."""
    rng = np.random.default_rng(61)
    N, H, Dk, Dv = 30, 3, 5, 4
    q, k, v, g, beta = _rand_inputs(rng, N, H, Dk, Dv)
    q *= 3.0
    k *= 2.0
    cu = np.array([0, 11, 11, 30])
    o, fs = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale=0.7, use_qk_l2norm=True)
    cq = rng.uniform(0.5, 3.0, (N, H, 1))
    ck = rng.uniform(0.5, 3.0, (N, H, 1))
    o2, fs2 = oracle.chunk_kda_varlen(q * cq, k * ck, v, g, beta, cu, scale=0.7, use_qk_l2norm=True)
    # eps / |x|^2 is at most about 1e-6 here: allow 1e-5 of each tensor's largest value
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-5 * np.abs(o).max())
    np.testing.assert_allclose(fs2, fs, rtol=0, atol=1e-5 * np.abs(fs).max())
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o3, fs3 = oracle.chunk_kda_varlen(qn, kn, v, g, beta, cu, scale=0.7)
    np.testing.assert_allclose(o3, o, rtol=0, atol=1e-5 * np.abs(o).max())
    np.testing.assert_allclose(fs3, fs, rtol=0, atol=1e-5 * np.abs(fs).max())
    o4, _ = oracle.chunk_kda_varlen(q, k, 2.5 * v, g, beta, cu, scale=0.7, use_qk_l2norm=True)
    np.testing.assert_allclose(o4, 2.5 * o, rtol=1e-12, atol=1e-12)
    # a normalisation over the wrong axis would not be invariant to these scales
    on, _ = oracle.chunk_kda_varlen(q, k, v, g, beta, cu, scale=0.7)
    assert np.linalg.norm(on - o) > 0.1 * np.linalg.norm(o)


def test_qk_l2norm_segment_ids_contract():
    """The [B, T] contract with the option, on scaled q and k, equals the
    contract without it on unit-norm q and k (to the eps term); padding
    positions stay 0."""
    rng = np.random.default_rng(62)
    B, T, H, Dk, Dv = 2, 20, 2, 3, 2
    q, k, v, g, beta = [a.reshape((B, T) + a.shape[1:]) for a in _rand_inputs(rng, B * T, H, Dk, Dv)]
    seg = np.array([[1] * 8 + [0] * 2 + [2] * 10, [3] * 20])
    q, k = 3 * q, 3 * k
    o, fs = oracle.chunk_kda_segment_ids(4 * q, 2 * k, v, g, beta, seg, use_qk_l2norm=True)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    o2, fs2 = oracle.chunk_kda_segment_ids(qn, kn, v, g, beta, seg)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-5 * np.abs(o).max())
    np.testing.assert_allclose(fs, fs2, rtol=0, atol=1e-5 * np.abs(fs).max())
    assert np.all(o[:, seg[0] == 0][0] == 0)
