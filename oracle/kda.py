"""Oracle for the packed (varlen) gated linear-attention recurrence of KDA.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

RFC-0026, Background ("KDA state leakage problem"), gives the state update

    S'_t = S_{t-1} * exp(g_t)
    S_t  = S'_t + beta_t * k_t (outer) v_t

and section 3.1.1 ("API contract") says the state is cleared where the segment
changes. Section 3.3's wrapper also takes an optional ``initial_state``; with
cu_seqlens it is read as one state per segment slot, [max_segs, H, Dk, Dv],
from which that segment's recurrence starts instead of zero (an empty slot
then keeps it as its final state). Readings (listed in the design doc): g_t has one entry per key channel, so
exp(g_t) scales the key (row) axis of the [Dk, Dv] state, i.e.
S_t = diag(exp g_t) S_{t-1} + beta_t k_t v_t^T; the readout is taken after the
update, o_t = scale * S_t^T q_t; segments come from cu_seqlens (FLA
convention, segment i = [cu[i], cu[i+1])); zero-length (phantom) segments
have a zero final state; positions at or beyond cu[max_segs] get o = 0;
cu_seqlens = None means one segment [0, N).

The chunked GPU method reaches this result up to rounding order, so the
oracle is the plain definition: the token-by-token recurrence in float64.
"""

import numpy as np

# Added to the squared norm so a zero row stays finite (the pages give no value).
L2NORM_EPS = 1e-6


def l2_normalize(x):
    """x / sqrt(sum over the last (head) axis of x^2 + L2NORM_EPS), per row.

    RFC-0026 section 3.3's kernel wrappers carry ``use_qk_l2norm_in_kernel``:
    the L2 normalisation of q and k over the head dimension, which RFC-0025
    Design section 5 places between the short conv and the kernel, is then done
    by the kernel itself.
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + L2NORM_EPS)


def _as_thd(a, name, ndim):
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == ndim + 1 and a.shape[0] == 1:
        a = a[0]
    if a.ndim != ndim:
        raise ValueError(f"{name} has shape {a.shape}")
    return a


def chunk_kda_varlen(q, k, v, g, beta, cu_seqlens=None, scale=1.0, initial_state=None,
                     use_qk_l2norm=False):
    """Return ``(o [N, H, Dv], final_state [max_segs, H, Dk, Dv])`` in float64.

    q, k, g: [N, H, Dk] (a leading unit batch axis is accepted);
    v: [N, H, Dv]; beta: [N, H]; cu_seqlens: int [max_segs + 1] or None;
    initial_state: [max_segs, H, Dk, Dv] or None (zeros); use_qk_l2norm: q and
    k are first L2-normalised per (token, head) (``l2_normalize``).
    """
    q = _as_thd(q, "q", 3)
    k = _as_thd(k, "k", 3)
    if use_qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    v = _as_thd(v, "v", 3)
    g = _as_thd(g, "g", 3)
    beta = _as_thd(beta, "beta", 2)
    N, H, Dk = q.shape
    Dv = v.shape[2]
    if cu_seqlens is None:
        cu = np.array([0, N], dtype=np.int64)
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
    max_segs = cu.shape[0] - 1
    if cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > N:
        raise ValueError("malformed cu_seqlens")

    if initial_state is not None:
        init = np.asarray(initial_state, dtype=np.float64)
        if init.shape != (max_segs, H, Dk, Dv):
            raise ValueError(f"initial_state has shape {init.shape}")
    o = np.zeros((N, H, Dv), dtype=np.float64)
    final_state = np.zeros((max_segs, H, Dk, Dv), dtype=np.float64)
    for i in range(max_segs):
        start, end = int(cu[i]), int(cu[i + 1])
        # reset at the boundary: zero, or the segment's given initial state
        S = np.zeros((H, Dk, Dv)) if initial_state is None else init[i].copy()
        if end <= start:
            final_state[i] = S  # phantom segment: no token changes the state
            continue
        for t in range(start, end):
            decay = np.exp(g[t])[:, :, None]                       # [H, Dk, 1]
            update = beta[t][:, None, None] * k[t][:, :, None] * v[t][:, None, :]
            S = decay * S + update
            # o_t[h, e] = sum_d S[h, d, e] * q_t[h, d]
            o[t] = scale * np.einsum("hde,hd->he", S, q[t])
        final_state[i] = S
    return o, final_state


def chunk_kda_segment_ids(q, k, v, g, beta, segment_ids, scale=1.0, initial_state=None,
                          use_qk_l2norm=False):
    """The [B, T] segment_ids contract of RFC-0026 section 3.1.1, row by row.

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H]; segment_ids: int
    [B, T]; initial_state: [B, H, Dk, Dv] or None. Rows never share state.
    Section 3.1.1 clears the state where segment_ids[b, t] != segment_ids[b, t - 1]
    (t = 0 always starts a segment); section 3.4 pads with id 0, which the kernel
    ignores. Read together: a padding position (id 0) leaves the state as it is
    and gets o = 0; a real position whose id differs from the previous
    position's starts a new segment from zero, except the row's first real
    position, which starts the row's first segment from initial_state[b]
    (section 3.3's per-row shape). Returns (o [B, T, H, Dv], final_state
    [B, H, Dk, Dv]): the state after each row's last real position
    (initial_state[b], or zero, for a row of padding only). use_qk_l2norm: q
    and k are first L2-normalised per (token, head) (``l2_normalize``).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if use_qk_l2norm:
        q, k = l2_normalize(q), l2_normalize(k)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    seg = np.asarray(segment_ids)
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if seg.shape != (B, T):
        raise ValueError(f"segment_ids has shape {seg.shape}")
    o = np.zeros((B, T, H, Dv), dtype=np.float64)
    final_state = np.zeros((B, H, Dk, Dv), dtype=np.float64)
    for b in range(B):
        S = np.zeros((H, Dk, Dv)) if initial_state is None else np.array(initial_state[b], dtype=np.float64)
        seen_real = False
        for t in range(T):
            if seg[b, t] == 0:
                continue  # padding: the state is untouched and o stays 0
            if seen_real and seg[b, t] != seg[b, t - 1]:
                S = np.zeros((H, Dk, Dv))  # a new segment: the state is cleared
            seen_real = True
            decay = np.exp(g[b, t])[:, :, None]
            S = decay * S + beta[b, t][:, None, None] * k[b, t][:, :, None] * v[b, t][:, None, :]
            o[b, t] = scale * np.einsum("hde,hd->he", S, q[b, t])
        final_state[b] = S
    return o, final_state


def chunk_kda_varlen_backward(q, k, v, g, beta, do, cu_seqlens=None, scale=1.0,
                              initial_state=None, dfinal_state=None):
    """Reverse mode of ``chunk_kda_varlen`` (the recurrence above), in float64.

    do: [N, H, Dv], the gradient of the loss with respect to o; dfinal_state:
    [max_segs, H, Dk, Dv] or None, with respect to the final states. Returns
    (dq, dk, dv, dg, dbeta, dinitial_state) shaped like q, k, v, g, beta and
    [max_segs, H, Dk, Dv] (zeros when there is no initial state). Positions
    outside every segment get zero gradients.

    Written from the forward step, S_t = exp(g_t) * S_{t-1} + beta_t k_t v_t^T
    (rows scaled by exp(g_t)) and o_t = scale * S_t^T q_t, by the chain rule
    taken backwards through the segment, with every S_t kept:
      dS_t   = dS (from t + 1) + scale * q_t do_t^T
      dq_t   = scale * S_t do_t
      dk_t   = beta_t * dS_t v_t,   dv_t = beta_t * dS_t^T k_t,
      dbeta_t = k_t^T dS_t v_t,     dg_t = sum_e dS_t * (exp(g_t) * S_{t-1})
      dS (for t - 1) = exp(g_t) * dS_t.
    """
    q = _as_thd(q, "q", 3)
    k = _as_thd(k, "k", 3)
    v = _as_thd(v, "v", 3)
    g = _as_thd(g, "g", 3)
    beta = _as_thd(beta, "beta", 2)
    do = _as_thd(do, "do", 3)
    N, H, Dk = q.shape
    Dv = v.shape[2]
    cu = np.array([0, N], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    max_segs = cu.shape[0] - 1
    dq, dk, dv, dg = (np.zeros_like(a) for a in (q, k, v, g))
    dbeta = np.zeros_like(beta)
    dinit = np.zeros((max_segs, H, Dk, Dv))
    for i in range(max_segs):
        start, end = int(cu[i]), int(cu[i + 1])
        S0 = np.zeros((H, Dk, Dv)) if initial_state is None else np.array(initial_state[i], dtype=np.float64)
        dS = np.zeros((H, Dk, Dv)) if dfinal_state is None else np.array(dfinal_state[i], dtype=np.float64)
        if end <= start:
            dinit[i] = dS  # an empty segment passes its initial state through
            continue
        states = [S0]  # states[j] = S after token start + j - 1
        for t in range(start, end):
            S = np.exp(g[t])[:, :, None] * states[-1] + beta[t][:, None, None] * k[t][:, :, None] * v[t][:, None, :]
            states.append(S)
        for t in range(end - 1, start - 1, -1):
            S_t, S_prev = states[t - start + 1], states[t - start]
            dS = dS + scale * q[t][:, :, None] * do[t][:, None, :]
            dq[t] = scale * np.einsum("hde,he->hd", S_t, do[t])
            u = np.einsum("hde,he->hd", dS, v[t])                 # dS_t v_t
            dk[t] = beta[t][:, None] * u
            dv[t] = beta[t][:, None] * np.einsum("hde,hd->he", dS, k[t])
            dbeta[t] = np.einsum("hd,hd->h", k[t], u)
            dg[t] = np.einsum("hde,hde->hd", dS, np.exp(g[t])[:, :, None] * S_prev)
            dS = np.exp(g[t])[:, :, None] * dS
        dinit[i] = dS
    return dq, dk, dv, dg, dbeta, dinit
