"""Pins for the oracle's segment_ids -> cu_seqlens conversion and doc(p).

Each pin is independent of the oracle's code: printed page examples, the
page's own listing on the domain where the readings do not matter, a
construction from document lengths, hand-derived cases and brute force of
the doc(s) definition.
"""

import numpy as np
import pytest

import oracle
from conftest import read_golden, parse_ints, parse_rows

import workloads


@pytest.mark.parametrize("row", read_golden("cu_seqlens_examples.txt"))
def test_printed_examples(row):
    # RFC-0025 Design section 1, docstring examples.
    seg = np.array([parse_ints(row[0])], dtype=np.int32)
    cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, int(row[1]))
    assert cu.tolist() == parse_ints(row[2])
    assert flags == 0


@pytest.mark.parametrize("row", read_golden("cu_seqlens_cases.txt"))
def test_hand_derived_cases(row):
    seg = np.array(parse_rows(row[0]), dtype=np.int32)
    cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, int(row[1]))
    assert cu.tolist() == parse_ints(row[2])
    assert n == int(row[3])
    assert flags == int(row[4])


def _page_listing(flat, max_segs):
    """RFC-0025 Design section 1 as the page's listing states it (no row-start
    rule, last end = count of non-padding tokens), restated with numpy."""
    BT = flat.shape[0]
    is_b = np.concatenate([[True], flat[1:] != flat[:-1]]) & (flat != 0)
    seg_idx = np.cumsum(is_b)
    n_segs = int(is_b.sum())
    n_real = int((flat != 0).sum())
    query = np.arange(1, max_segs + 1)
    starts = np.searchsorted(seg_idx, query, side="left")
    ends_from_starts = np.concatenate([starts[1:], [BT]])
    ends = np.where(query < n_segs, ends_from_starts, n_real)
    return np.concatenate([[0], ends])


def test_agrees_with_page_listing_on_its_domain():
    # Where all padding is trailing in flattened order and no row starts with
    # the previous row's last id, the readings change nothing.
    rng = np.random.default_rng(123)
    checked = 0
    for _ in range(400):
        B = int(rng.integers(1, 5))
        T = int(rng.integers(1, 40))
        seg = workloads.random_segment_ids(rng, B, T, max_len=int(rng.integers(1, 12)))
        flat = seg.reshape(-1)
        # trailing padding on the flattened buffer only
        if rng.random() < 0.5:
            cut = int(rng.integers(0, flat.size + 1))
            flat = flat.copy()
            flat[cut:] = 0
            seg = flat.reshape(B, T)
        collide = any(seg[b, -1] != 0 and seg[b, -1] == seg[b + 1, 0] for b in range(B - 1))
        if collide:
            continue
        if B > 1 and any((seg[b] == 0).any() for b in range(B - 1)) and (seg[-1] != 0).any():
            continue
        max_segs = int(rng.integers(1, 20))
        cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, max_segs)
        assert cu.tolist() == _page_listing(seg.reshape(-1), max_segs).tolist(), seg
        checked += 1
    assert checked > 150


def _expected_from_docs(docs, B, T, max_segs):
    """cu_seqlens from the documents themselves (Drill "The math": cu[i] is the
    running sum of segment lengths), where a segment runs from its document's
    first token to the next document's first token and the last one ends at
    its last real token."""
    starts = [d[0] * T + d[1] for d in docs]
    n = len(starts)
    assert n <= max_segs
    if n == 0:
        return [0] * (max_segs + 1)
    last_end = starts[-1] + docs[-1][2]
    lengths = [starts[i + 1] - starts[i] for i in range(n - 1)] + [last_end - starts[-1]]
    lengths[0] += starts[0]          # cu[0] = 0: anything before the first document joins segment 0
    cu = [0]
    for L in lengths:
        cu.append(cu[-1] + L)
    cu += [cu[-1]] * (max_segs - n)
    return cu


def test_construction_from_document_lengths():
    rng = np.random.default_rng(7)
    for trial in range(300):
        B = int(rng.integers(1, 5))
        T = int(rng.integers(2, 50))
        docs = []
        seg = np.zeros((B, T), dtype=np.int32)
        for b in range(B):
            pos = int(rng.integers(0, 4)) if rng.random() < 0.3 else 0   # leading padding
            nid = 0
            while pos < T:
                L = int(min(T - pos, rng.integers(1, 10)))
                nid += 1
                docs.append((b, pos, L))
                seg[b, pos:pos + L] = nid
                pos += L
                if rng.random() < 0.3:
                    pos += int(rng.integers(1, 5))                        # padding gap
        max_segs = len(docs) + int(rng.integers(0, 5))
        if max_segs == 0:
            max_segs = 1
        cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, max_segs)
        assert n == len(docs)
        assert cu.tolist() == _expected_from_docs(docs, B, T, max_segs), (seg, docs)
        lead = len(docs) > 0 and (docs[0][0] != 0 or docs[0][1] != 0)
        assert flags == (2 if lead else 0)


def test_workload_documents_match():
    for name in workloads.CONFIGS:
        wl = workloads.make_workload(name, tensors=False)
        cfg = wl.cfg
        cu, n, flags = oracle.segment_ids_to_cu_seqlens(wl.segment_ids, cfg.max_segs)
        docs = [(d.row, d.start, d.length) for d in wl.docs]
        assert n == len(docs)
        assert flags == 0
        assert cu.tolist() == _expected_from_docs(docs, cfg.B, cfg.T, cfg.max_segs)


def test_overflow_merges_into_last_slot():
    # More documents than slots: the last slot ends at B*T (page behaviour),
    # flag bit 0 reports it.
    seg = np.array([[1, 1, 2, 3, 3, 4, 5, 0]], dtype=np.int32)
    cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, 3)
    assert cu.tolist() == [0, 2, 3, 8]
    assert n == 5 and flags == oracle.FLAG_OVERFLOW


def test_shape_and_monotone_invariants():
    rng = np.random.default_rng(5)
    for _ in range(200):
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 30))
        seg = workloads.random_segment_ids(rng, B, T, 6, pad_prob=0.4, lead_pad=True, mid_pad=True)
        max_segs = int(rng.integers(1, 12))
        cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, max_segs)
        assert cu.shape == (max_segs + 1,)
        assert cu[0] == 0 and np.all(np.diff(cu) >= 0) and cu[-1] <= B * T


def test_token_segment_brute_force():
    # "Drill: Sequence Packing", The math: doc(s) = i iff cu[i] <= s < cu[i+1].
    rng = np.random.default_rng(11)
    for _ in range(200):
        B, T = int(rng.integers(1, 4)), int(rng.integers(1, 30))
        seg = workloads.random_segment_ids(rng, B, T, 6, pad_prob=0.4, lead_pad=True, mid_pad=True)
        max_segs = int(rng.integers(1, 12))
        cu, _, _ = oracle.segment_ids_to_cu_seqlens(seg, max_segs)
        N = B * T
        got = oracle.token_segment(cu, N)
        for s in range(N):
            hits = [i for i in range(max_segs) if cu[i] <= s < cu[i + 1]]
            assert len(hits) <= 1
            assert got[s] == (hits[0] if hits else -1)
