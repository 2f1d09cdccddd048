"""Pins of the EOD -> segment ids / positions / loss ids oracle (RFC-0025
"Support attention varlen and align loss", Design section 6, data pipeline
alignment)."""

import numpy as np
import pytest

import oracle
from conftest import read_golden, parse_rows


@pytest.mark.parametrize("row", read_golden("eod_cases.txt"))
def test_hand_derived_cases(row):
    tokens, eod, seg, pos, loss = row
    x = np.array(parse_rows(tokens))
    got = oracle.eod_to_segment_ids(x, int(eod))
    for g, want in zip(got, (seg, pos, loss)):
        assert g.tolist() == parse_rows(want)


def test_construction_from_document_lengths():
    """Rows built by concatenating documents that each end with the EOD token:
    the document index is the segment id, the index inside the document the
    position, and only the closing EOD positions carry loss id 0."""
    rng = np.random.default_rng(7)
    eod = 0
    for _ in range(50):
        B = int(rng.integers(1, 4))
        T = int(rng.integers(1, 300))
        tokens = np.zeros((B, T), dtype=np.int64)
        seg = np.zeros((B, T), dtype=np.int64)
        pos = np.zeros((B, T), dtype=np.int64)
        loss = np.zeros((B, T), dtype=np.int64)
        for b in range(B):
            t, d = 0, 1
            while t < T:
                n = int(rng.integers(1, 40))          # document length with its EOD
                body = rng.integers(1, 1000, size=n)  # non-EOD tokens
                body[-1] = eod                       # the EOD closes the document
                for j in range(n):
                    if t >= T:
                        break                        # the row cuts the last document
                    tokens[b, t] = body[j]
                    seg[b, t] = d
                    pos[b, t] = j
                    loss[b, t] = 0 if j == n - 1 else d
                    t += 1
                d += 1
        got = oracle.eod_to_segment_ids(tokens, eod)
        assert np.array_equal(got[0], seg)
        assert np.array_equal(got[1], pos)
        assert np.array_equal(got[2], loss)


def test_feeds_cu_seqlens_with_ends_after_each_eod():
    """The ids are a valid segment_ids input: cu_seqlens then ends each segment
    one past an EOD (or at the row end), and no slot is padding."""
    x = np.array([[3, 0, 4, 4, 0, 5], [0, 1, 1, 1, 1, 1]])
    seg, _, _ = oracle.eod_to_segment_ids(x, 0)
    cu, n, flags = oracle.segment_ids_to_cu_seqlens(seg, 8)
    assert list(cu) == [0, 2, 5, 6, 7, 12, 12, 12, 12]
    assert (n, flags) == (5, 0)
