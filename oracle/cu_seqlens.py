"""Oracle for segment_ids -> cu_seqlens and the token -> segment index.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows RFC-0025, Design section 1 ("segment_ids -> cu_seqlens conversion"):
flatten the [B, T] ids, mark boundaries where the id changes and is not
padding (0), take the inclusive cumulative sum as a 1-based segment index,
find each segment's start with a left searchsorted, turn starts into ends and
fill phantom slots so the result has the fixed length max_segs + 1 in the FLA
convention [0, n1, n1 + n2, ...].

Two readings depart from the page's listing where the listing and its own
comments disagree (both are spelled out in the design doc and pinned by
hand-derived cases in tests/golden/cu_seqlens_cases.txt):

1. Every row start is a boundary when it holds a real token. RFC-0026 section
   3.1.1 states that t = 0 always starts a new segment; without this a row
   whose last id equals the next row's first id would merge two documents
   of different rows in the flattened batch.
2. The last real segment ends one past the last non-padding position
   (``e_last``), which is what the page's comment says ("end of last real
   segment"). The listing's count of non-padding tokens agrees with that only
   when all padding is trailing.

Overflow (more segments than max_segs) keeps the page's behaviour: the last
slot ends at B*T and swallows the rest; FLAG_OVERFLOW is raised, which plays
the role of the page's debug-callback warning. Padding in front of the first
real token cannot be absorbed by a preceding segment; it falls into segment 0
(cu[0] = 0) and FLAG_LEADING_PAD marks it.
"""

import numpy as np

FLAG_OVERFLOW = 1
FLAG_LEADING_PAD = 2


def segment_ids_to_cu_seqlens(segment_ids, max_segs):
    """Return ``(cu_seqlens int64[max_segs + 1], n_segs, flags)``.

    segment_ids: integer array [B, T]; 1-based document ids that restart per
    row, 0 = padding.
    """
    seg = np.asarray(segment_ids)
    if seg.ndim != 2:
        raise ValueError("segment_ids must be [B, T]")
    if max_segs < 1:
        raise ValueError("max_segs must be >= 1")
    B, T = seg.shape
    N = B * T
    flat = seg.reshape(-1).astype(np.int64)

    # Boundary detection: a real token that starts a row or whose id differs
    # from the previous position's id.
    pos = np.arange(N)
    changed = np.ones(N, dtype=bool)
    changed[1:] = flat[1:] != flat[:-1]
    row_start = (pos % T) == 0 if T > 0 else np.zeros(N, dtype=bool)
    is_boundary = (changed | row_start) & (flat != 0)

    # 1-based segment index of every position (0 before the first boundary).
    seg_idx = np.cumsum(is_boundary.astype(np.int64))
    n_segs = int(seg_idx[-1]) if N > 0 else 0

    nonzero = np.nonzero(flat != 0)[0]
    e_last = int(nonzero[-1]) + 1 if nonzero.size else 0

    # Start of the segment with 1-based index q = first position whose
    # seg_idx reaches q (N when there is none).
    query = np.arange(1, max_segs + 1, dtype=np.int64)
    starts = np.searchsorted(seg_idx, query, side="left")

    ends = np.empty(max_segs, dtype=np.int64)
    for i in range(max_segs):
        if i + 1 < n_segs:
            # Interior segment: ends where the next one starts; the last slot
            # on overflow ends at N and merges every remaining segment.
            ends[i] = starts[i + 1] if i + 1 < max_segs else N
        else:
            # Last real segment and phantom slots.
            ends[i] = e_last

    cu = np.concatenate([np.zeros(1, dtype=np.int64), ends])

    flags = 0
    if n_segs > max_segs:
        flags |= FLAG_OVERFLOW
    if N > 0 and flat[0] == 0 and e_last > 0:
        flags |= FLAG_LEADING_PAD
    return cu, n_segs, flags


def token_segment(cu_seqlens, N):
    """Segment index of every packed position, or -1 outside all segments.

    "Drill: Sequence Packing from scratch", section "The math": doc(s) = i
    exactly when cu[i] <= s < cu[i + 1]. With zero-length phantom slots the
    index is the number of slot ends cu[1..max_segs] that are <= s.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    max_segs = cu.shape[0] - 1
    out = np.full(N, -1, dtype=np.int64)
    for p in range(N):
        if p < cu[max_segs]:
            out[p] = int(np.count_nonzero(cu[1:] <= p))
    return out
