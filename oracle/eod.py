"""Oracle for EOD-separated token rows -> segment ids, positions and loss ids.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

RFC-0025 "Support attention varlen and align loss", Design section 6 (data
pipeline alignment), states what the pipeline derives from a packed token row whose documents are
separated by an EOD token:

* input segmentation: an EOD token keeps the id of the document it ends, and
  a new segment starts right after it;
* target segmentation (the loss mask): positions whose input is the EOD
  token get 0, so they carry no loss;
* input positions restart at 0 after an EOD.

Readings (listed in the design doc): ids start at 1 in every row (rows are
independent samples), so seg[b, t] = 1 + (number of EODs in row b before t);
pos[b, t] = t - s, with s one past the last EOD before t in the row (0 if
none); loss[b, t] = 0 where tokens[b, t] == eod_id, else seg[b, t]. There is no
padding: every position of a packed sample is a real token.

Plain per-position loops, written from those three statements.
"""

import numpy as np


def eod_to_segment_ids(tokens, eod_id):
    """tokens: int [B, T] -> (segment_ids, positions, loss_segment_ids), int32 [B, T]."""
    x = np.asarray(tokens)
    if x.ndim != 2:
        raise ValueError(f"tokens has shape {x.shape}")
    B, T = x.shape
    seg = np.zeros((B, T), dtype=np.int32)
    pos = np.zeros((B, T), dtype=np.int32)
    loss = np.zeros((B, T), dtype=np.int32)
    for b in range(B):
        current = 1       # id of the document the next token belongs to
        doc_start = 0     # position where that document started
        for t in range(T):
            seg[b, t] = current
            pos[b, t] = t - doc_start
            is_eod = int(x[b, t]) == int(eod_id)
            loss[b, t] = 0 if is_eod else current
            if is_eod:    # the EOD closes its document; the next token opens one
                current += 1
                doc_start = t + 1
    return seg, pos, loss
