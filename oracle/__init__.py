"""Oracle: plain, slow, fp64 CPU implementations of the packed varlen KDA path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links
this package. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it. It shares no code with the HIP
library under ``packed_varlen_gated_amd/`` and imports nothing from it.

Sources (the pages; cited by title and section):

* RFC-0025 "Support attention varlen and align loss" (wiki-b2l, rfc/0025),
  Design section 1 "segment_ids -> cu_seqlens conversion" and section 3
  "ShortConvolution segment boundary mask".
* RFC-0026 "Ling3 KDA varlen support" (wiki-b2l, rfc/0026), Background
  "KDA state leakage problem" (the recurrence) and section 3.1.1 "API
  contract" (reset semantics).
* "Drill: Sequence Packing from scratch" (ac.fzhiy.net), section "The math"
  (cu_seqlens, doc(s), block-diagonal mask).
* RFC-0025, Design section 6 (data pipeline alignment: EOD segmentation,
  positions, loss mask).
* RFC-0026, section 3.3 (the wrapper's ``initial_state`` and
  ``use_qk_l2norm_in_kernel``; the norm's place in the module is RFC-0025
  Design section 5), section 3.1.1's
  [B, T] ``segment_ids`` contract (reset where the id changes or a row starts)
  and section 3.4 (padding id 0, which the kernel ignores).

Functions and their pin status (every function is pinned; see tests/):

==================================  =========================================
``segment_ids_to_cu_seqlens``       pinned: printed examples, page algorithm
                                    on its own domain, construction from
                                    document lengths, hand-derived deviations
``token_segment``                   pinned: brute force of the doc(s) definition
``short_conv_segmask``              pinned: numpy.convolve per channel, single
                                    tap closed form, hand-computed fixture
``chunk_kda_varlen``                pinned: unrolled closed form, g=0 masked
                                    matmul, geometric series, single-token
                                    segments, gate injection, invariants;
                                    initial states: decayed closed form,
                                    split-and-resume identity
``l2_normalize`` (the
``use_qk_l2norm`` option of the
two recurrences above)              pinned: a hand-computed single token,
                                    invariance to positive per-(token, head)
                                    scales of q and k, unit-norm inputs
                                    unchanged, v not normalised
``chunk_kda_varlen_backward``       pinned: central finite differences of a
                                    random linear loss for every input
                                    (q, k, v, g, beta, initial state)
``chunk_kda_segment_ids``           pinned: gate injection (g = -inf at each
                                    segment start, RFC-0026 Alternatives) on
                                    the row's real positions, trailing padding
                                    cut off gives the same bits, hand-derived
                                    four-row case (padding before, between,
                                    after and instead of documents)
``eod_to_segment_ids``              pinned: hand-derived rows, construction
                                    from document lengths
==================================  =========================================
"""

from .cu_seqlens import segment_ids_to_cu_seqlens, token_segment, FLAG_OVERFLOW, FLAG_LEADING_PAD
from .short_conv import short_conv_segmask
from .kda import chunk_kda_varlen, chunk_kda_segment_ids, chunk_kda_varlen_backward, l2_normalize
from .eod import eod_to_segment_ids

__all__ = [
    "segment_ids_to_cu_seqlens",
    "token_segment",
    "short_conv_segmask",
    "chunk_kda_varlen",
    "chunk_kda_segment_ids",
    "chunk_kda_varlen_backward",
    "l2_normalize",
    "eod_to_segment_ids",
    "FLAG_OVERFLOW",
    "FLAG_LEADING_PAD",
]
