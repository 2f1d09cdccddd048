"""Pins for the oracle's segment-masked short causal convolution."""

import numpy as np
import pytest

import oracle
from conftest import read_golden, parse_ints


@pytest.mark.parametrize("row", read_golden("short_conv_cases.txt"))
def test_hand_computed_cases(row):
    x = np.array(parse_ints(row[0]), dtype=np.float64)[None, :, None]
    seg = np.array([parse_ints(row[1])], dtype=np.int32)
    w = np.array(parse_ints(row[2]), dtype=np.float64)[None, :]
    y = oracle.short_conv_segmask(x, w, seg)
    assert y[0, :, 0].tolist() == [float(t) for t in parse_ints(row[3])]


def test_one_document_per_row_is_plain_causal_conv():
    # With a single segment per row the mask never fires: numpy.convolve per
    # channel (full convolution truncated to the first T outputs).
    rng = np.random.default_rng(0)
    B, T, F, Kc = 3, 37, 5, 4
    x = rng.standard_normal((B, T, F))
    w = rng.standard_normal((F, Kc))
    seg = np.ones((B, T), dtype=np.int32)
    for s in (seg, None):
        y = oracle.short_conv_segmask(x, w, s)
        for b in range(B):
            for f in range(F):
                ref = np.convolve(x[b, :, f], w[f])[:T]
                np.testing.assert_allclose(y[b, :, f], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("tap", [0, 1, 3])
def test_single_tap_closed_form(tap):
    rng = np.random.default_rng(1)
    B, T, F, Kc = 2, 30, 3, 4
    x = rng.standard_normal((B, T, F))
    w = np.zeros((F, Kc))
    w[:, tap] = rng.standard_normal(F)
    seg = np.array([[1] * 7 + [2] * 3 + [3] * 15 + [0] * 5, [1] * 30], dtype=np.int32)
    y = oracle.short_conv_segmask(x, w, seg)
    for b in range(B):
        for t in range(T):
            src = t - tap
            same = src >= 0 and seg[b, src] == seg[b, t]
            ref = w[:, tap] * x[b, src] if same else np.zeros(F)
            assert np.array_equal(y[b, t], ref)


def test_no_leak_across_documents():
    rng = np.random.default_rng(2)
    B, T, F, Kc = 1, 40, 4, 4
    x = rng.standard_normal((B, T, F))
    w = rng.standard_normal((F, Kc))
    seg = np.array([[1] * 12 + [2] * 20 + [3] * 8], dtype=np.int32)
    y = oracle.short_conv_segmask(x, w, seg)
    x2 = x.copy()
    x2[0, 12:32] += 5.0       # perturb document 2 only
    y2 = oracle.short_conv_segmask(x2, w, seg)
    assert np.array_equal(y[0, :12], y2[0, :12]) and np.array_equal(y[0, 32:], y2[0, 32:])
    assert not np.allclose(y[0, 12:32], y2[0, 12:32])
