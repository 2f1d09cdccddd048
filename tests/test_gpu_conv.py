"""GPU parity of pkv_short_conv_segmask against the oracle (element-wise bound)."""

import numpy as np
import pytest
import torch

import workloads
from parity import check_conv, f64

pytestmark = pytest.mark.gpu


def _run(x, w, seg):
    import packed_varlen_gated_amd as pkv
    segd = None if seg is None else torch.from_numpy(np.ascontiguousarray(seg, dtype=np.int32)).cuda()
    y = pkv.short_conv_segmask(x.cuda(), w.cuda(), segd)
    torch.cuda.synchronize()
    return y.cpu()


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_midpad", "ling3_tiny_sample"])
def test_workloads(name):
    wl = workloads.make_workload(name)
    y = _run(wl.conv_x, wl.conv_w, wl.segment_ids)
    check_conv(f64(y), f64(wl.conv_x), f64(wl.conv_w), wl.segment_ids, wl.cfg.dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("Kc", [1, 2, 3, 4, 5, 8])
@pytest.mark.parametrize("F", [8, 13, 64, 2056])
def test_shapes(dtype, Kc, F):
    rng = np.random.default_rng(Kc * 1000 + F)
    B, T = 3, 77
    seg = workloads.random_segment_ids(rng, B, T, 20, pad_prob=0.5, mid_pad=True)
    x = torch.from_numpy(rng.standard_normal((B, T, F))).to(dtype)
    w = torch.from_numpy(rng.standard_normal((F, Kc))).float()
    for s in (seg, None):
        y = _run(x, w, s)
        check_conv(f64(y), f64(x), f64(w), s, "bf16" if dtype == torch.bfloat16 else "f32")


def test_masked_taps_contribute_nothing():
    rng = np.random.default_rng(3)
    B, T, F = 1, 96, 64
    seg = np.array([[1] * 30 + [2] * 40 + [0] * 6 + [3] * 20], dtype=np.int32)
    x = torch.from_numpy(rng.standard_normal((B, T, F))).float()
    w = torch.from_numpy(rng.standard_normal((F, 4))).float()
    y = _run(x, w, seg)
    x2 = x.clone()
    x2[0, 30:70] = 1e30          # huge values in document 2 only
    y2 = _run(x2, w, seg)
    keep = np.r_[0:30, 70:96]
    assert torch.equal(y[0, keep], y2[0, keep])
