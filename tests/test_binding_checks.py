"""The Python binding refuses, before any library call, an ``out`` tensor of
the wrong shape and a workspace that is not a contiguous uint8 tensor on the
call's device holding enough bytes (CPU tensors: nothing reaches a kernel)."""

import os

import pytest
import torch

import packed_varlen_gated_amd as pkv


@pytest.fixture(scope="module", autouse=True)
def built():
    if not os.path.exists(pkv.LIB_PATH):
        from packed_varlen_gated_amd import build
        build.build(verbose=False)


def _kda(N=256, H=2, D=64, dtype=torch.bfloat16):
    q, k, g = (torch.zeros(1, N, H, D, dtype=dtype) for _ in range(3))
    v = torch.zeros(1, N, H, D, dtype=dtype)
    beta = torch.zeros(1, N, H, dtype=dtype)
    return q, k, v, g, beta


def test_chunk_kda_out_shape():
    q, k, v, g, beta = _kda()
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.chunk_kda_varlen(q, k, v, g, beta, out=torch.empty(1, 255, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.chunk_kda_varlen(q, k, v, g, beta, out=torch.empty(1, 256, 2, 32, dtype=torch.bfloat16))


def test_segment_ids_out_shape():
    q, k, v, g, beta = (t.view(2, 128, *t.shape[2:]) for t in _kda())
    seg = torch.ones(2, 128, dtype=torch.int32)
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.chunk_kda_segment_ids(q, k, v, g, beta, seg, out=torch.empty(2, 128, 2, 128, dtype=torch.bfloat16))


def test_short_conv_out_shape():
    x = torch.zeros(2, 16, 32)
    w = torch.zeros(32, 4)
    with pytest.raises(ValueError, match="out must have shape"):
        pkv.short_conv_segmask(x, w, out=torch.empty(2, 16, 31))


@pytest.mark.parametrize("bad,err", [
    (lambda n: torch.empty(n, dtype=torch.float32), TypeError),           # not uint8
    (lambda n: torch.empty(n, dtype=torch.uint8, device="meta"), ValueError),  # another device
    (lambda n: torch.empty(2 * n, dtype=torch.uint8)[::2], ValueError),   # not contiguous
    (lambda n: torch.empty(n - 1, dtype=torch.uint8), ValueError),        # too small
])
def test_workspace_checked(bad, err):
    q, k, v, g, beta = _kda()
    need = pkv.chunk_kda_varlen_workspace_size(256, 2, 64, 64, 1, torch.bfloat16)
    assert need > 0
    with pytest.raises(err):
        pkv.chunk_kda_varlen(q, k, v, g, beta, workspace=bad(need))
    do = torch.zeros_like(v)
    need_b = pkv.chunk_kda_varlen_backward_workspace_size(256, 2, 64, 64, 1, torch.bfloat16)
    with pytest.raises(err):
        pkv.chunk_kda_varlen_backward(q, k, v, g, beta, do, workspace=bad(need_b))
