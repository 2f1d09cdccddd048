"""GPU parity of pkv_segment_ids_to_cu_seqlens against the oracle (bit-exact)."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import read_golden, parse_ints, parse_rows

pytestmark = pytest.mark.gpu


def _run(seg_np, max_segs):
    import packed_varlen_gated_amd as pkv
    seg = torch.from_numpy(np.ascontiguousarray(seg_np, dtype=np.int32)).cuda()
    r = pkv.segment_ids_to_cu_seqlens(seg, max_segs, with_token_seg=True)
    torch.cuda.synchronize()
    return (r.cu_seqlens.cpu().numpy(), r.token_seg.cpu().numpy(), int(r.n_segs.item()),
            int(r.flags.item()))


def _check(seg_np, max_segs):
    cu, tok, n, flags = _run(seg_np, max_segs)
    rcu, rn, rflags = oracle.segment_ids_to_cu_seqlens(seg_np, max_segs)
    assert cu.tolist() == rcu.tolist(), (seg_np.tolist() if seg_np.size < 200 else seg_np.shape)
    assert n == rn and flags == rflags
    N = seg_np.size
    assert tok.tolist() == oracle.token_segment(rcu, N).tolist()


@pytest.mark.parametrize("name", ["cu_seqlens_examples.txt", "cu_seqlens_cases.txt"])
def test_golden(name):
    for row in read_golden(name):
        seg = np.array(parse_rows(row[0]), dtype=np.int32)
        cu, tok, n, flags = _run(seg, int(row[1]))
        assert cu.tolist() == parse_ints(row[2]), row
        if len(row) > 3:
            assert n == int(row[3]) and flags == int(row[4]), row


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_workloads(name):
    wl = workloads.make_workload(name, tensors=False)
    _check(wl.segment_ids, wl.cfg.max_segs)


def test_fuzz():
    rng = np.random.default_rng(2024)
    for i in range(300):
        B = int(rng.integers(1, 6))
        T = int(rng.integers(1, 3000 if i % 10 == 0 else 80))
        seg = workloads.random_segment_ids(rng, B, T, int(rng.integers(1, 40)),
                                           pad_prob=float(rng.random()), lead_pad=bool(rng.random() < 0.3),
                                           mid_pad=bool(rng.random() < 0.5))
        if rng.random() < 0.05:
            seg[:] = 0
        max_segs = int(rng.integers(1, 64))
        print(f"fuzz case {i}: B={B} T={T} max_segs={max_segs}", flush=True)
        _check(seg, max_segs)


@pytest.mark.parametrize("N", [8191, 8192, 8193, 65536 + 3, 3 * 8192 - 1])
def test_tile_edges(N):
    rng = np.random.default_rng(N)
    seg = workloads.random_segment_ids(rng, 1, N, 700, pad_prob=0.5)
    _check(seg, 512)
    seg2 = workloads.random_segment_ids(rng, 1, N, 50)
    _check(seg2, 64)   # overflow


def test_row_start_collision_and_overflow_flags():
    seg = np.array([[1, 1, 1, 1], [1, 1, 2, 2], [1, 1, 1, 1]], dtype=np.int32)
    _check(seg, 8)
    _check(seg, 2)
    _check(np.array([[0, 0, 3, 3, 0, 4]], dtype=np.int32), 4)


@pytest.mark.parametrize("N", [65535, 65536, 65537, 2 * 65536 + 5, 3 * 65536 - 1])
def test_large_tile_edges(N):
    rng = np.random.default_rng(N + 1)
    seg = workloads.random_segment_ids(rng, 1, N, 900, pad_prob=0.5, mid_pad=True)
    _check(seg, 1024)
    _check(seg, 40)    # overflow


def test_long_trailing_and_leading_pad():
    # last real token in the first tile, then more than a tile of padding
    seg = np.zeros((1, 3 * 65536 + 7), dtype=np.int32)
    seg[0, 5:1000] = 1
    seg[0, 1000:40000] = 2
    _check(seg, 4)
    _check(seg, 1)   # overflow: the trailing pad joins the merged slot
    # real tokens only near the end: the backward sweep stops after one step
    seg2 = np.zeros((1, 2 * 65536 + 3), dtype=np.int32)
    seg2[0, -50:-20] = 7
    _check(seg2, 4)
    # real tokens only at the start: the backward sweep walks the whole pad
    seg3 = np.zeros((2, 70001), dtype=np.int32)
    seg3[0, :3] = 9
    _check(seg3, 4)


@pytest.mark.parametrize("T", [1, 2, 3, 5])
def test_short_rows(T):
    rng = np.random.default_rng(T)
    seg = workloads.random_segment_ids(rng, 4099, T, 5, pad_prob=0.3, mid_pad=True)
    _check(seg, 8192)
    _check(seg, 100)


def test_unaligned_input():
    """segment_ids at a 4-byte (not 16-byte) aligned address: the scalar-load path."""
    import packed_varlen_gated_amd as pkv
    rng = np.random.default_rng(11)
    B, T = 3, 30001
    seg_np = workloads.random_segment_ids(rng, B, T, 60, pad_prob=0.3, mid_pad=True)
    buf = torch.zeros(B * T + 1, dtype=torch.int32, device="cuda")
    buf[1:] = torch.from_numpy(seg_np.reshape(-1)).cuda()
    seg = buf[1:].view(B, T)
    assert seg.data_ptr() % 16 != 0
    r = pkv.segment_ids_to_cu_seqlens(seg, 256, with_token_seg=True)
    rcu, rn, rflags = oracle.segment_ids_to_cu_seqlens(seg_np, 256)
    assert r.cu_seqlens.cpu().numpy().tolist() == rcu.tolist()
    assert int(r.n_segs.item()) == rn and int(r.flags.item()) == rflags
    assert r.token_seg.cpu().numpy().tolist() == oracle.token_segment(rcu, B * T).tolist()
