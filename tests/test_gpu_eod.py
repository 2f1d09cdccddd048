"""GPU parity of pkv_eod_to_segment_ids against the oracle: bit-exact segment
ids, positions and loss ids (RFC-0025, Design section 6)."""

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden, parse_rows
from parity import device

pytestmark = pytest.mark.gpu


def _pkv():
    import packed_varlen_gated_amd as pkv
    return pkv


def _check(tokens, eod, with_positions=True, with_loss=True):
    pkv = _pkv()
    x = torch.from_numpy(np.ascontiguousarray(tokens).astype(np.int32)).to(device())
    r = pkv.eod_to_segment_ids(x, eod, with_positions, with_loss)
    torch.cuda.synchronize()
    seg, pos, loss = oracle.eod_to_segment_ids(tokens, eod)
    assert np.array_equal(r.segment_ids.cpu().numpy(), seg)
    if with_positions:
        assert np.array_equal(r.positions.cpu().numpy(), pos)
    if with_loss:
        assert np.array_equal(r.loss_segment_ids.cpu().numpy(), loss)


@pytest.mark.parametrize("row", read_golden("eod_cases.txt"))
def test_golden_cases(row):
    tokens, eod = row[0], int(row[1])
    rows = parse_rows(tokens)
    _check(np.array(rows), eod)


@pytest.mark.parametrize("B,T,p_eod", [(1, 1, 0.5), (3, 7, 0.3), (2, 4095, 0.01), (2, 4096, 0.001),
                                       (4, 4097, 0.05), (8, 8192, 0.0007), (1, 131072, 0.00005),
                                       (2, 12289, 0.0), (1, 9000, 1.0)])
def test_random_rows(B, T, p_eod):
    """Several tiles of 4096 positions, ragged tails, no EOD, only EODs."""
    rng = np.random.default_rng(B * 100003 + T)
    eod = 0
    tokens = rng.integers(1, 50000, size=(B, T))
    tokens[rng.random((B, T)) < p_eod] = eod
    print(f"B={B} T={T} p_eod={p_eod}", flush=True)
    _check(tokens, eod)


def test_optional_outputs_and_unaligned_rows():
    """Only the ids requested; rows whose start is not 16-byte aligned (odd T)."""
    rng = np.random.default_rng(5)
    tokens = rng.integers(0, 4, size=(3, 4101))  # eod_id = 3, frequent
    _check(tokens, 3, with_positions=False, with_loss=False)
    _check(tokens, 3, with_positions=True, with_loss=False)
    _check(tokens, 3, with_positions=False, with_loss=True)


def test_feeds_segment_ids_to_cu_seqlens():
    """The GPU ids fed to the GPU conversion give the oracle's cu_seqlens."""
    pkv = _pkv()
    rng = np.random.default_rng(11)
    tokens = rng.integers(1, 100, size=(4, 2048))
    tokens[rng.random(tokens.shape) < 0.004] = 0
    x = torch.from_numpy(tokens.astype(np.int32)).to(device())
    seg = pkv.eod_to_segment_ids(x, 0).segment_ids
    res = pkv.segment_ids_to_cu_seqlens(seg, 128)
    torch.cuda.synchronize()
    ref_seg, _, _ = oracle.eod_to_segment_ids(tokens, 0)
    cu, n, flags = oracle.segment_ids_to_cu_seqlens(ref_seg, 128)
    assert np.array_equal(res.cu_seqlens.cpu().numpy(), cu)
    assert int(res.n_segs.item()) == n and int(res.flags.item()) == flags
