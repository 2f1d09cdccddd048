"""pkv_chunk_kda_varlen_noalloc, the entry point for callers that cannot
allocate, through the C ABI: on two calls in a row (the second smaller) its
outputs and final states equal those of pkv_chunk_kda_varlen (the entry point
with a caller workspace) bit for bit, and the smaller case matches the oracle;
sizes beyond its scratch array are refused before any launch."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity import check_close, device, f64

pytestmark = pytest.mark.gpu


def _pkv():
    import packed_varlen_gated_amd as pkv
    return pkv


def _case(seed, lens, tail, H, D):
    rng = np.random.default_rng(seed)
    real = np.concatenate([[0], np.cumsum(lens)])
    cu = np.concatenate([real, [real[-1]]])                  # one phantom slot
    N = int(real[-1]) + tail                                 # uncovered tail
    q = rng.standard_normal((N, H, D)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((N, H, D)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((N, H, D))
    g = -rng.uniform(0.0005, 0.05, (N, H, D))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N, H))))
    ts = [torch.from_numpy(a).to(torch.bfloat16) for a in (q, k, v, g, beta)]
    return ts, cu


def _noalloc(ts, cu):
    """One pkv_chunk_kda_varlen_noalloc call on torch's current stream."""
    lib = _pkv().library()
    dev = device()
    q, k, v, g, beta = [t.to(dev)[None] for t in ts]
    N, H, D = q.shape[1], q.shape[2], q.shape[3]
    cud = torch.from_numpy(cu.astype(np.int32)).to(dev)
    max_segs = len(cu) - 1
    o = torch.empty(1, N, H, D, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(max_segs, H, D, D, dtype=torch.float32, device=dev)
    flags = torch.zeros(1, dtype=torch.int32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    st = lib.pkv_chunk_kda_varlen_noalloc(p(q), p(k), p(v), p(g), p(beta), p(cud), max_segs, N, H, D, D,
                                          1.0, 0, 0, None, p(o), p(fs), p(flags),
                                          ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == 0, lib.pkv_status_string(st)
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    return o, fs


def _with_workspace(ts, cu):
    pkv = _pkv()
    dev = device()
    q, k, v, g, beta = [t.to(dev)[None] for t in ts]
    o, fs = pkv.chunk_kda_varlen(q, k, v, g, beta, torch.from_numpy(cu.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    return o, fs


def test_noalloc_matches_workspace_entry_twice():
    # first call: a 12000-token document cut into 3 runs (their states go through
    # the scratch array), others uncut, an empty slot, a phantom and a tail
    big, cu_big = _case(1, [12000, 700, 0, 3000], 40, 4, 128)
    # second call, smaller: D = 64, ragged short segments
    small, cu_small = _case(2, [300, 65, 1], 7, 2, 64)
    print("no-alloc: call 1 (N 15740, H 4, D 128)", flush=True)
    o1, f1 = _noalloc(big, cu_big)
    r1 = _with_workspace(big, cu_big)
    assert torch.equal(o1, r1[0]) and torch.equal(f1, r1[1])
    print("no-alloc: call 2 (N 373, H 2, D 64)", flush=True)
    o2, f2 = _noalloc(small, cu_small)
    r2 = _with_workspace(small, cu_small)
    assert torch.equal(o2, r2[0]) and torch.equal(f2, r2[1])
    ro, rfs = oracle.chunk_kda_varlen(*[f64(t) for t in small], cu_small)
    check_close(f64(o2[0]), ro, "bf16", "o")
    check_close(f64(f2), rfs, "bf16", "final states")
    # the first case again after the smaller one: nothing stale is read back
    o3, f3 = _noalloc(big, cu_big)
    assert torch.equal(o3, r1[0]) and torch.equal(f3, r1[1])


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = _pkv().library()
    A = lambda i: ctypes.c_void_p(i << 44)  # fake, far apart, never dereferenced
    N, H, D = 1 << 20, 32, 128
    st = lib.pkv_chunk_kda_varlen_noalloc(A(1), A(2), A(3), A(4), A(5), None, 1, N, H, D, D, 1.0, 0, 0,
                                          None, A(6), None, None, None)
    assert st == 3  # PKV_ERR_WORKSPACE, before any launch
    assert lib.pkv_chunk_kda_varlen_workspace_size(N, H, D, D, 1, 0) > (96 << 20)
