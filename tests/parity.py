"""Shared helpers of the GPU parity tests: moving workloads to the device,
running the oracle on chosen (segment, head) pairs and the tolerance checks.

Tolerances (stated for the path's outputs):
  * integers (cu_seqlens, token_seg, n_segs, flags): bit-exact;
  * fp32 inputs: max |x - ref| <= 1e-4 * max |ref| per compared tensor;
  * bf16 inputs: ||x - ref||_2 / ||ref||_2 <= 2e-2 per compared tensor (and per
    segment as a diagnostic that a global norm cannot hide);
  * conv: |y - ref| <= gamma_Kc * sum_k |w x| (+ one bf16 ulp of ref for bf16
    output), gamma_n = n u / (1 - n u), u = 2^-24 (dot-product error bound,
    Higham, Accuracy and Stability of Numerical Algorithms, section 3.1).
"""

import math

import numpy as np
import torch

import oracle

FP32_MAXABS = 1e-4
BF16_RELL2 = 2e-2


def device():
    return torch.device("cuda", 0)


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def kda_inputs_to_device(wl, dev=None):
    dev = dev or device()
    N, H = wl.N, wl.cfg.H
    q = wl.q.reshape(1, N, H, -1).to(dev)
    k = wl.k.reshape(1, N, H, -1).to(dev)
    v = wl.v.reshape(1, N, H, -1).to(dev)
    g = wl.g.reshape(1, N, H, -1).to(dev)
    beta = wl.beta.reshape(1, N, H).to(dev)
    return q, k, v, g, beta


def oracle_segment_head(wl, a, e, h, scale=1.0):
    """Oracle o [e-a, Dv] and final state [Dk, Dv] of one (segment, head)."""
    sl = slice(a, e)
    hs = slice(h, h + 1)
    o, fs = oracle.chunk_kda_varlen(f64(wl.q[sl, hs]), f64(wl.k[sl, hs]), f64(wl.v[sl, hs]),
                                    f64(wl.g[sl, hs]), f64(wl.beta[sl, hs]), None, scale)
    return o[:, 0], fs[0, 0]


def check_close(got, ref, dtype, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if dtype == "f32":
        bound = FP32_MAXABS * max(np.max(np.abs(ref)), 1e-30)
        err = np.max(np.abs(got - ref)) if got.size else 0.0
        assert err <= bound, f"{what}: max abs err {err:.3e} > {bound:.3e}"
        return err / max(np.max(np.abs(ref)), 1e-30)
    nref = np.linalg.norm(ref)
    err = np.linalg.norm(got - ref)
    if nref == 0:
        assert err == 0, f"{what}: expected zeros"
        return 0.0
    rel = err / nref
    assert rel <= BF16_RELL2, f"{what}: rel-L2 {rel:.3e} > {BF16_RELL2}"
    return rel


def gamma(n, u=2.0 ** -24):
    return n * u / (1 - n * u)


def ulp_bf16(x):
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_conv(y, x, w, seg, dtype):
    """Element-wise bound of the masked conv against the oracle."""
    xd = np.asarray(x, dtype=np.float64)
    wd = np.asarray(w, dtype=np.float64)
    ref = oracle.short_conv_segmask(xd, wd, seg)
    absref = oracle.short_conv_segmask(np.abs(xd), np.abs(wd), seg)
    Kc = wd.shape[1]
    bound = gamma(Kc) * absref
    if dtype == "bf16":
        bound = bound + ulp_bf16(ref)
    err = np.abs(np.asarray(y, dtype=np.float64) - ref)
    bad = err > bound
    assert not bad.any(), f"conv: {int(bad.sum())} elements out of bound, worst {np.max(err - bound):.3e}"
