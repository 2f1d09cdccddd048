"""Python binding of libpkv: packed (varlen) gated linear attention (KDA) on MI355X.

Thin argument marshalling over the C ABI in ``include/pkv.h``: shapes and
dtypes are checked, device pointers and torch's current HIP stream are passed
through ctypes, and every step of the computation runs in the library's HIP
kernels. Nothing here computes the method; if the library is not built the
calls raise instead of falling back to anything else.

Entry points (names follow RFC-0025 / RFC-0026):

* ``segment_ids_to_cu_seqlens(segment_ids, max_segs)``
* ``short_conv_segmask(x, w, segment_ids=None)``
* ``chunk_kda_varlen(q, k, v, g, beta, cu_seqlens=None, scale=1.0, output_final_state=True)``
* ``chunk_kda_varlen_backward(q, k, v, g, beta, do, cu_seqlens=None, scale=1.0, ...)``
* ``eod_to_segment_ids(tokens, eod_id)`` and ``chunk_kda_segment_ids(q, k, v, g, beta, segment_ids)``
"""

import ctypes
import os
from typing import NamedTuple, Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libpkv.so")

PKV_BF16 = 0
PKV_F32 = 1
FLAG_OVERFLOW = 1
FLAG_LEADING_PAD = 2
FLAG_BAD_CU_SEQLENS = 4
FLAG_GATE_RANGE = 8
OPT_QK_L2NORM = 1

_lib = None


class PkvError(RuntimeError):
    pass


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise PkvError(
            f"{LIB_PATH} is not built; run `python -m packed_varlen_gated_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.pkv_segment_ids_to_cu_seqlens.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp, vp]
    lib.pkv_segment_ids_to_cu_seqlens.restype = i32
    lib.pkv_eod_to_segment_ids.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    lib.pkv_eod_to_segment_ids.restype = i32
    lib.pkv_short_conv_segmask.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, i32, vp]
    lib.pkv_short_conv_segmask.restype = i32
    lib.pkv_chunk_kda_varlen_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.pkv_chunk_kda_varlen_workspace_size.restype = sz
    lib.pkv_chunk_kda_varlen.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, i32, i32,
                                         vp, vp, vp, vp, vp, sz, vp]
    lib.pkv_chunk_kda_varlen.restype = i32
    lib.pkv_chunk_kda_varlen_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, i32,
                                                 i32, vp, vp, vp, vp, vp]
    lib.pkv_chunk_kda_varlen_noalloc.restype = i32
    lib.pkv_chunk_kda_segment_ids_workspace_size.argtypes = [i64, i64, i32, i32, i32, i32]
    lib.pkv_chunk_kda_segment_ids_workspace_size.restype = sz
    lib.pkv_chunk_kda_segment_ids.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i32, i32, i32, f32, i32,
                                              i32, vp, vp, vp, vp, vp, sz, vp]
    lib.pkv_chunk_kda_segment_ids.restype = i32
    lib.pkv_chunk_kda_varlen_backward.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                                  f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                  vp, vp, sz, vp]
    lib.pkv_chunk_kda_varlen_backward.restype = i32
    lib.pkv_chunk_kda_varlen_backward_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.pkv_chunk_kda_varlen_backward_workspace_size.restype = sz
    lib.pkv_chunk_kda_states_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.pkv_chunk_kda_states_size.restype = sz
    lib.pkv_chunk_kda_varlen_states.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, f32, i32, i32,
                                                vp, vp, vp, vp, vp, sz, vp, sz, vp]
    lib.pkv_chunk_kda_varlen_states.restype = i32
    lib.pkv_chunk_kda_varlen_backward_states_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.pkv_chunk_kda_varlen_backward_states_workspace_size.restype = sz
    lib.pkv_chunk_kda_varlen_backward_states.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                                         f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                         vp, vp, sz, vp, sz, vp]
    lib.pkv_chunk_kda_varlen_backward_states.restype = i32
    lib.pkv_status_string.argtypes = [i32]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_abi_version.argtypes = []
    lib.pkv_abi_version.restype = i32
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(status):
    if status != 0:
        raise PkvError(_load().pkv_status_string(status).decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return PKV_BF16
    if dt == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {dt}; use bfloat16 or float32")


def _need(t, name, device, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(workspace, need, device):
    """The caller's workspace (checked: a contiguous uint8 tensor on the
    call's device holding at least `need` bytes), or a new one."""
    if need <= 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    _need(workspace, "workspace", device, torch.uint8)
    nbytes = workspace.numel()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, the call needs {need}")
    return workspace, nbytes


class EodSegments(NamedTuple):
    segment_ids: torch.Tensor                 # int32 [B, T]
    positions: Optional[torch.Tensor]         # int32 [B, T] or None
    loss_segment_ids: Optional[torch.Tensor]  # int32 [B, T] or None


class CuSeqlens(NamedTuple):
    cu_seqlens: torch.Tensor          # int32 [max_segs + 1]
    token_seg: Optional[torch.Tensor]  # int32 [B*T] or None
    n_segs: torch.Tensor              # int32 [1]
    flags: torch.Tensor               # int32 [1]


def segment_ids_to_cu_seqlens(segment_ids, max_segs, with_token_seg=False):
    """segment_ids int32 [B, T] (device) -> CuSeqlens (all device tensors, no sync)."""
    lib = _load()
    dev = segment_ids.device
    _need(segment_ids, "segment_ids", dev, torch.int32, 2)
    B, T = segment_ids.shape
    cu = torch.empty(max_segs + 1, dtype=torch.int32, device=dev)
    tok = torch.empty(B * T, dtype=torch.int32, device=dev) if with_token_seg else None
    n = torch.empty(1, dtype=torch.int32, device=dev)
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib.pkv_segment_ids_to_cu_seqlens(_ptr(segment_ids), B, T, max_segs, _ptr(cu), _ptr(tok),
                                             _ptr(n), _ptr(flags), _stream(dev)))
    return CuSeqlens(cu, tok, n, flags)


def eod_to_segment_ids(tokens, eod_id, with_positions=True, with_loss=True):
    """tokens int32 [B, T] (device) -> EodSegments of int32 [B, T] device tensors
    (positions / loss_segment_ids None when not requested). No sync."""
    lib = _load()
    dev = tokens.device
    _need(tokens, "tokens", dev, torch.int32, 2)
    B, T = tokens.shape
    seg = torch.empty(B, T, dtype=torch.int32, device=dev)
    pos = torch.empty(B, T, dtype=torch.int32, device=dev) if with_positions else None
    loss = torch.empty(B, T, dtype=torch.int32, device=dev) if with_loss else None
    _check(lib.pkv_eod_to_segment_ids(_ptr(tokens), B, T, int(eod_id), _ptr(seg), _ptr(pos), _ptr(loss),
                                      _stream(dev)))
    return EodSegments(seg, pos, loss)


def short_conv_segmask(x, w, segment_ids=None, out=None):
    """x [B, T, F] (bf16 or fp32), w fp32 [F, Kc], segment_ids int32 [B, T] or None -> y [B, T, F]."""
    lib = _load()
    dev = x.device
    _need(x, "x", dev, None, 3)
    dt = _dtype_code(x.dtype)
    _need(w, "w", dev, torch.float32, 2)
    B, T, F = x.shape
    if w.shape[0] != F:
        raise ValueError("w must be [F, Kc]")
    if segment_ids is not None:
        _need(segment_ids, "segment_ids", dev, torch.int32, 2)
        if tuple(segment_ids.shape) != (B, T):
            raise ValueError("segment_ids must be [B, T]")
    y = torch.empty_like(x) if out is None else out
    _need(y, "out", dev, x.dtype, 3)
    _need_shape(y, "out", x.shape)
    _check(lib.pkv_short_conv_segmask(_ptr(x), _ptr(w), _ptr(segment_ids), _ptr(y), B, T, F,
                                      w.shape[1], dt, _stream(dev)))
    return y


def chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, dtype):
    return int(_load().pkv_chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, _dtype_code(dtype)))


def chunk_kda_states_size(N, H, Dk, Dv, max_segs, dtype=torch.bfloat16):
    """Bytes of the per-chunk state buffer (0 when the shape has no chunked path)."""
    return int(_load().pkv_chunk_kda_states_size(N, H, Dk, Dv, max_segs, _dtype_code(dtype)))


def new_chunk_states(N, H, Dk, Dv, max_segs, device, dtype=torch.bfloat16):
    """A device buffer for ``chunk_kda_varlen(..., chunk_states=...)``."""
    n = chunk_kda_states_size(N, H, Dk, Dv, max_segs, dtype)
    if n == 0:
        raise PkvError("per-chunk states need the chunked path (bf16, Dk and Dv in {64, 128})")
    return torch.empty(n, dtype=torch.uint8, device=device)


def chunk_kda_varlen(q, k, v, g, beta, cu_seqlens=None, scale=1.0, output_final_state=True,
                     flags=None, out=None, workspace=None, initial_state=None,
                     use_qk_l2norm_in_kernel=False, chunk_states=None):
    """Packed KDA forward.

    q, k, g: [1, N, H, Dk] (or [B, T, H, Dk], taken as the flattened [1, B*T, H, Dk]);
    v: [..., Dv]; beta: [1, N, H]; cu_seqlens: int32 [max_segs + 1] or None (one segment).
    initial_state: fp32 [max_segs, H, Dk, Dv] or None (each segment starts from its slot's state).
    use_qk_l2norm_in_kernel: q and k are L2-normalised per (token, head) inside the call.
    chunk_states: None, or a device buffer (``new_chunk_states``) that receives the state before
    every 64-token chunk, for ``chunk_kda_varlen_backward(..., chunk_states=...)``.
    Returns (o [same leading shape as q, Dv], final_state fp32 [max_segs, H, Dk, Dv] or None).
    """
    lib = _load()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    for name, t, nd in (("q", q, 4), ("k", k, 4), ("v", v, 4), ("g", g, 4), ("beta", beta, 3)):
        _need(t, name, dev, dt, nd)
    Bq, Tq, H, Dk = q.shape
    N = Bq * Tq
    Dv = v.shape[3]
    if tuple(k.shape) != tuple(q.shape) or tuple(g.shape) != tuple(q.shape):
        raise ValueError("q, k and g must have the same shape")
    if tuple(v.shape[:3]) != (Bq, Tq, H) or tuple(beta.shape) != (Bq, Tq, H):
        raise ValueError("v must be [.., N, H, Dv] and beta [.., N, H]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dev, torch.int32, 1)
        max_segs = cu_seqlens.shape[0] - 1
    else:
        max_segs = 1
    o = torch.empty(Bq, Tq, H, Dv, dtype=dt, device=dev) if out is None else out
    _need(o, "out", dev, dt, 4)
    _need_shape(o, "out", (Bq, Tq, H, Dv))
    fs = torch.empty(max_segs, H, Dk, Dv, dtype=torch.float32, device=dev) if output_final_state else None
    if flags is not None:
        _need(flags, "flags", dev, torch.int32, 1)
    if initial_state is not None:
        _need(initial_state, "initial_state", dev, torch.float32, 4)
        if tuple(initial_state.shape) != (max_segs, H, Dk, Dv):
            raise ValueError(f"initial_state must be [{max_segs}, {H}, {Dk}, {Dv}]")
    need = int(lib.pkv_chunk_kda_varlen_workspace_size(N, H, Dk, Dv, max_segs, code))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), max_segs, N, H, Dk, Dv,
            float(scale), code, OPT_QK_L2NORM if use_qk_l2norm_in_kernel else 0, _ptr(initial_state),
            _ptr(o), _ptr(fs), _ptr(flags), _ptr(workspace), ws_bytes)
    if chunk_states is None:
        _check(lib.pkv_chunk_kda_varlen(*args, _stream(dev)))
    else:
        _need(chunk_states, "chunk_states", dev, None, None)
        _check(lib.pkv_chunk_kda_varlen_states(*args, _ptr(chunk_states),
                                               chunk_states.numel() * chunk_states.element_size(),
                                               _stream(dev)))
    return o, fs


def chunk_kda_segment_ids_workspace_size(B, T, H, Dk, Dv, dtype):
    return int(_load().pkv_chunk_kda_segment_ids_workspace_size(B, T, H, Dk, Dv, _dtype_code(dtype)))


def chunk_kda_segment_ids(q, k, v, g, beta, segment_ids, scale=1.0, output_final_state=True,
                          initial_state=None, flags=None, out=None, workspace=None,
                          use_qk_l2norm_in_kernel=False):
    """Packed KDA from [B, T] segment ids (reset where the id changes and at each row start).

    q, k, g: [B, T, H, Dk]; v: [B, T, H, Dv]; beta: [B, T, H]; segment_ids: int32 [B, T];
    initial_state: fp32 [B, H, Dk, Dv] or None (the first segment of each row starts from it).
    Returns (o [B, T, H, Dv], final_state fp32 [B, H, Dk, Dv] (the state after each row) or None).
    """
    lib = _load()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    for name, t, nd in (("q", q, 4), ("k", k, 4), ("v", v, 4), ("g", g, 4), ("beta", beta, 3)):
        _need(t, name, dev, dt, nd)
    _need(segment_ids, "segment_ids", dev, torch.int32, 2)
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if tuple(k.shape) != tuple(q.shape) or tuple(g.shape) != tuple(q.shape):
        raise ValueError("q, k and g must have the same shape")
    if tuple(v.shape[:3]) != (B, T, H) or tuple(beta.shape) != (B, T, H) or tuple(segment_ids.shape) != (B, T):
        raise ValueError("v must be [B, T, H, Dv], beta [B, T, H] and segment_ids [B, T]")
    o = torch.empty(B, T, H, Dv, dtype=dt, device=dev) if out is None else out
    _need(o, "out", dev, dt, 4)
    _need_shape(o, "out", (B, T, H, Dv))
    fs = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev) if output_final_state else None
    if initial_state is not None:
        _need(initial_state, "initial_state", dev, torch.float32, 4)
        if tuple(initial_state.shape) != (B, H, Dk, Dv):
            raise ValueError(f"initial_state must be [{B}, {H}, {Dk}, {Dv}]")
    if flags is not None:
        _need(flags, "flags", dev, torch.int32, 1)
    need = int(lib.pkv_chunk_kda_segment_ids_workspace_size(B, T, H, Dk, Dv, code))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    _check(lib.pkv_chunk_kda_segment_ids(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(segment_ids),
                                         B, T, H, Dk, Dv, float(scale), code,
                                         OPT_QK_L2NORM if use_qk_l2norm_in_kernel else 0, _ptr(initial_state), _ptr(o),
                                         _ptr(fs), _ptr(flags), _ptr(workspace), ws_bytes, _stream(dev)))
    return o, fs


class KdaGrads(NamedTuple):
    dq: torch.Tensor                         # like q
    dk: torch.Tensor                         # like k
    dv: torch.Tensor                         # like v
    dg: torch.Tensor                         # like g
    dbeta: torch.Tensor                      # like beta
    d_initial_state: Optional[torch.Tensor]  # fp32 [max_segs, H, Dk, Dv] or None


def chunk_kda_varlen_backward_workspace_size(N, H, Dk, Dv, max_segs, dtype):
    return int(_load().pkv_chunk_kda_varlen_backward_workspace_size(N, H, Dk, Dv, max_segs,
                                                                    _dtype_code(dtype)))


def chunk_kda_varlen_backward_states_workspace_size(N, H, Dk, Dv, max_segs, dtype):
    return int(_load().pkv_chunk_kda_varlen_backward_states_workspace_size(N, H, Dk, Dv, max_segs,
                                                                           _dtype_code(dtype)))


def chunk_kda_varlen_backward(q, k, v, g, beta, do, cu_seqlens=None, scale=1.0, initial_state=None,
                              dfinal_state=None, output_d_initial_state=None, flags=None,
                              workspace=None, chunk_states=None):
    """Reverse pass of ``chunk_kda_varlen`` on the same inputs.

    do: dL/do, shaped like the forward output; dfinal_state: fp32 [max_segs, H, Dk, Dv] or None
    (dL/dfinal_state). Returns KdaGrads; d_initial_state is returned when
    ``output_d_initial_state`` is true (default: when initial_state is given). The chunked path
    (bf16, Dk and Dv in {64, 128}) needs a workspace (allocated here when not given).
    chunk_states: None (the states are recomputed), or the buffer the forward call filled
    (``chunk_kda_varlen(..., chunk_states=...)`` on the same inputs).
    """
    lib = _load()
    dev = q.device
    dt = q.dtype
    code = _dtype_code(dt)
    for name, t, nd in (("q", q, 4), ("k", k, 4), ("v", v, 4), ("g", g, 4), ("beta", beta, 3),
                        ("do", do, 4)):
        _need(t, name, dev, dt, nd)
    Bq, Tq, H, Dk = q.shape
    N = Bq * Tq
    Dv = v.shape[3]
    if tuple(k.shape) != tuple(q.shape) or tuple(g.shape) != tuple(q.shape):
        raise ValueError("q, k and g must have the same shape")
    if tuple(v.shape) != (Bq, Tq, H, Dv) or tuple(do.shape) != (Bq, Tq, H, Dv) or \
            tuple(beta.shape) != (Bq, Tq, H):
        raise ValueError("v and do must be [.., N, H, Dv] and beta [.., N, H]")
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", dev, torch.int32, 1)
        max_segs = cu_seqlens.shape[0] - 1
    else:
        max_segs = 1
    for name, t in (("initial_state", initial_state), ("dfinal_state", dfinal_state)):
        if t is not None:
            _need(t, name, dev, torch.float32, 4)
            if tuple(t.shape) != (max_segs, H, Dk, Dv):
                raise ValueError(f"{name} must be [{max_segs}, {H}, {Dk}, {Dv}]")
    if flags is not None:
        _need(flags, "flags", dev, torch.int32, 1)
    if output_d_initial_state is None:
        output_d_initial_state = initial_state is not None
    dq, dk, dg = (torch.empty_like(q) for _ in range(3))
    dv = torch.empty_like(v)
    dbeta = torch.empty_like(beta)
    dinit = torch.empty(max_segs, H, Dk, Dv, dtype=torch.float32, device=dev) if output_d_initial_state else None
    size_fn = (lib.pkv_chunk_kda_varlen_backward_workspace_size if chunk_states is None
               else lib.pkv_chunk_kda_varlen_backward_states_workspace_size)
    need = int(size_fn(N, H, Dk, Dv, max_segs, code))
    workspace, ws_bytes = _workspace(workspace, need, dev)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), max_segs, N, H, Dk, Dv,
            float(scale), code, _ptr(initial_state), _ptr(do), _ptr(dfinal_state), _ptr(dq), _ptr(dk),
            _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dinit), _ptr(flags), _ptr(workspace), ws_bytes)
    if chunk_states is None:
        _check(lib.pkv_chunk_kda_varlen_backward(*args, _stream(dev)))
    else:
        _need(chunk_states, "chunk_states", dev, None, None)
        _check(lib.pkv_chunk_kda_varlen_backward_states(*args, _ptr(chunk_states),
                                                        chunk_states.numel() * chunk_states.element_size(),
                                                        _stream(dev)))
    return KdaGrads(dq, dk, dv, dg, dbeta, dinit)
