"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/pkv.h, and rejects bad arguments before launching."""

import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pkv.h")


@pytest.fixture(scope="module")
def lib():
    import packed_varlen_gated_amd as pkv
    if not os.path.exists(pkv.LIB_PATH):
        from packed_varlen_gated_amd import build
        build.build(verbose=False)
    return pkv.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) == 16, names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.pkv_abi_version() == 6
    for code, name in [(0, b"PKV_OK"), (1, b"PKV_ERR_INVALID_ARGUMENT"), (2, b"PKV_ERR_UNSUPPORTED"),
                       (3, b"PKV_ERR_WORKSPACE"), (4, b"PKV_ERR_HIP"), (99, b"PKV_ERR_UNKNOWN")]:
        assert lib.pkv_status_string(code) == name


# Fake, never dereferenced device addresses: every call below fails validation first.
P = ctypes.c_void_p(0x1000)
Q = ctypes.c_void_p(0x100000)
NUL = None


@pytest.mark.parametrize("args,code", [
    ((NUL, 2, 8, 4, Q, NUL, NUL, NUL, NUL), 1),           # no segment_ids
    ((P, 2, 8, 4, NUL, NUL, NUL, NUL, NUL), 1),           # no cu_seqlens
    ((P, 0, 8, 4, Q, NUL, NUL, NUL, NUL), 1),             # B < 1
    ((P, 2, 0, 4, Q, NUL, NUL, NUL, NUL), 1),             # T < 1
    ((P, 2, 8, 0, Q, NUL, NUL, NUL, NUL), 1),             # max_segs < 1
    ((P, 1 << 16, 1 << 16, 4, Q, NUL, NUL, NUL, NUL), 1),  # B*T > INT32_MAX
])
def test_cu_seqlens_validation(lib, args, code):
    assert lib.pkv_segment_ids_to_cu_seqlens(*args) == code


@pytest.mark.parametrize("args,code", [
    ((NUL, P, NUL, Q, 1, 8, 16, 4, 0, NUL), 1),      # no x
    ((P, NUL, NUL, Q, 1, 8, 16, 4, 0, NUL), 1),      # no w
    ((P, P, NUL, P, 1, 8, 16, 4, 0, NUL), 1),        # y aliases x
    ((P, P, NUL, Q, 1, 8, 0, 4, 0, NUL), 1),         # F < 1
    ((P, P, NUL, Q, 1, 8, 16, 0, 0, NUL), 2),        # Kc < 1
    ((P, P, NUL, Q, 1, 8, 16, 9, 0, NUL), 2),        # Kc > 8
    ((P, P, NUL, Q, 1, 8, 16, 4, 7, NUL), 2),        # unknown dtype
])
def test_short_conv_validation(lib, args, code):
    assert lib.pkv_short_conv_segmask(*args) == code


@pytest.mark.parametrize("args,code", [
    ((NUL, 2, 8, 0, Q, NUL, NUL, NUL), 1),                 # no tokens
    ((P, 2, 8, 0, NUL, NUL, NUL, NUL), 1),                 # no segment_ids
    ((P, 0, 8, 0, Q, NUL, NUL, NUL), 1),                   # B < 1
    ((P, 2, 0, 0, Q, NUL, NUL, NUL), 1),                   # T < 1
    ((P, 1 << 16, 1 << 16, 0, Q, NUL, NUL, NUL), 1),       # B*T > INT32_MAX
    ((P, 2, 8, 0, P, NUL, NUL, NUL), 1),                   # segment_ids overlaps tokens
    ((P, 2, 8, 0, Q, Q, NUL, NUL), 1),                     # positions overlaps segment_ids
])
def test_eod_validation(lib, args, code):
    assert lib.pkv_eod_to_segment_ids(*args) == code


def _kda_args(**kw):
    base = dict(q=ctypes.c_void_p(0x10000000), k=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x30000000),
                g=ctypes.c_void_p(0x40000000), beta=ctypes.c_void_p(0x50000000), cu=P, max_segs=4, N=256,
                H=2, Dk=64, Dv=64, scale=1.0, dtype=0, options=0, s0=NUL, o=ctypes.c_void_p(0x60000000), fs=NUL,
                flags=NUL, ws=NUL, ws_bytes=0, stream=NUL)
    base.update(kw)
    return tuple(base.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=NUL), 1), (dict(k=NUL), 1), (dict(v=NUL), 1), (dict(g=NUL), 1), (dict(beta=NUL), 1),
    (dict(o=NUL), 1), (dict(N=0), 1), (dict(N=1 << 31), 1), (dict(H=0), 1), (dict(max_segs=0), 1),
    (dict(Dk=48), 2), (dict(Dv=256), 2), (dict(dtype=5), 2), (dict(options=2), 2), (dict(options=-1), 2),
    (dict(o=ctypes.c_void_p(0x10000000 + 64)), 1),    # o overlaps q
    (dict(o=ctypes.c_void_p(0x60000008)), 1),         # o not 16-byte aligned
    (dict(k=ctypes.c_void_p(0x20000002)), 1),         # k not 16-byte aligned
    (dict(beta=ctypes.c_void_p(0x50000001)), 1),      # beta not element-aligned
    (dict(s0=ctypes.c_void_p(0x70000004)), 1),        # initial_state not 16-byte aligned
    (dict(s0=ctypes.c_void_p(0x70000000), fs=ctypes.c_void_p(0x70000000 + 4096)), 1),  # initial overlaps final
])
def test_chunk_kda_validation(lib, kw, code):
    args = _kda_args(**kw)
    lib.pkv_chunk_kda_varlen.argtypes  # loaded signature
    assert lib.pkv_chunk_kda_varlen(*args) == code


def test_workspace_query_is_host_only(lib):
    for N, H, D in [(512, 2, 32), (65536, 32, 128), (131072, 32, 128)]:
        ws = lib.pkv_chunk_kda_varlen_workspace_size(N, H, D, D, 256, 0)
        assert ws >= 0


def test_workspace_size_and_check(lib):
    """The chunk path (bf16, Dk/Dv in {64, 128}) keeps its work plan in the
    workspace: a run table (8 int32 per run, up to max_segs + s runs) and the
    states (Dk x Dv fp32) and decay products (Dk fp32) of s cut pieces per head.
    Only segments over 8192 tokens are cut, into runs of about 64 chunks, so
    with c = N // 8193 such segments at most, s = (N + 63 c) // 4096 + 1 (0
    when c = 0); other paths need none."""
    size = lib.pkv_chunk_kda_varlen_workspace_size

    def expect(N, H, Dk, Dv, S):
        c = N // 8193
        s = 0 if c == 0 else (N + 63 * c) // 4096 + 1
        up = lambda x: (x + 255) // 256 * 256
        table = (64 + 8 * (S + s) + 4 * s) * 4
        return up(table) + up(s * H * Dk * Dv * 4) + up(s * H * Dk * 4)

    for N, H, Dk, Dv, S in [(65536, 32, 128, 128, 256), (131072, 32, 128, 128, 8),
                            (32768, 32, 64, 64, 1024), (65536, 32, 128, 128, 1),
                            (100, 2, 64, 128, 3), (8192, 16, 128, 128, 128), (8193, 16, 128, 128, 128),
                            (1 << 20, 1, 64, 64, 1)]:
        assert size(N, H, Dk, Dv, S, 0) == expect(N, H, Dk, Dv, S), (N, H, S)
    # the saved pieces take about 1/16 of one [N, H, Dk] bf16 tensor at Dv = 128
    N = 1 << 24
    assert size(N, 32, 128, 128, 4, 0) < N * 32 * 128 * 2 / 15
    assert size(512, 2, 32, 32, 16, 1) == 0              # fp32 token-serial path
    assert size(512, 2, 32, 32, 16, 0) == 0              # Dk = 32: token-serial path
    # no workspace, too little, or misaligned: refused before any launch
    need = size(256, 2, 64, 64, 4, 0)
    assert lib.pkv_chunk_kda_varlen(*_kda_args(max_segs=4)) == 3
    assert lib.pkv_chunk_kda_varlen(*_kda_args(ws=P, ws_bytes=8)) == 3
    assert lib.pkv_chunk_kda_varlen(*_kda_args(ws=ctypes.c_void_p(0x1004), ws_bytes=need)) == 3
    # too many (segment, head) pairs for one launch
    assert lib.pkv_chunk_kda_varlen(*_kda_args(max_segs=1 << 21, H=4)) == 1


def _ids_args(**kw):
    base = dict(q=ctypes.c_void_p(0x10000000), k=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x30000000),
                g=ctypes.c_void_p(0x40000000), beta=ctypes.c_void_p(0x50000000), seg=ctypes.c_void_p(0x58000000),
                B=2, T=128, H=2, Dk=64, Dv=64, scale=1.0, dtype=0, options=0, s0=NUL,
                o=ctypes.c_void_p(0x60000000), fs=NUL, flags=NUL, ws=NUL, ws_bytes=0, stream=NUL)
    base.update(kw)
    return tuple(base.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=NUL), 1), (dict(seg=NUL), 1), (dict(o=NUL), 1), (dict(B=0), 1), (dict(T=0), 1),
    (dict(B=1 << 16, T=1 << 15), 1),                                   # B*T too large
    (dict(Dk=48), 2), (dict(dtype=5), 2), (dict(options=4), 2),
    (dict(o=ctypes.c_void_p(0x58000000)), 1),                          # o overlaps segment_ids
    (dict(s0=ctypes.c_void_p(0x70000000), fs=ctypes.c_void_p(0x70000000)), 1),  # initial == final
    (dict(), 3),                                                       # no workspace
])
def test_segment_ids_entry_validation(lib, kw, code):
    assert lib.pkv_chunk_kda_segment_ids(*_ids_args(**kw)) == code


def test_segment_ids_workspace_size(lib):
    """Bounds of at most B*T segments (one int32 each, after a 256-byte count
    word) and the chunk path's plan for that many slots; 0 off the chunk path."""
    size = lib.pkv_chunk_kda_segment_ids_workspace_size
    plan = lib.pkv_chunk_kda_varlen_workspace_size
    for B, T, H, D in [(8, 8192, 32, 128), (1, 300, 2, 64), (3, 1000, 4, 64)]:
        N = B * T
        assert size(B, T, H, D, D, 0) == (N * 4 + 4 + 256 + 255) // 256 * 256 + plan(N, H, D, D, N, 0)
    assert size(2, 64, 2, 32, 32, 0) == 0 and size(2, 64, 2, 64, 64, 1) == 0


def _bwd_args(**kw):
    A = lambda a: ctypes.c_void_p(a)
    base = dict(q=A(0x10000000), k=A(0x20000000), v=A(0x30000000), g=A(0x40000000), beta=A(0x50000000),
                cu=P, max_segs=4, N=256, H=2, Dk=64, Dv=64, scale=1.0, dtype=0, s0=NUL, do=A(0x58000000),
                dF=NUL, dq=A(0x60000000), dk=A(0x68000000), dv=A(0x70000000), dg=A(0x78000000),
                dbeta=A(0x7c000000), dinit=NUL, flags=NUL, ws=NUL, ws_bytes=0, stream=NUL)
    base.update(kw)
    return tuple(base.values())


@pytest.mark.parametrize("kw,code", [
    (dict(do=NUL), 1), (dict(dq=NUL), 1), (dict(dk=NUL), 1), (dict(dv=NUL), 1), (dict(dg=NUL), 1),
    (dict(dbeta=NUL), 1), (dict(q=NUL), 1), (dict(N=0), 1), (dict(H=0), 1), (dict(max_segs=0), 1),
    (dict(Dk=48), 2), (dict(Dv=16), 2), (dict(dtype=7), 2),
    (dict(dq=ctypes.c_void_p(0x10000000 + 256)), 1),     # dq overlaps q
    (dict(dg=ctypes.c_void_p(0x58000000)), 1),           # dg overlaps do
    (dict(dk=ctypes.c_void_p(0x60000000 + 512)), 1),     # dk overlaps dq
    (dict(dbeta=ctypes.c_void_p(0x7c000001)), 1),        # dbeta not element-aligned
    (dict(dv=ctypes.c_void_p(0x70000008)), 1),           # dv not 16-byte aligned
    (dict(dinit=ctypes.c_void_p(0x7e000000), dF=ctypes.c_void_p(0x7e000000)), 1),  # d initial == dfinal
    (dict(dinit=ctypes.c_void_p(0x7e000000), s0=ctypes.c_void_p(0x7e000000 + 4096)), 1),
    (dict(max_segs=1 << 21, H=4), 1),
])
def test_backward_entry_validation(lib, kw, code):
    assert lib.pkv_chunk_kda_varlen_backward(*_bwd_args(**kw)) == code


def test_backward_workspace(lib):
    """The chunked reverse pass (bf16, Dk and Dv in {64, 128}) keeps its plan
    (chunk, piece and summary offsets: 3 (max_segs + 1) int32, a work counter
    and an 8-int32 record of each piece in longest-first order, for max_segs +
    summaries pieces, padded to 256 bytes), one bf16 state of Dk x Dv per (chunk, head), chunks =
    ceil(N / 64) + max_segs, and for the pieces of cut segments, at most
    chunks / 16 + 1 of them, an fp32 Dk x Dv state and Dk decay products per
    (piece, role, head), and Dk fp32 final-state gate terms per (slot, head);
    other shapes need none."""
    size = lib.pkv_chunk_kda_varlen_backward_workspace_size
    up = lambda x: (x + 255) // 256 * 256
    for N, H, Dk, Dv, S in [(65536, 32, 128, 128, 256), (256, 2, 64, 64, 4), (1000, 3, 64, 128, 7),
                            (131072, 32, 128, 64, 8)]:
        chunks = (N + 63) // 64 + S
        sums = chunks // 16 + 1
        expect = (up(4 * (3 * (S + 1) + 1 + 8 * (S + sums))) + up(chunks * H * Dk * Dv * 2)
                  + up(sums * 2 * H * Dk * Dv * 4) + up(sums * 2 * H * Dk * 4) + up(S * H * Dk * 4))
        assert size(N, H, Dk, Dv, S, 0) == expect, (N, H, S)
    assert size(256, 2, 32, 32, 4, 0) == 0 and size(256, 2, 64, 64, 4, 1) == 0
    need = size(256, 2, 64, 64, 4, 0)
    assert lib.pkv_chunk_kda_varlen_backward(*_bwd_args()) == 3                       # missing
    assert lib.pkv_chunk_kda_varlen_backward(*_bwd_args(ws=P, ws_bytes=need - 1)) == 3
    assert lib.pkv_chunk_kda_varlen_backward(*_bwd_args(ws=ctypes.c_void_p(0x1080), ws_bytes=need)) == 3
    # a workspace over an input
    assert lib.pkv_chunk_kda_varlen_backward(*_bwd_args(ws=ctypes.c_void_p(0x10000000), ws_bytes=need)) == 1


def test_header_flag_and_option_bits_match_the_binding():
    import packed_varlen_gated_amd as pkv
    text = open(HEADER).read()
    bits = dict((n, int(v)) for n, v in re.findall(r"#define PKV_((?:FLAG|OPT)_[A-Z0-9_]+)\s+(\d+)", text))
    assert bits == {"FLAG_OVERFLOW": 1, "FLAG_LEADING_PAD": 2, "FLAG_BAD_CU_SEQLENS": 4,
                    "FLAG_GATE_RANGE": 8, "OPT_QK_L2NORM": 1}
    for n, v in bits.items():
        assert getattr(pkv, n) == v, n


# ---- the forward call that keeps the per-chunk states, and the reverse pass
# that reads them (argument checks only: nothing here reaches a launch)

def _kda_states_args(states=ctypes.c_void_p(0x7f000000), states_bytes=1 << 24, **kw):
    a = list(_kda_args(**kw))
    return tuple(a[:-1] + [states, states_bytes, a[-1]])


def _bwd_states_args(states=ctypes.c_void_p(0x7f000000), states_bytes=1 << 24, **kw):
    a = list(_bwd_args(**kw))
    return tuple(a[:-1] + [states, states_bytes, a[-1]])


def test_chunk_states_size(lib):
    """bf16 [ceil(N / 64) + max_segs, H, Dk, Dv] on the chunked path, else 0."""
    size = lib.pkv_chunk_kda_states_size
    for N, H, Dk, Dv, S in [(65536, 32, 128, 128, 256), (345, 2, 64, 64, 7), (1000, 3, 64, 128, 1),
                            (64, 1, 128, 64, 1)]:
        assert size(N, H, Dk, Dv, S, 0) == ((N + 63) // 64 + S) * H * Dk * Dv * 2
    assert size(256, 2, 32, 32, 4, 0) == 0       # Dk = 32: token-serial path
    assert size(256, 2, 64, 64, 4, 1) == 0       # fp32
    # the reverse pass given the states keeps none of its own
    full = lib.pkv_chunk_kda_varlen_backward_workspace_size
    lean = lib.pkv_chunk_kda_varlen_backward_states_workspace_size
    up = lambda x: (x + 255) // 256 * 256
    for N, H, Dk, Dv, S in [(65536, 32, 128, 128, 256), (1000, 3, 64, 128, 7)]:
        assert lean(N, H, Dk, Dv, S, 0) == full(N, H, Dk, Dv, S, 0) - up(size(N, H, Dk, Dv, S, 0))
    assert lean(256, 2, 32, 32, 4, 0) == 0


def test_forward_with_states_validation(lib):
    need = lib.pkv_chunk_kda_states_size(256, 2, 64, 64, 4, 0)
    ws = lib.pkv_chunk_kda_varlen_workspace_size(256, 2, 64, 64, 4, 0)
    W = dict(ws=ctypes.c_void_p(0x7e000000), ws_bytes=ws)
    f = lib.pkv_chunk_kda_varlen_states
    assert f(*_kda_states_args(states=NUL, **W)) == 1                                  # missing
    assert f(*_kda_states_args(states_bytes=need - 1, **W)) == 1                       # too small
    assert f(*_kda_states_args(states=ctypes.c_void_p(0x7f000008), **W)) == 1          # misaligned
    assert f(*_kda_states_args(states=ctypes.c_void_p(0x60000000), **W)) == 1          # over o
    assert f(*_kda_states_args(states=ctypes.c_void_p(0x7e000000), **W)) == 1          # over the workspace
    assert f(*_kda_states_args(Dk=32, Dv=32, **W)) == 2                                # no chunked path
    assert f(*_kda_states_args(dtype=1, **W)) == 2                                     # fp32
    assert f(*_kda_states_args()) == 3                                                 # no workspace
    assert f(*_kda_states_args(q=NUL, **W)) == 1                                       # the forward's own checks


def test_backward_with_states_validation(lib):
    need = lib.pkv_chunk_kda_states_size(256, 2, 64, 64, 4, 0)
    ws = lib.pkv_chunk_kda_varlen_backward_states_workspace_size(256, 2, 64, 64, 4, 0)
    W = dict(ws=ctypes.c_void_p(0x7e000000), ws_bytes=ws)
    f = lib.pkv_chunk_kda_varlen_backward_states
    assert f(*_bwd_states_args(states=NUL, **W)) == 1
    assert f(*_bwd_states_args(states_bytes=need - 1, **W)) == 1
    assert f(*_bwd_states_args(states=ctypes.c_void_p(0x7f000004), **W)) == 1
    assert f(*_bwd_states_args(states=ctypes.c_void_p(0x60000000), **W)) == 1          # under dq
    assert f(*_bwd_states_args(Dk=32, Dv=32, **W)) == 2
    assert f(*_bwd_states_args(dtype=1, **W)) == 2
    assert f(*_bwd_states_args()) == 3                                                 # no workspace
    assert f(*_bwd_states_args(ws=ctypes.c_void_p(0x7e000000), ws_bytes=ws - 1)) == 3
    assert f(*_bwd_states_args(dq=NUL, **W)) == 1
