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
    assert len(names) == 6, names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.pkv_abi_version() == 1
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


def _kda_args(**kw):
    base = dict(q=ctypes.c_void_p(0x10000000), k=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x30000000),
                g=ctypes.c_void_p(0x40000000), beta=ctypes.c_void_p(0x50000000), cu=P, max_segs=4, N=256,
                H=2, Dk=64, Dv=64, scale=1.0, dtype=0, o=ctypes.c_void_p(0x60000000), fs=NUL, flags=NUL,
                ws=NUL, ws_bytes=0, stream=NUL)
    base.update(kw)
    return tuple(base.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q=NUL), 1), (dict(k=NUL), 1), (dict(v=NUL), 1), (dict(g=NUL), 1), (dict(beta=NUL), 1),
    (dict(o=NUL), 1), (dict(N=0), 1), (dict(N=1 << 31), 1), (dict(H=0), 1), (dict(max_segs=0), 1),
    (dict(Dk=48), 2), (dict(Dv=256), 2), (dict(dtype=5), 2),
    (dict(o=ctypes.c_void_p(0x10000000 + 64)), 1),    # o overlaps q
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
    """The chunk path (bf16, Dk/Dv in {64, 128}) keeps a longest-first order of
    the segment slots (int32 per slot) in the workspace; other paths need none."""
    size = lib.pkv_chunk_kda_varlen_workspace_size
    assert size(65536, 32, 128, 128, 256, 0) >= 256 * 4
    assert size(65536, 32, 128, 128, 1, 0) == 0          # one segment: nothing to order
    assert size(512, 2, 32, 32, 16, 1) == 0              # fp32 token-serial path
    assert size(512, 2, 32, 32, 16, 0) == 0              # Dk = 32: token-serial path
    # a valid call without the workspace is refused before any launch
    assert lib.pkv_chunk_kda_varlen(*_kda_args(max_segs=4)) == 3
    assert lib.pkv_chunk_kda_varlen(*_kda_args(ws=P, ws_bytes=8)) == 3
