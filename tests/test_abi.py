"""The C ABI without a GPU: the library loads, exports what include/fa.h declares,
and rejects bad arguments on the host before any HIP call is made."""
import ctypes
import math
import os
import re

import pytest

import online_softmax_04_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]

# Fake device addresses: validation rejects every call below before touching them.
A = 0x7f0000000000
MB = 1 << 20


def declared_functions():
    names = []
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", text, flags=re.M)
    return names


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_f16", "fa_fwd_f32", "fa_fwd_local", "fa_fwd_local_f16",
              "fa_fwd_blocksparse", "fa_fwd_blocksparse_f16", "fa_bwd",
              "fa_bwd_f16", "fa_bwd_workspace_bytes",
              "fa_decode", "fa_decode_f16", "fa_decode_workspace_bytes", "fa_fwd_fp8",
              "fa_decode_static", "fa_stream_copy", "fa_mfma_stream",
              "online_softmax_rows", "online_softmax_rows_split",
              "online_softmax_split_workspace_bytes", "fa_status_string", "fa_kernel_attributes"):
        assert n in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_declared_symbol(name):
    lib = ctypes.CDLL(fa.LIB_PATH)
    assert hasattr(lib, name), f"libfa.so does not export {name}"


def test_status_strings():
    for s in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_ALIGNMENT,
              fa.FA_ERR_HIP, fa.FA_ERR_SCRATCH_LIMIT):
        assert fa.fa_status_string(s).startswith("FA_")
    assert fa.fa_status_string(12345) == "unknown fa_status"


def call_attn(name="fa_fwd", q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB,
              lse=A + 256 * MB, B=1, H=2, N=128, d=64, scale=0.125, causal=0):
    fn = getattr(fa.lib(), name)
    return fn(q, k, v, o, lse, B, H, N, d, scale, causal, None)


ENTRIES = ["fa_fwd", "fa_fwd_f16", "fa_fwd_f32"]


@pytest.mark.parametrize("name", ENTRIES)
@pytest.mark.parametrize("kw", [dict(q=0), dict(k=0), dict(v=0), dict(o=0)])
def test_attn_null_pointer(name, kw):
    assert call_attn(name, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ENTRIES)
@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(B=-1),
                                dict(N=-5)])
def test_attn_bad_sizes(name, kw):
    assert call_attn(name, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ENTRIES)
@pytest.mark.parametrize("scale", [0.0, -0.125, math.inf, -math.inf, math.nan])
def test_attn_bad_scale(name, scale):
    assert call_attn(name, scale=scale) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ENTRIES)
def test_attn_bad_causal_flag(name):
    assert call_attn(name, causal=2) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ENTRIES)
@pytest.mark.parametrize("d", [1, 16, 32, 63, 96, 127, 192, 256])
def test_attn_unsupported_head_dim(name, d):
    """Head dims without a kernel are an error, never a silent slow path."""
    assert call_attn(name, d=d) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ENTRIES)
def test_attn_size_overflow(name):
    assert call_attn(name, B=1 << 20, H=1 << 20, N=1 << 20, d=128) == fa.FA_ERR_INVALID_ARG
    # more workgroups than a 1-D grid holds
    assert call_attn(name, B=1 << 16, H=1 << 16, N=256, d=64) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ENTRIES)
@pytest.mark.parametrize("kw", [dict(q=A + 2), dict(k=A + 64 * MB + 8), dict(v=A + 128 * MB + 4),
                                dict(o=A + 192 * MB + 2), dict(lse=A + 256 * MB + 2)])
def test_attn_alignment(name, kw):
    assert call_attn(name, **kw) == fa.FA_ERR_ALIGNMENT


@pytest.mark.parametrize("name", ENTRIES)
@pytest.mark.parametrize("kw", [dict(o=A), dict(o=A + 64 * MB + 1024), dict(o=A + 128 * MB - 1024),
                                dict(lse=A + 192 * MB + 16), dict(lse=A)])
def test_attn_overlap(name, kw):
    assert call_attn(name, **kw) == fa.FA_ERR_INVALID_ARG


def call_local(name="fa_fwd_local", doc=A + 320 * MB, window=16, **kw):
    base = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, H=2,
                N=128, d=64, scale=0.125)
    base.update(kw)
    fn = getattr(fa.lib(), name)
    return fn(base["q"], base["k"], base["v"], base["o"], base["lse"], doc, window, base["B"],
              base["H"], base["N"], base["d"], base["scale"], None)


@pytest.mark.parametrize("name", ["fa_fwd_local", "fa_fwd_local_f16"])
@pytest.mark.parametrize("kw,status", [
    (dict(window=-1), fa.FA_ERR_INVALID_ARG), (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG), (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(doc=A + 320 * MB + 2), fa.FA_ERR_ALIGNMENT),
    (dict(doc=A + 192 * MB), fa.FA_ERR_INVALID_ARG), (dict(doc=A + 256 * MB + 64), fa.FA_ERR_INVALID_ARG),
    (dict(o=A + 16), fa.FA_ERR_INVALID_ARG),
])
def test_local_validation(name, kw, status):
    assert call_local(name, **kw) == status


def call_sparse(name="fa_fwd_blocksparse", ptr=A + 320 * MB, idx=A + 384 * MB, nnz=4, **kw):
    base = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, H=2,
                N=128, d=64, scale=0.125, causal=0)
    base.update(kw)
    fn = getattr(fa.lib(), name)
    return fn(base["q"], base["k"], base["v"], base["o"], base["lse"], ptr, idx, nnz, base["B"],
              base["H"], base["N"], base["d"], base["scale"], base["causal"], None)


# every case fails validation before a launch (the addresses are not device memory)
@pytest.mark.parametrize("name", ["fa_fwd_blocksparse", "fa_fwd_blocksparse_f16"])
@pytest.mark.parametrize("kw,status", [
    (dict(ptr=0), fa.FA_ERR_INVALID_ARG), (dict(nnz=-1), fa.FA_ERR_INVALID_ARG),
    (dict(idx=0), fa.FA_ERR_INVALID_ARG), (dict(q=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG), (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG), (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(ptr=A + 320 * MB + 2), fa.FA_ERR_ALIGNMENT), (dict(idx=A + 384 * MB + 1), fa.FA_ERR_ALIGNMENT),
    (dict(ptr=A + 192 * MB + 8), fa.FA_ERR_INVALID_ARG),  # inside o
    (dict(idx=A + 256 * MB), fa.FA_ERR_INVALID_ARG),      # on lse
    (dict(ptr=A + 256 * MB - 4), fa.FA_ERR_INVALID_ARG),  # reaches into lse
    (dict(o=A + 64 * MB + 16), fa.FA_ERR_INVALID_ARG),    # o over k
])
def test_blocksparse_validation(name, kw, status):
    assert call_sparse(name, **kw) == status


# backward: ten buffers, 64 MiB apart (each [1, 2, 128, 64] 16-bit tensor is 32 KiB)
BWD_NAMES = ["q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "ws"]
BWD_ENTRIES = ["fa_bwd", "fa_bwd_f16"]


def call_bwd(name="fa_bwd", B=1, H=2, N=128, d=64, scale=0.125, causal=0, **ptrs):
    p = {n: A + 64 * MB * i for i, n in enumerate(BWD_NAMES)}
    p.update(ptrs)
    fn = getattr(fa.lib(), name)
    return fn(*(p[n] for n in BWD_NAMES), B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("name", BWD_ENTRIES)
@pytest.mark.parametrize("which", BWD_NAMES)
def test_bwd_null_pointer(name, which):
    assert call_bwd(name, **{which: 0}) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", BWD_ENTRIES)
@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(d=0), dict(N=-5),
                                dict(scale=0.0), dict(scale=math.nan), dict(causal=2),
                                dict(B=1 << 20, H=1 << 20, N=1 << 20, d=128),
                                dict(B=1 << 16, H=1 << 16, N=256, d=64)])
def test_bwd_bad_arguments(name, kw):
    assert call_bwd(name, **kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", BWD_ENTRIES)
@pytest.mark.parametrize("d", [32, 96, 256])
def test_bwd_unsupported_head_dim(name, d):
    assert call_bwd(name, d=d) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", BWD_ENTRIES)
@pytest.mark.parametrize("which,off", [("q", 2), ("dout", 8), ("dq", 4), ("dv", 2), ("ws", 4),
                                       ("lse", 2)])
def test_bwd_alignment(name, which, off):
    base = A + 64 * MB * BWD_NAMES.index(which)
    assert call_bwd(name, **{which: base + off}) == fa.FA_ERR_ALIGNMENT


@pytest.mark.parametrize("name", BWD_ENTRIES)
@pytest.mark.parametrize("kw", [dict(dq=A), dict(dk=A + 64 * MB * 4 + 1024),
                                dict(dv=A + 64 * MB * 6), dict(ws=A + 64 * MB * 7 + 16),
                                dict(dq=A + 64 * MB * 5 + 512), dict(ws=A + 64 * MB * 5)])
def test_bwd_overlap(name, kw):
    """Outputs may overlap neither an input nor each other."""
    assert call_bwd(name, **kw) == fa.FA_ERR_INVALID_ARG


def test_bwd_workspace_bytes():
    assert fa.fa_bwd_workspace_bytes(2, 3, 100) == 4 * 2 * 3 * 100
    assert fa.fa_bwd_workspace_bytes(0, 3, 100) == 0
    assert fa.fa_bwd_workspace_bytes(1 << 30, 1 << 30, 1 << 30) == 0


def call_softmax(x=A, y=A + 64 * MB, rows=4, cols=100):
    return fa.lib().online_softmax_rows(x, y, rows, cols, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), fa.FA_ERR_INVALID_ARG), (dict(y=0), fa.FA_ERR_INVALID_ARG),
    (dict(rows=0), fa.FA_ERR_INVALID_ARG), (dict(cols=0), fa.FA_ERR_INVALID_ARG),
    (dict(rows=-3), fa.FA_ERR_INVALID_ARG),
    (dict(x=A + 2), fa.FA_ERR_ALIGNMENT), (dict(y=A + 64 * MB + 1), fa.FA_ERR_ALIGNMENT),
    (dict(y=A + 1200), fa.FA_ERR_INVALID_ARG), (dict(y=A), fa.FA_ERR_INVALID_ARG),
    (dict(x=A + 64 * MB - 400), fa.FA_ERR_INVALID_ARG),
])
def test_softmax_validation(kw, status):
    assert call_softmax(**kw) == status


def test_split_workspace_bytes():
    # 4096-column chunks at least, about 2048 workgroups in all, 8 bytes per chunk
    assert fa.online_softmax_split_workspace_bytes(1, 1) == 8
    assert fa.online_softmax_split_workspace_bytes(1, 4096) == 8
    assert fa.online_softmax_split_workspace_bytes(1, 4097) == 16
    assert fa.online_softmax_split_workspace_bytes(4, 1 << 24) == 4 * 512 * 8
    assert fa.online_softmax_split_workspace_bytes(3000, 1 << 20) == 3000 * 8
    assert fa.online_softmax_split_workspace_bytes(0, 100) == 0
    assert fa.online_softmax_split_workspace_bytes(5, -1) == 0


WS = A + 128 * MB


def call_split(x=A, y=A + 64 * MB, rows=4, cols=100, ws=WS, wsb=None):
    if wsb is None:
        wsb = fa.online_softmax_split_workspace_bytes(4, 100)
    return fa.lib().online_softmax_rows_split(x, y, rows, cols, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), fa.FA_ERR_INVALID_ARG), (dict(y=0), fa.FA_ERR_INVALID_ARG),
    (dict(ws=0), fa.FA_ERR_INVALID_ARG),
    (dict(rows=0), fa.FA_ERR_INVALID_ARG), (dict(cols=0), fa.FA_ERR_INVALID_ARG),
    (dict(rows=1 << 30, cols=1 << 30), fa.FA_ERR_INVALID_ARG),
    (dict(wsb=31), fa.FA_ERR_INVALID_ARG),
    (dict(cols=5000), fa.FA_ERR_INVALID_ARG),          # needs two chunks a row: 64 bytes
    (dict(x=A + 2), fa.FA_ERR_ALIGNMENT), (dict(y=A + 64 * MB + 1), fa.FA_ERR_ALIGNMENT),
    (dict(ws=WS + 4), fa.FA_ERR_ALIGNMENT),
    (dict(y=A + 1200), fa.FA_ERR_INVALID_ARG), (dict(ws=A + 1592), fa.FA_ERR_INVALID_ARG),
    (dict(ws=A + 64 * MB + 8), fa.FA_ERR_INVALID_ARG),
])
def test_split_validation(kw, status):
    assert call_split(**kw) == status


def test_decode_workspace_bytes():
    # (batch*head, chunk, query) rows of d fp32 + an (m, l) pair; chunks of 32 tiles of
    # 32 keys, fewer tiles (down to 4) while the grid has under 2048 waves
    assert fa.fa_decode_workspace_bytes(8, 32, 1, 32768, 128) == 256 * 32 * 1 * (4 * 128 + 8)
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 131072, 64) == 1024 * (4 * 64 + 8)
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 1, 64) == 4 * 64 + 8
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 100, 96) == 0
    assert fa.fa_decode_workspace_bytes(0, 1, 1, 100, 64) == 0


def call_decode(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 200 * MB,
                ws=A + 256 * MB, wsb=None, B=1, H=2, Nq=3, Nk=100, d=128, scale=0.1, causal=1):
    if wsb is None:
        wsb = fa.fa_decode_workspace_bytes(1, 2, 3, 100, 128)
    return fa.lib().fa_decode(q, k, v, o, lse, ws, wsb, B, H, Nq, Nk, d, scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG), (dict(k=0), fa.FA_ERR_INVALID_ARG),
    (dict(v=0), fa.FA_ERR_INVALID_ARG), (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(ws=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG), (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(B=-1), fa.FA_ERR_INVALID_ARG), (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG), (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=101), fa.FA_ERR_INVALID_ARG),                 # causal needs Nq <= Nk
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=1 << 23), fa.FA_ERR_UNSUPPORTED),              # a head's K over 2^31 bytes
    (dict(wsb=100), fa.FA_ERR_INVALID_ARG),
    (dict(q=A + 8), fa.FA_ERR_ALIGNMENT), (dict(o=A + 192 * MB + 2), fa.FA_ERR_ALIGNMENT),
    (dict(ws=A + 256 * MB + 8), fa.FA_ERR_ALIGNMENT), (dict(lse=A + 200 * MB + 2), fa.FA_ERR_ALIGNMENT),
    (dict(o=A + 64 * MB + 512), fa.FA_ERR_INVALID_ARG),     # o inside k
    (dict(lse=A + 192 * MB + 16), fa.FA_ERR_INVALID_ARG),   # lse inside o
    (dict(ws=A + 192 * MB), fa.FA_ERR_INVALID_ARG),         # workspace on o
    (dict(ws=A), fa.FA_ERR_INVALID_ARG),                    # workspace on q
])
def test_decode_validation(kw, status):
    assert call_decode(**kw) == status


def call_decode_static(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 200 * MB,
                       B=1, H=2, Nq=3, Nk=100, d=128, scale=0.1, causal=1):
    return fa.lib().fa_decode_static(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG), (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG), (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG), (dict(Nq=101), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(B=8, H=32, Nq=64, Nk=65536), fa.FA_ERR_SCRATCH_LIMIT),  # 545 MB of partials
    (dict(q=A + 8), fa.FA_ERR_ALIGNMENT), (dict(lse=A + 200 * MB + 2), fa.FA_ERR_ALIGNMENT),
    (dict(o=A + 64 * MB + 512), fa.FA_ERR_INVALID_ARG),     # o inside k
])
def test_decode_static_validation(kw, status):
    """Every error of fa_decode_static is found on the host, before the scratch
    array is looked up (no GPU here)."""
    assert call_decode_static(**kw) == status


def test_decode_static_limit_is_the_headers():
    hdr = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_DECODE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.DECODE_STATIC_SCRATCH_BYTES
    # the decode workload fits
    assert fa.fa_decode_workspace_bytes(8, 32, 1, 32768, 128) <= fa.DECODE_STATIC_SCRATCH_BYTES
    assert fa.fa_status_string(fa.FA_ERR_SCRATCH_LIMIT).startswith("FA_ERR_SCRATCH_LIMIT")


def call_fp8(q=A, k=A + 64 * MB, v=A + 128 * MB, o=A + 192 * MB, lse=A + 256 * MB, B=1, H=2,
             N=100, d=128, scale=0.1, qs=0.5, ks=0.5, vs=0.5, causal=1):
    return fa.lib().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, qs, ks, vs, causal, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_INVALID_ARG), (dict(o=0), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG), (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(qs=0.0), fa.FA_ERR_INVALID_ARG), (dict(ks=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(vs=float("nan")), fa.FA_ERR_INVALID_ARG), (dict(causal=3), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED), (dict(N=1 << 23), fa.FA_ERR_UNSUPPORTED),
    (dict(q=A + 8), fa.FA_ERR_ALIGNMENT), (dict(o=A + 192 * MB + 4), fa.FA_ERR_ALIGNMENT),
    (dict(lse=A + 256 * MB + 1), fa.FA_ERR_ALIGNMENT),
    (dict(o=A + 128 * MB + 16), fa.FA_ERR_INVALID_ARG),    # o over v
    (dict(lse=A + 192 * MB + 64), fa.FA_ERR_INVALID_ARG),  # lse inside o
])
def test_fp8_validation(kw, status):
    assert call_fp8(**kw) == status


@pytest.mark.parametrize("args,status", [
    ((0, A + 64 * MB, 1024), fa.FA_ERR_INVALID_ARG), ((A, 0, 1024), fa.FA_ERR_INVALID_ARG),
    ((A, A + 64 * MB, 0), fa.FA_ERR_INVALID_ARG), ((A, A + 64 * MB, 1000), fa.FA_ERR_INVALID_ARG),
    ((A + 4, A + 64 * MB, 1024), fa.FA_ERR_ALIGNMENT), ((A, A + 64 * MB + 8, 1024), fa.FA_ERR_ALIGNMENT),
    ((A, A + 512, 1024), fa.FA_ERR_INVALID_ARG),            # overlapping
])
def test_stream_copy_validation(args, status):
    assert fa.lib().fa_stream_copy(*args, None) == status


OPB = fa.MFMA_STREAM_OPERAND_BYTES


@pytest.mark.parametrize("args,status", [
    ((0, OPB, A + MB, 1024, 2, 1), fa.FA_ERR_INVALID_ARG),           # no operands
    ((A, OPB, 0, 1024, 2, 1), fa.FA_ERR_INVALID_ARG),                # no output
    ((A, OPB - 16, A + MB, 1024, 2, 1), fa.FA_ERR_INVALID_ARG),      # operands too small
    ((A, OPB, A + MB, 1023, 2, 1), fa.FA_ERR_INVALID_ARG),           # output too small
    ((A, OPB, A + MB, 1024, 0, 1), fa.FA_ERR_INVALID_ARG),           # no workgroups
    ((A, OPB, A + MB, 1 << 30, (1 << 20) + 1, 1), fa.FA_ERR_INVALID_ARG),
    ((A, OPB, A + MB, 1024, 2, 0), fa.FA_ERR_INVALID_ARG),           # no iterations
    ((A, OPB, A + MB, 1024, 2, (1 << 20) + 1), fa.FA_ERR_INVALID_ARG),
    ((A + 8, OPB, A + MB, 1024, 2, 1), fa.FA_ERR_ALIGNMENT),
    ((A, OPB, A + MB + 2, 1024, 2, 1), fa.FA_ERR_ALIGNMENT),
    ((A, OPB, A + OPB - 64, 1024, 2, 1), fa.FA_ERR_INVALID_ARG),     # overlapping
])
def test_mfma_stream_validation(args, status):
    assert fa.lib().fa_mfma_stream(*args, None) == status


def test_python_wrappers_raise():
    with pytest.raises(fa.FaError) as e:
        fa.fa_fwd(0, A, A, A, None, 1, 1, 16, 64, 0.1, 0)
    assert e.value.status == fa.FA_ERR_INVALID_ARG
    with pytest.raises(fa.FaError) as e:
        fa.online_softmax_rows(A, A + 64 * MB, 0, 8)
    assert e.value.status == fa.FA_ERR_INVALID_ARG


def test_product_path_has_no_cpu_fallback():
    """The package never reaches the oracle and never computes on the host."""
    pkg = os.path.join(ROOT, "online_softmax_04_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text, f"{f} mentions the oracle"
                assert "import numpy" not in text, f"{f} imports numpy"
