"""Python binding of libfa.so: attention forward and row softmax on gfx950.

The functions named like the C ABI (``fa_fwd``, ``fa_fwd_f16``, ``fa_fwd_f32``,
``online_softmax_rows``) marshal arguments only: tensors become device
pointers, the stream defaults to torch's current HIP stream, and a non-zero
status becomes a ``FaError``.  Every step of the computation runs in the HIP
kernels of libfa.so; there is no other implementation in this package.
``attention`` and ``softmax`` allocate outputs with torch and call those.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FaError", "lib", "fa_fwd", "fa_fwd_f16", "fa_fwd_f32", "online_softmax_rows",
    "online_softmax_rows_split", "online_softmax_split_workspace_bytes", "softmax_split",
    "fa_decode", "fa_decode_f16", "fa_decode_workspace_bytes", "attention_decode", "fa_fwd_fp8",
    "fa_decode_static", "DECODE_STATIC_SCRATCH_BYTES", "FA_ERR_SCRATCH_LIMIT", "fa_stream_copy",
    "fa_mfma_stream", "MFMA_STREAM_OPERAND_BYTES",
    "fa_fwd_local", "fa_fwd_local_f16", "fa_fwd_blocksparse", "fa_fwd_blocksparse_f16",
    "attention_blocksparse", "SPARSE_QBLOCK", "SPARSE_KBLOCK",
    "fa_status_string", "kernel_attributes", "attention", "softmax", "LIB_PATH",
    "FA_OK", "FA_ERR_INVALID_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_ALIGNMENT", "FA_ERR_HIP",
]

# ONLINE_SOFTMAX_04_AMD_LIB names another build of the same library (for example one
# whose host code carries sanitizers); by default the in-tree libfa.so.
LIB_PATH = (os.environ.get("ONLINE_SOFTMAX_04_AMD_LIB")
            or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so"))

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_ALIGNMENT = -3
FA_ERR_HIP = -4
FA_ERR_SCRATCH_LIMIT = -5

# bytes of the static device array fa_decode_static takes its partials from
DECODE_STATIC_SCRATCH_BYTES = 8 << 20
# operand bytes fa_mfma_stream reads (16 sets x 16 fragments x 64 lanes x 16 bytes)
MFMA_STREAM_OPERAND_BYTES = 16 * 16 * 64 * 16

OP_FA_FWD, OP_FA_FWD_F16, OP_FA_FWD_F32, OP_SOFTMAX = 0, 1, 2, 3
OP_FA_BWD_DQ, OP_FA_BWD_DKDV, OP_FA_DECODE, OP_FA_FWD_FP8 = 4, 5, 6, 7
OP_FA_FWD_BLOCKSPARSE, OP_FA_FWD_LOCAL = 8, 9

# block sizes of a block-sparse pattern: query rows and keys per block
SPARSE_QBLOCK, SPARSE_KBLOCK = 256, 128


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)} (status {status})")


class _Attrs(ctypes.Structure):
    _fields_ = [("regs_per_lane", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("private_bytes", ctypes.c_int), ("threads_per_block", ctypes.c_int),
                ("blocks_per_cu", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m online_softmax_04_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        for name in ("fa_fwd", "fa_fwd_f16", "fa_fwd_f32"):
            fn = getattr(L, name)
            fn.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
            fn.restype = i
        for name in ("fa_fwd_local", "fa_fwd_local_f16"):
            fn = getattr(L, name)
            fn.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
            fn.restype = i
        for name in ("fa_fwd_blocksparse", "fa_fwd_blocksparse_f16"):
            fn = getattr(L, name)
            fn.argtypes = [vp] * 7 + [i, i, i, i, i, f, i, vp]
            fn.restype = i
        for name in ("fa_bwd", "fa_bwd_f16"):
            fn = getattr(L, name)
            fn.argtypes = [vp] * 10 + [i, i, i, i, f, i, vp]
            fn.restype = i
        L.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, f, f, f, i, vp]
        L.fa_fwd_fp8.restype = i
        for name in ("fa_decode", "fa_decode_f16"):
            fn = getattr(L, name)
            fn.argtypes = [vp] * 6 + [ctypes.c_size_t, i, i, i, i, i, f, i, vp]
            fn.restype = i
        L.fa_decode_static.argtypes = [vp] * 5 + [i, i, i, i, i, f, i, vp]
        L.fa_decode_static.restype = i
        L.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
        L.fa_decode_workspace_bytes.restype = ctypes.c_size_t
        L.fa_bwd_workspace_bytes.argtypes = [i, i, i]
        L.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.online_softmax_rows.argtypes = [vp, vp, i, i, vp]
        L.online_softmax_rows.restype = i
        L.online_softmax_split_workspace_bytes.argtypes = [i, i]
        L.online_softmax_split_workspace_bytes.restype = ctypes.c_size_t
        L.online_softmax_rows_split.argtypes = [vp, vp, i, i, vp, ctypes.c_size_t, vp]
        L.online_softmax_rows_split.restype = i
        L.fa_stream_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        L.fa_stream_copy.restype = i
        L.fa_mfma_stream.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_size_t, i, i, vp]
        L.fa_mfma_stream.restype = i
        L.fa_status_string.argtypes = [i]
        L.fa_status_string.restype = ctypes.c_char_p
        L.fa_kernel_attributes.argtypes = [i, i, i, ctypes.POINTER(_Attrs)]
        L.fa_kernel_attributes.restype = i
        _lib = L
    return _lib


def fa_stream_copy(x, y, nbytes, stream=None):
    """Copy nbytes (multiple of 16) with non-temporal 16-byte accesses: the HBM
    ceiling the benchmark reports beside the row softmax (see include/fa.h)."""
    _check(lib().fa_stream_copy(_ptr(x), _ptr(y), int(nbytes), _stream(stream)), "fa_stream_copy")


def fa_mfma_stream(operands, out, blocks, iters, stream=None):
    """Run blocks x 8 waves of iters x 8 bf16 32x32x16 MFMAs on `operands`
    (MFMA_STREAM_OPERAND_BYTES of bf16 values) into `out` (blocks x 512 floats):
    the matrix-unit ceiling the benchmark reports beside the attention forward
    (see include/fa.h)."""
    nbytes = operands.numel() * operands.element_size()
    _check(lib().fa_mfma_stream(_ptr(operands), nbytes, _ptr(out), out.numel(), int(blocks),
                                int(iters), _stream(stream)), "fa_mfma_stream")


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(int(status)).decode()


def _ptr(x):
    """Device address of a tensor-like (``data_ptr()``), an int, or None."""
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(stream):
    if stream is not None:
        return int(getattr(stream, "cuda_stream", stream))
    import torch
    if torch.cuda.is_available():
        return int(torch.cuda.current_stream().cuda_stream)
    return 0


def _check(status: int, where: str):
    if status != FA_OK:
        raise FaError(status, where)


def _attn(name, q, k, v, o, lse, B, H, N, d, scale, causal, stream):
    fn = getattr(lib(), name)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N), int(d),
              float(scale), int(causal), _stream(stream)), name)


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    """bf16 attention forward (see include/fa.h); q, k, v, o, lse are device buffers."""
    _attn("fa_fwd", q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f16(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    """fp16 attention forward (see include/fa.h)."""
    _attn("fa_fwd_f16", q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def fa_fwd_f32(q, k, v, o, lse, B, H, N, d, scale, causal, stream=None):
    """fp32 attention forward (see include/fa.h)."""
    _attn("fa_fwd_f32", q, k, v, o, lse, B, H, N, d, scale, causal, stream)


def _local(name, q, k, v, o, lse, doc_start, window, B, H, N, d, scale, stream):
    fn = getattr(lib(), name)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(doc_start), int(window), int(B),
              int(H), int(N), int(d), float(scale), _stream(stream)), name)


def fa_fwd_local(q, k, v, o, lse, doc_start, window, B, H, N, d, scale, stream=None):
    """bf16 causal attention with a sliding window and document starts (see include/fa.h)."""
    _local("fa_fwd_local", q, k, v, o, lse, doc_start, window, B, H, N, d, scale, stream)


def fa_fwd_local_f16(q, k, v, o, lse, doc_start, window, B, H, N, d, scale, stream=None):
    """fp16 causal attention with a sliding window and document starts (see include/fa.h)."""
    _local("fa_fwd_local_f16", q, k, v, o, lse, doc_start, window, B, H, N, d, scale, stream)


def _blocksparse(name, q, k, v, o, lse, blk_ptr, blk_idx, nnz, B, H, N, d, scale, causal,
                 stream):
    fn = getattr(lib(), name)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(blk_ptr), _ptr(blk_idx),
              int(nnz), int(B), int(H), int(N), int(d), float(scale), int(causal),
              _stream(stream)), name)


def fa_fwd_blocksparse(q, k, v, o, lse, blk_ptr, blk_idx, nnz, B, H, N, d, scale, causal,
                       stream=None):
    """bf16 attention under a block-sparse pattern in CSR form (see include/fa.h)."""
    _blocksparse("fa_fwd_blocksparse", q, k, v, o, lse, blk_ptr, blk_idx, nnz, B, H, N, d, scale,
                 causal, stream)


def fa_fwd_blocksparse_f16(q, k, v, o, lse, blk_ptr, blk_idx, nnz, B, H, N, d, scale, causal,
                           stream=None):
    """fp16 attention under a block-sparse pattern in CSR form (see include/fa.h)."""
    _blocksparse("fa_fwd_blocksparse_f16", q, k, v, o, lse, blk_ptr, blk_idx, nnz, B, H, N, d,
                 scale, causal, stream)


def _bwd(name, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, stream):
    fn = getattr(lib(), name)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
              _ptr(dv), _ptr(workspace), int(B), int(H), int(N), int(d), float(scale), int(causal),
              _stream(stream)), name)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, stream=None):
    """bf16 attention backward (see include/fa.h); every argument buffer is on the device."""
    _bwd("fa_bwd", q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal, stream)


def fa_bwd_f16(q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal,
               stream=None):
    """fp16 attention backward (see include/fa.h)."""
    _bwd("fa_bwd_f16", q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale, causal,
         stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, q_descale, k_descale, v_descale, causal,
               stream=None):
    """Attention forward with fp8 E4M3 Q/K/V (value = descale * code) and bf16 O
    (see include/fa.h)."""
    _check(lib().fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H), int(N),
                            int(d), float(scale), float(q_descale), float(k_descale),
                            float(v_descale), int(causal), _stream(stream)), "fa_fwd_fp8")


def _decode(name, q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
            stream):
    fn = getattr(lib(), name)
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace), int(workspace_bytes),
              int(B), int(H), int(Nq), int(Nk), int(d), float(scale), int(causal), _stream(stream)),
           name)


def fa_decode(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
              stream=None):
    """bf16 split-KV attention of Nq queries at the end of Nk keys (see include/fa.h)."""
    _decode("fa_decode", q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
            stream)


def fa_decode_f16(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale, causal,
                  stream=None):
    """fp16 split-KV attention of Nq queries at the end of Nk keys (see include/fa.h)."""
    _decode("fa_decode_f16", q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d, scale,
            causal, stream)


def fa_decode_static(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, stream=None):
    """fa_decode (bf16) with its partials in the library's static device array: no
    workspace argument, nothing allocated (see include/fa.h)."""
    _check(lib().fa_decode_static(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), int(B), int(H),
                                  int(Nq), int(Nk), int(d), float(scale), int(causal),
                                  _stream(stream)), "fa_decode_static")


def fa_decode_workspace_bytes(B, H, Nq, Nk, d) -> int:
    """Bytes of workspace fa_decode needs (0 for invalid sizes)."""
    return int(lib().fa_decode_workspace_bytes(int(B), int(H), int(Nq), int(Nk), int(d)))


def fa_bwd_workspace_bytes(B, H, N) -> int:
    """Bytes of fp32 workspace fa_bwd needs (0 for invalid sizes)."""
    return int(lib().fa_bwd_workspace_bytes(int(B), int(H), int(N)))


def online_softmax_rows(x, y, rows, cols, stream=None):
    """Row softmax of an fp32 [rows, cols] device buffer into y (see include/fa.h)."""
    _check(lib().online_softmax_rows(_ptr(x), _ptr(y), int(rows), int(cols), _stream(stream)),
           "online_softmax_rows")


def online_softmax_split_workspace_bytes(rows, cols) -> int:
    """Bytes of workspace online_softmax_rows_split needs (0 for invalid sizes)."""
    return int(lib().online_softmax_split_workspace_bytes(int(rows), int(cols)))


def online_softmax_rows_split(x, y, rows, cols, workspace, workspace_bytes, stream=None):
    """Row softmax with each row spread over several workgroups (see include/fa.h)."""
    _check(lib().online_softmax_rows_split(_ptr(x), _ptr(y), int(rows), int(cols), _ptr(workspace),
                                           int(workspace_bytes), _stream(stream)),
           "online_softmax_rows_split")


def kernel_attributes(op: int, d: int, causal: bool = False) -> dict:
    """Registers, LDS, spill bytes, block size and occupancy of the kernel an op launches."""
    a = _Attrs()
    _check(lib().fa_kernel_attributes(int(op), int(d), int(causal), ctypes.byref(a)),
           "fa_kernel_attributes")
    return {f: getattr(a, f) for f, _ in _Attrs._fields_}


# ---------------------------------------------------------------------------
# torch conveniences
# ---------------------------------------------------------------------------
def _entry_for(dtype):
    import torch
    return {torch.bfloat16: "fa_fwd", torch.float16: "fa_fwd_f16",
            torch.float32: "fa_fwd_f32"}.get(dtype)


def attention(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None,
              stream=None):
    """O, LSE = attention forward of [B, H, N, d] device tensors (bf16, fp16 or fp32).

    Returns (o, lse) with o like q and lse fp32 [B, H, N].
    """
    import torch
    for t in (q, k, v):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise TypeError("q, k, v must be device tensors")
        if not t.is_contiguous() or t.dim() != 4 or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous [B, H, N, d] tensors of one dtype")
    name = _entry_for(q.dtype)
    if name is None:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _attn(name, q, k, v, out, lse, B, H, N, d, scale, causal, stream)
    return out, lse


def attention_blocksparse(q, k, v, blk_ptr, blk_idx, causal: bool = False,
                          scale: float | None = None, out=None, lse=None, stream=None):
    """O, LSE of [B, H, N, d] bf16 or fp16 device tensors under a block-sparse pattern:
    blk_ptr (int32, ceil(N / SPARSE_QBLOCK) + 1) and blk_idx (int32, nnz) on the device
    list, per query block, the key blocks of SPARSE_KBLOCK keys it sees."""
    import torch
    for t in (q, k, v):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise TypeError("q, k, v must be device tensors")
        if not t.is_contiguous() or t.dim() != 4 or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous [B, H, N, d] tensors of one dtype")
    names = {torch.bfloat16: "fa_fwd_blocksparse", torch.float16: "fa_fwd_blocksparse_f16"}
    if q.dtype not in names:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    n_qb = (N + SPARSE_QBLOCK - 1) // SPARSE_QBLOCK
    for t, n in ((blk_ptr, n_qb + 1), (blk_idx, None)):
        if (not isinstance(t, torch.Tensor) or t.device != q.device or t.dtype != torch.int32
                or t.dim() != 1 or not t.is_contiguous() or (n is not None and t.numel() != n)):
            raise ValueError("blk_ptr (ceil(N / 256) + 1) and blk_idx must be contiguous int32 "
                             "device vectors")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _blocksparse(names[q.dtype], q, k, v, out, lse, blk_ptr,
                 blk_idx if blk_idx.numel() else None, blk_idx.numel(), B, H, N, d, scale,
                 causal, stream)
    return out, lse


def attention_backward(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None,
                       stream=None):
    """dq, dk, dv = gradients of attention for [B, H, N, d] device tensors (bf16 or fp16);
    o and lse are what ``attention`` returned for q, k, v."""
    import torch
    for t in (q, k, v, o, dout):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise TypeError("q, k, v, o, dout must be device tensors")
        if not t.is_contiguous() or t.dim() != 4 or t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError("q, k, v, o, dout must be contiguous [B, H, N, d] tensors of one dtype")
    names = {torch.bfloat16: "fa_bwd", torch.float16: "fa_bwd_f16"}
    if q.dtype not in names:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, H, N, d = q.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(max(1, fa_bwd_workspace_bytes(B, H, N) // 4), dtype=torch.float32,
                     device=q.device)
    _bwd(names[q.dtype], q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, N, d, scale, causal, stream)
    return dq, dk, dv


def attention_decode(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """O, LSE of q [B, H, Nq, d] against k, v [B, H, Nk, d] (bf16 or fp16 device tensors), the
    queries being the last Nq positions of the key sequence."""
    import torch
    for t in (q, k, v):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise TypeError("q, k, v must be device tensors")
        if not t.is_contiguous() or t.dim() != 4 or t.dtype != q.dtype:
            raise ValueError("q, k, v must be contiguous 4-d tensors of one dtype")
    names = {torch.bfloat16: "fa_decode", torch.float16: "fa_decode_f16"}
    if q.dtype not in names:
        raise TypeError(f"unsupported dtype {q.dtype}")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, d):
        raise ValueError("k and v must be [B, H, Nk, d] with q's B, H and d")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    nbytes = fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    ws = torch.empty(max(4, nbytes // 4), dtype=torch.float32, device=q.device)
    _decode(names[q.dtype], q, k, v, out, lse, ws, nbytes, B, H, Nq, Nk, d, scale, causal, stream)
    return out, lse


def softmax(x, out=None, stream=None):
    """Row softmax of a contiguous fp32 [rows, cols] device tensor."""
    import torch
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.float32:
        raise TypeError("x must be an fp32 device tensor")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [rows, cols] tensor")
    if out is None:
        out = torch.empty_like(x)
    online_softmax_rows(x, out, x.shape[0], x.shape[1], stream)
    return out


def softmax_split(x, out=None, stream=None):
    """Row softmax of a contiguous fp32 [rows, cols] device tensor, each row spread
    over several workgroups (for few, very long rows)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != torch.float32:
        raise TypeError("x must be an fp32 device tensor")
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [rows, cols] tensor")
    if out is None:
        out = torch.empty_like(x)
    nbytes = online_softmax_split_workspace_bytes(x.shape[0], x.shape[1])
    ws = torch.empty(max(1, nbytes // 4), dtype=torch.float32, device=x.device)
    online_softmax_rows_split(x, out, x.shape[0], x.shape[1], ws, nbytes, stream)
    return out
