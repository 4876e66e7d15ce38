// C ABI of the library: argument validation on the host, then one kernel launch.
// Validation happens before any HIP runtime call, so every error path below is
// reachable and testable without a GPU.
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa.h"
#include "kernels.h"

// Scratch memory of fa_decode_static: the decode partials (m, l, unnormalised
// O) live in this file-scope device array instead of a caller's workspace.
// Every GPU the library runs on holds one copy until the process ends, and
// every fa_decode_static call on that GPU shares it.  In host code `scratch`
// names a host-side stand-in, not the device array: its device address is
// looked up per device with hipGetSymbolAddress (decode_scratch below) and
// only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call per device and kept.
int decode_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bbytes && y < x + abytes;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// Bytes of a B*H*N*d tensor (0 on overflow of 63 bits).
uint64_t tensor_bytes(int B, int H, int N, int d, uint64_t elem) {
  unsigned __int128 n = (unsigned __int128)B * (unsigned __int128)H * (unsigned __int128)N *
                        (unsigned __int128)d * elem;
  if (n >= ((unsigned __int128)1 << 63)) return 0;
  return (uint64_t)n;
}

// mask: osm::kMaskNone, kMaskLocal (doc_start, window) or kMaskSparse (blk_ptr,
// blk_idx, nnz); the masked kernels take 16-bit operands only.
int attn_entry(osm::Elem elem, const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream,
               int mask = osm::kMaskNone, const int* doc_start = nullptr, int window = 0,
               const int* blk_ptr = nullptr, const int* blk_idx = nullptr, int nnz = 0) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  const uint64_t esz = elem == osm::Elem::f32 ? 4 : 2;
  const uint64_t bytes = tensor_bytes(B, H, N, d, esz);
  const uint64_t lse_bytes = tensor_bytes(B, H, N, 1, 4);
  if (bytes == 0 || lse_bytes == 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // one head's tensor is addressed with 32-bit byte offsets
  if ((uint64_t)N * (uint64_t)d * esz >= ((uint64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  // one workgroup per (batch*head, query block) must fit a 1-D grid
  const uint64_t rows_per_block = 128;
  const uint64_t blocks = (uint64_t)B * (uint64_t)H * (((uint64_t)N + rows_per_block - 1) / rows_per_block);
  if (blocks > (uint64_t)INT_MAX) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_ALIGNMENT;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGNMENT;
  if (overlaps(o, bytes, q, bytes) || overlaps(o, bytes, k, bytes) || overlaps(o, bytes, v, bytes))
    return FA_ERR_INVALID_ARG;
  if (lse && (overlaps(lse, lse_bytes, o, bytes) || overlaps(lse, lse_bytes, q, bytes) ||
              overlaps(lse, lse_bytes, k, bytes) || overlaps(lse, lse_bytes, v, bytes)))
    return FA_ERR_INVALID_ARG;
  if (mask == osm::kMaskSparse) {
    // CSR over the query blocks: n_qb + 1 row offsets, nnz key-block indices
    const uint64_t n_qb = ((uint64_t)N + osm::kSparseQBlock - 1) / osm::kSparseQBlock;
    if (!blk_ptr || nnz < 0 || (nnz > 0 && !blk_idx)) return FA_ERR_INVALID_ARG;
    if (!aligned(blk_ptr, 4) || (blk_idx && !aligned(blk_idx, 4))) return FA_ERR_ALIGNMENT;
    const uint64_t ptr_bytes = (n_qb + 1) * 4, idx_bytes = (uint64_t)nnz * 4;
    if (overlaps(blk_ptr, ptr_bytes, o, bytes) || (lse && overlaps(blk_ptr, ptr_bytes, lse, lse_bytes)))
      return FA_ERR_INVALID_ARG;
    if (nnz > 0 && (overlaps(blk_idx, idx_bytes, o, bytes) ||
                    (lse && overlaps(blk_idx, idx_bytes, lse, lse_bytes))))
      return FA_ERR_INVALID_ARG;
    // with nnz = 0 every row range clamps to empty and blk_idx is never read
    hipError_t e = osm::launch_attn_fwd_blocksparse(elem, q, k, v, o, lse, blk_ptr, blk_idx, nnz,
                                                    B, H, N, d, scale, causal != 0, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  if (mask == osm::kMaskLocal) {
    if (window < 0) return FA_ERR_INVALID_ARG;
    if (doc_start) {
      if (!aligned(doc_start, 4)) return FA_ERR_ALIGNMENT;
      const uint64_t doc_bytes = tensor_bytes(B, N, 1, 1, 4);
      if (doc_bytes == 0) return FA_ERR_INVALID_ARG;
      if (overlaps(doc_start, doc_bytes, o, bytes) ||
          (lse && overlaps(doc_start, doc_bytes, lse, lse_bytes)))
        return FA_ERR_INVALID_ARG;
    }
    hipError_t e = osm::launch_attn_fwd_local(elem, q, k, v, o, lse, doc_start, window, B, H, N, d,
                                              scale, stream);
    return e == hipSuccess ? FA_OK : FA_ERR_HIP;
  }
  hipError_t e = osm::launch_attn_fwd(elem, q, k, v, o, lse, B, H, N, d, scale, causal != 0, stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fp8_entry(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
              int N, int d, float scale, float q_descale, float k_descale, float v_descale,
              int causal, hipStream_t stream) {
  if (!q || !k || !v || !o) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  const float f[] = {scale, q_descale, k_descale, v_descale};
  for (float x : f)
    if (!std::isfinite(x) || !(x > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  const uint64_t in_bytes = tensor_bytes(B, H, N, d, 1);
  const uint64_t out_bytes = tensor_bytes(B, H, N, d, 2);
  const uint64_t lse_bytes = tensor_bytes(B, H, N, 1, 4);
  if (in_bytes == 0 || out_bytes == 0 || lse_bytes == 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)N * (uint64_t)d * 2 >= ((uint64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  const uint64_t blocks = (uint64_t)B * (uint64_t)H * (((uint64_t)N + 255) / 256);
  if (blocks > (uint64_t)INT_MAX) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return FA_ERR_ALIGNMENT;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGNMENT;
  if (overlaps(o, out_bytes, q, in_bytes) || overlaps(o, out_bytes, k, in_bytes) ||
      overlaps(o, out_bytes, v, in_bytes))
    return FA_ERR_INVALID_ARG;
  if (lse && (overlaps(lse, lse_bytes, o, out_bytes) || overlaps(lse, lse_bytes, q, in_bytes) ||
              overlaps(lse, lse_bytes, k, in_bytes) || overlaps(lse, lse_bytes, v, in_bytes)))
    return FA_ERR_INVALID_ARG;
  hipError_t e = osm::launch_attn_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, q_descale, k_descale,
                                          v_descale, causal != 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int bwd_entry(osm::Elem elem, const void* q, const void* k, const void* v, const void* o,
              const void* dout, const float* lse, void* dq, void* dk, void* dv, float* workspace,
              int B, int H, int N, int d, float scale, int causal, hipStream_t stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  const uint64_t bytes = tensor_bytes(B, H, N, d, 2);
  const uint64_t row_bytes = tensor_bytes(B, H, N, 1, 4);  // lse and the workspace
  if (bytes == 0 || row_bytes == 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)N * (uint64_t)d * 2 >= ((uint64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  // the dK/dV kernel has the larger grid: one workgroup per 128 keys of a head
  const uint64_t blocks = (uint64_t)B * (uint64_t)H * (((uint64_t)N + 127) / 128);
  if (blocks > (uint64_t)INT_MAX) return FA_ERR_INVALID_ARG;
  const void* in[] = {q, k, v, o, dout};
  for (const void* p : in)
    if (!aligned(p, 16)) return FA_ERR_ALIGNMENT;
  if (!aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(workspace, 16))
    return FA_ERR_ALIGNMENT;
  if (!aligned(lse, 4)) return FA_ERR_ALIGNMENT;
  // outputs (dq, dk, dv, workspace) overlap neither each other nor any input
  const void* outs[] = {dq, dk, dv, workspace};
  const uint64_t out_bytes[] = {bytes, bytes, bytes, row_bytes};
  for (int a = 0; a < 4; ++a) {
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_INVALID_ARG;
    for (const void* p : in)
      if (overlaps(outs[a], out_bytes[a], p, bytes)) return FA_ERR_INVALID_ARG;
    if (overlaps(outs[a], out_bytes[a], lse, row_bytes)) return FA_ERR_INVALID_ARG;
  }
  hipError_t e = osm::launch_attn_bwd(elem, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N,
                                      d, scale, causal != 0, stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

// Workspace of fa_decode: partial O (fp32, d per row) then (m, l) pairs, one
// row per (batch*head, key chunk, query); 0 on invalid sizes or overflow.
uint64_t decode_workspace(int B, int H, int Nq, int Nk, int d, int* n_chunks) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 0;
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  if (bh > (uint64_t)INT_MAX) return 0;
  int nc, ct;
  osm::decode_split_plan((int)bh, Nq, Nk, &nc, &ct);
  if (n_chunks) *n_chunks = nc;
  return tensor_bytes((int)bh, nc, Nq, 1, 4 * (uint64_t)d + 8);
}

// static_scratch: take the partials from the library's scratch array (workspace
// and workspace_bytes are ignored); a call needing more than it holds gets
// FA_ERR_SCRATCH_LIMIT.
int decode_entry(osm::Elem elem, const void* q, const void* k, const void* v, void* o, float* lse,
                 float* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                 float scale, int causal, hipStream_t stream, bool static_scratch = false) {
  if (!q || !k || !v || !o || (!workspace && !static_scratch)) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;  // the queries are the last Nq positions
  const uint64_t qbytes = tensor_bytes(B, H, Nq, d, 2);
  const uint64_t kbytes = tensor_bytes(B, H, Nk, d, 2);
  const uint64_t lse_bytes = tensor_bytes(B, H, Nq, 1, 4);
  if (qbytes == 0 || kbytes == 0 || lse_bytes == 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((uint64_t)Nk * (uint64_t)d * 2 >= ((uint64_t)1 << 31)) return FA_ERR_UNSUPPORTED;
  int n_chunks = 0;
  const uint64_t ws = decode_workspace(B, H, Nq, Nk, d, &n_chunks);
  if (ws == 0) return FA_ERR_INVALID_ARG;
  // grids: one wave per (batch*head, chunk, 32-query group); one merge workgroup per query
  const uint64_t bh = (uint64_t)B * (uint64_t)H;
  if (bh * (uint64_t)n_chunks * (((uint64_t)Nq + 31) / 32) > (uint64_t)INT_MAX ||
      bh * (uint64_t)Nq > (uint64_t)INT_MAX)
    return FA_ERR_INVALID_ARG;
  if (static_scratch) {
    if (ws > (uint64_t)FA_DECODE_STATIC_SCRATCH_BYTES) return FA_ERR_SCRATCH_LIMIT;
  } else if ((uint64_t)workspace_bytes < ws) {
    return FA_ERR_INVALID_ARG;
  }
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      (!static_scratch && !aligned(workspace, 16)))
    return FA_ERR_ALIGNMENT;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGNMENT;
  // outputs (o, lse, workspace) overlap neither each other nor any input
  const void* outs[] = {o, lse, workspace};
  const uint64_t out_bytes[] = {qbytes, lse_bytes, ws};
  for (int a = 0; a < 3; ++a) {
    if (!outs[a]) continue;
    for (int b = a + 1; b < 3; ++b)
      if (outs[b] && overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return FA_ERR_INVALID_ARG;
    if (overlaps(outs[a], out_bytes[a], q, qbytes) || overlaps(outs[a], out_bytes[a], k, kbytes) ||
        overlaps(outs[a], out_bytes[a], v, kbytes))
      return FA_ERR_INVALID_ARG;
  }
  if (static_scratch) {
    // every host-side check has passed: only now touch the runtime
    void* p = nullptr;
    const int st = decode_scratch(&p);
    if (st != FA_OK) return st;
    if (overlaps(o, qbytes, p, ws) || (lse && overlaps(lse, lse_bytes, p, ws)))
      return FA_ERR_INVALID_ARG;
    workspace = static_cast<float*>(p);
  }
  hipError_t e = osm::launch_attn_decode(elem, q, k, v, o, lse, workspace, B, H, Nq, Nk, d, scale,
                                         causal != 0, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  if (d != 64 && d != 128) return 0;
  return (size_t)decode_workspace(B, H, Nq, Nk, d, nullptr);
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
              size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, float scale, int causal,
              hipStream_t stream) {
  return decode_entry(osm::Elem::bf16, q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d,
                      scale, causal, stream);
}

int fa_decode_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                  float* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                  float scale, int causal, hipStream_t stream) {
  return decode_entry(osm::Elem::f16, q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d,
                      scale, causal, stream);
}

int fa_decode_static(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream) {
  return decode_entry(osm::Elem::bf16, q, k, v, o, lse, nullptr, 0, B, H, Nq, Nk, d, scale, causal,
                      stream, true);
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, float scale, int causal, hipStream_t stream) {
  return attn_entry(osm::Elem::bf16, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream) {
  return attn_entry(osm::Elem::f16, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream) {
  return attn_entry(osm::Elem::f32, q, k, v, o, lse, B, H, N, d, scale, causal, stream);
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, float q_descale, float k_descale, float v_descale,
               int causal, hipStream_t stream) {
  return fp8_entry(q, k, v, o, lse, B, H, N, d, scale, q_descale, k_descale, v_descale, causal,
                   stream);
}

int fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                 const int* doc_start, int window, int B, int H, int N, int d, float scale,
                 hipStream_t stream) {
  return attn_entry(osm::Elem::bf16, q, k, v, o, lse, B, H, N, d, scale, 1, stream, osm::kMaskLocal,
                    doc_start, window);
}

int fa_fwd_local_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int* doc_start, int window, int B, int H, int N, int d, float scale,
                     hipStream_t stream) {
  return attn_entry(osm::Elem::f16, q, k, v, o, lse, B, H, N, d, scale, 1, stream, osm::kMaskLocal,
                    doc_start, window);
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int* blk_ptr, const int* blk_idx, int nnz, int B, int H, int N,
                       int d, float scale, int causal, hipStream_t stream) {
  return attn_entry(osm::Elem::bf16, q, k, v, o, lse, B, H, N, d, scale, causal, stream,
                    osm::kMaskSparse, nullptr, 0, blk_ptr, blk_idx, nnz);
}

int fa_fwd_blocksparse_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int* blk_ptr, const int* blk_idx, int nnz, int B, int H, int N,
                           int d, float scale, int causal, hipStream_t stream) {
  return attn_entry(osm::Elem::f16, q, k, v, o, lse, B, H, N, d, scale, causal, stream,
                    osm::kMaskSparse, nullptr, 0, blk_ptr, blk_idx, nnz);
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H, int N,
           int d, float scale, int causal, hipStream_t stream) {
  return bwd_entry(osm::Elem::bf16, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale,
                   causal, stream);
}

int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream) {
  return bwd_entry(osm::Elem::f16, q, k, v, o, dout, lse, dq, dk, dv, workspace, B, H, N, d, scale,
                   causal, stream);
}

size_t fa_bwd_workspace_bytes(int B, int H, int N) {
  if (B < 1 || H < 1 || N < 1) return 0;
  return (size_t)tensor_bytes(B, H, N, 1, 4);
}

int online_softmax_rows(const float* x, float* y, int rows, int cols, hipStream_t stream) {
  if (!x || !y) return FA_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1) return FA_ERR_INVALID_ARG;
  const uint64_t bytes = tensor_bytes(rows, cols, 1, 1, 4);
  if (bytes == 0) return FA_ERR_INVALID_ARG;
  if (!aligned(x, 4) || !aligned(y, 4)) return FA_ERR_ALIGNMENT;
  if (overlaps(x, bytes, y, bytes)) return FA_ERR_INVALID_ARG;
  const bool vec_ok = aligned(x, 16) && aligned(y, 16) && (cols % 4 == 0);
  hipError_t e = osm::launch_softmax(x, y, rows, cols, vec_ok, stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

size_t online_softmax_split_workspace_bytes(int rows, int cols) {
  if (rows < 1 || cols < 1) return 0;
  int chunk, nchunks;
  osm::softmax_split_plan(rows, cols, &chunk, &nchunks);
  return (size_t)tensor_bytes(rows, nchunks, 1, 1, 8);
}

int online_softmax_rows_split(const float* x, float* y, int rows, int cols, float* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (!x || !y || !workspace) return FA_ERR_INVALID_ARG;
  if (rows < 1 || cols < 1) return FA_ERR_INVALID_ARG;
  const uint64_t bytes = tensor_bytes(rows, cols, 1, 1, 4);
  if (bytes == 0) return FA_ERR_INVALID_ARG;
  int chunk, nchunks;
  osm::softmax_split_plan(rows, cols, &chunk, &nchunks);
  const uint64_t ws = tensor_bytes(rows, nchunks, 1, 1, 8);
  // one workgroup per (row, chunk) must fit a 1-D grid
  if (ws == 0 || (uint64_t)rows * (uint64_t)nchunks > (uint64_t)INT_MAX) return FA_ERR_INVALID_ARG;
  if ((uint64_t)workspace_bytes < ws) return FA_ERR_INVALID_ARG;
  if (!aligned(x, 4) || !aligned(y, 4) || !aligned(workspace, 8)) return FA_ERR_ALIGNMENT;
  if (overlaps(x, bytes, y, bytes) || overlaps(workspace, ws, x, bytes) ||
      overlaps(workspace, ws, y, bytes))
    return FA_ERR_INVALID_ARG;
  const bool vec_ok = aligned(x, 16) && aligned(y, 16) && (cols % 4 == 0);
  hipError_t e = osm::launch_softmax_split(x, y, rows, cols, vec_ok, workspace, stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_stream_copy(const void* x, void* y, size_t bytes, hipStream_t stream) {
  if (!x || !y || bytes == 0 || bytes % 16 != 0) return FA_ERR_INVALID_ARG;
  if (bytes >= ((uint64_t)1 << 62) || osm::stream_copy_blocks(bytes) > (uint64_t)INT_MAX)
    return FA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16)) return FA_ERR_ALIGNMENT;
  if (overlaps(x, bytes, y, bytes)) return FA_ERR_INVALID_ARG;
  return osm::launch_stream_copy(x, y, bytes, stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static_assert(FA_MFMA_STREAM_OPERAND_BYTES ==
                  (size_t)osm::kMfmaStreamVariants * osm::kMfmaStreamFragments * 64 * 16,
              "operand layout of the MFMA stream");

int fa_mfma_stream(const void* operands, size_t operand_bytes, float* out, size_t out_floats,
                   int blocks, int iters, hipStream_t stream) {
  if (!operands || !out || blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20))
    return FA_ERR_INVALID_ARG;
  if (operand_bytes < FA_MFMA_STREAM_OPERAND_BYTES || out_floats < (size_t)blocks * 512)
    return FA_ERR_INVALID_ARG;
  if (!aligned(operands, 16) || !aligned(out, 4)) return FA_ERR_ALIGNMENT;
  if (overlaps(operands, FA_MFMA_STREAM_OPERAND_BYTES, out, (size_t)blocks * 512 * sizeof(float)))
    return FA_ERR_INVALID_ARG;
  return osm::launch_mfma_stream(operands, out, blocks, iters, stream) == hipSuccess ? FA_OK
                                                                                     : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: null pointer, size, scale, overlap or overflow";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head dimension without a kernel (64 and 128 are supported)";
    case FA_ERR_ALIGNMENT: return "FA_ERR_ALIGNMENT: pointer not aligned as the operation requires";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported a launch error";
    case FA_ERR_SCRATCH_LIMIT:
      return "FA_ERR_SCRATCH_LIMIT: the call needs more scratch memory than the library's static array holds";
    default: return "unknown fa_status";
  }
}

int fa_kernel_attributes(int op, int d, int causal, fa_kernel_attrs* out) {
  if (!out) return FA_ERR_INVALID_ARG;
  hipFuncAttributes attr;
  int threads = 0, blocks = 0;
  hipError_t e;
  if (op >= 0 && op <= 2) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    const osm::Elem elem = op == 0 ? osm::Elem::bf16 : (op == 1 ? osm::Elem::f16 : osm::Elem::f32);
    e = osm::attn_fwd_attributes(elem, d, causal != 0, &attr, &threads, &blocks);
  } else if (op == 4 || op == 5) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    e = osm::attn_bwd_attributes(osm::Elem::bf16, d, causal != 0, op - 4, &attr, &threads, &blocks);
  } else if (op == 8 || op == 9) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (op == 9 && causal == 0) return FA_ERR_INVALID_ARG;  // the window kernel is causal
    e = osm::attn_fwd_attributes(osm::Elem::bf16, d, causal != 0, &attr, &threads, &blocks,
                                 op == 8 ? osm::kMaskSparse : osm::kMaskLocal);
  } else if (op == 7) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    e = osm::attn_fwd_fp8_attributes(d, causal != 0, &attr, &threads, &blocks);
  } else if (op == 6) {
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    e = osm::attn_decode_attributes(d, causal != 0, &attr, &threads, &blocks);
  } else if (op == 3) {
    if (d < 1) return FA_ERR_INVALID_ARG;
    e = osm::softmax_attributes(d, d % 4 == 0, &attr, &threads, &blocks);
  } else {
    return FA_ERR_INVALID_ARG;
  }
  if (e != hipSuccess) return FA_ERR_HIP;
  out->regs_per_lane = attr.numRegs;
  out->lds_bytes = (int)attr.sharedSizeBytes;
  out->private_bytes = (int)attr.localSizeBytes;
  out->threads_per_block = threads;
  out->blocks_per_cu = blocks;
  return FA_OK;
}

}  // extern "C"
