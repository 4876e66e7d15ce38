// Internal launchers of the HIP library (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>

namespace osm {

enum class Elem { bf16, f16, f32 };

// Key masks of the 16-bit attention forward: none (dense, or causal alone), the
// causal sliding window over packed documents, and block-sparse (per block of
// kSparseQBlock queries, a list of kSparseKBlock-key blocks).
constexpr int kMaskNone = 0, kMaskLocal = 1, kMaskSparse = 2;
constexpr int kSparseQBlock = 256;
constexpr int kSparseKBlock = 128;

// Attention forward on `stream`; arguments already validated by the C ABI layer.
hipError_t launch_attn_fwd(Elem elem, const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream);
hipError_t attn_fwd_attributes(Elem elem, int d, bool causal, hipFuncAttributes* attr,
                               int* threads, int* blocks_per_cu, int mask = kMaskNone);
// Causal attention where query i also skips keys before max(doc_start[b, i], i - window + 1)
// (doc_start may be null, window 0 = unbounded); bf16 / fp16 only.
hipError_t launch_attn_fwd_local(Elem elem, const void* q, const void* k, const void* v, void* o,
                                 float* lse, const int* doc_start, int window, int B, int H, int N,
                                 int d, float scale, hipStream_t stream);
// Block-sparse attention: query block qb (rows 256 qb ..) sees the 128-key blocks
// blk_idx[blk_ptr[qb] .. blk_ptr[qb + 1]) (CSR over ceil(N / 256) query blocks,
// nnz entries, shared by all batches and heads), with causal masking on top.
hipError_t launch_attn_fwd_blocksparse(Elem elem, const void* q, const void* k, const void* v,
                                       void* o, float* lse, const int* blk_ptr,
                                       const int* blk_idx, int nnz, int B, int H, int N, int d,
                                       float scale, bool causal, hipStream_t stream);

// Attention forward with fp8 E4M3 Q/K/V (value = descale * code), bf16 O; d = 64 or 128.
hipError_t launch_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, float scale, float q_descale,
                               float k_descale, float v_descale, bool causal, hipStream_t stream);
hipError_t attn_fwd_fp8_attributes(int d, bool causal, hipFuncAttributes* attr, int* threads,
                                   int* blocks_per_cu);

// Attention backward (bf16 / fp16): dQ and D into `workspace` ([B, H, N] fp32),
// then dK and dV; arguments already validated by the C ABI layer.
hipError_t launch_attn_bwd(Elem elem, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* workspace, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream);
// which: 0 = the dQ kernel, 1 = the dK/dV kernel
hipError_t attn_bwd_attributes(Elem elem, int d, bool causal, int which, hipFuncAttributes* attr,
                               int* threads, int* blocks_per_cu);

// Split-KV attention of Nq queries at the end of Nk keys (bf16 / fp16): partial
// results per key chunk into `workspace`, then the merge; see decode_split_plan
// for the chunking and the workspace layout in attn_decode.hip.
void decode_split_plan(int BH, int Nq, int Nk, int* n_chunks, int* chunk_tiles);
hipError_t launch_attn_decode(Elem elem, const void* q, const void* k, const void* v, void* o,
                              float* lse, float* workspace, int B, int H, int Nq, int Nk, int d,
                              float scale, bool causal, hipStream_t stream);
hipError_t attn_decode_attributes(int d, bool causal, hipFuncAttributes* attr, int* threads,
                                  int* blocks_per_cu);

// Row softmax on `stream`; vec_ok = 16-byte aligned pointers and cols % 4 == 0.
hipError_t launch_softmax(const float* x, float* y, int rows, int cols, bool vec_ok,
                          hipStream_t stream);
hipError_t softmax_attributes(int cols, bool vec_ok, hipFuncAttributes* attr, int* threads,
                              int* blocks_per_cu);
// Split path: chunk length and chunks per row; then the two passes with
// rows * nchunks (m, l) pairs in `workspace`.
void softmax_split_plan(int rows, int cols, int* chunk, int* nchunks);
hipError_t launch_softmax_split(const float* x, float* y, int rows, int cols, bool vec_ok,
                                float* workspace, hipStream_t stream);

// Copy of `bytes` (a multiple of 16, 16-byte aligned) with non-temporal 16-byte
// accesses; the grid size it uses.
uint64_t stream_copy_blocks(uint64_t bytes);
hipError_t launch_stream_copy(const void* x, void* y, size_t bytes, hipStream_t stream);

// MFMA stream: `blocks` workgroups of 8 waves, each wave running iters x 8
// 32x32x16 bf16 MFMAs on operands read once from one of kMfmaStreamVariants sets
// of kMfmaStreamFragments 16-byte fragments per lane (64 lanes); out receives
// blocks x 512 floats.
constexpr int kMfmaStreamVariants = 16;
constexpr int kMfmaStreamFragments = 16;
hipError_t launch_mfma_stream(const void* operands, float* out, int blocks, int iters,
                              hipStream_t stream);

}  // namespace osm
