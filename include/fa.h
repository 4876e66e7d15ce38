/*
 * fa.h -- C ABI of the MI355X (gfx950) attention-forward and row-softmax library.
 *
 * Three operations, all from the pages on online softmax:
 *
 *  - fa_fwd*: the attention forward pass O = softmax(scale * Q K^T) V computed
 *    tile by tile with the online-softmax recurrence, so the N x N score
 *    matrix never reaches device memory.  The running statistics follow the
 *    update equations of "Online softmax, and the register that can't move"
 *    (section "Online softmax"): per query row, m_new = max(m_old, rowmax S),
 *    l and O both rescaled by exp(m_old - m_new), O / l once after the last
 *    key tile.  The causal rule (query i sees keys j <= i) and the skipping of
 *    key tiles that lie wholly after the query tile follow the causal
 *    paragraphs of "Online Softmax: Tiling Across a Reduction".  The per-row
 *    statistic saved for a backward pass is the natural-log logsumexp
 *    lse_i = ln sum_j exp(scale * q_i . k_j) over the visible keys (the same
 *    page stores the final maximum and sum; one logsumexp carries both).
 *
 *  - fa_bwd*: the gradients of that forward pass, by recomputation from the
 *    saved statistic (backward-pass paragraphs of the same page).
 *
 *  - online_softmax_rows: y = softmax(x) along each row, with the maximum and
 *    the sum of exponentials gathered in one fused pass and merged across
 *    threads by the associative (m, d) rule of the infra-guide page
 *    "5.2 CUDA Online Softmax" (sections 2.1 and 4.2), then one normalise
 *    pass.  online_softmax_rows_split spreads each row over several
 *    workgroups for few, very long rows.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state between calls, so concurrent calls
 *    on different streams are safe.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream); the
 *    call returns once the kernel is launched.  Outputs are valid after the
 *    stream is synchronised.
 *  - Return value: FA_OK or a negative fa_status.  Argument errors are found
 *    on the host before anything is enqueued and nothing is written; a launch
 *    failure reported by the HIP runtime is FA_ERR_HIP.  Nothing is printed
 *    and nothing aborts.
 *  - Layouts are dense row-major: Q, K, V, O are [B, H, N, d] (d fastest),
 *    LSE is [B, H, N], softmax X and Y are [rows, cols].  Element offsets are
 *    64-bit.
 */
#ifndef ONLINE_SOFTMAX_04_AMD_FA_H
#define ONLINE_SOFTMAX_04_AMD_FA_H

#include <stddef.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null pointer, size < 1, bad scale, overlapping buffers, size overflow */
  FA_ERR_UNSUPPORTED = -2, /* a head dimension the library has no kernel for (d other than 64, 128) */
  FA_ERR_ALIGNMENT = -3,   /* a pointer without the alignment the operation needs */
  FA_ERR_HIP = -4,         /* the HIP runtime reported an error at launch */
  FA_ERR_SCRATCH_LIMIT = -5 /* fa_decode_static: the sizes need more than its static scratch */
} fa_status;

/*
 * Attention forward, bfloat16 Q/K/V/O, fp32 accumulation and statistics.
 *
 *  q, k, v  [B, H, N, d] bfloat16, 16-byte aligned, read only (may alias each other).
 *  o        [B, H, N, d] bfloat16, 16-byte aligned, written; must not overlap q, k, v or lse.
 *  lse      [B, H, N] fp32, 4-byte aligned, written; may be NULL (not written).
 *  B, H, N  >= 1; B*H*N*d must fit in 63 bits.
 *  d        head dimension: 64 or 128 (else FA_ERR_UNSUPPORTED).
 *           One head (N*d elements) must span less than 2 GiB (else FA_ERR_UNSUPPORTED).
 *  scale    softmax scale applied to the fp32 dot products (typically 1/sqrt(d));
 *           must be finite and > 0.
 *  causal   0: every query sees all N keys; 1: query i sees keys j <= i.
 *  O is rounded to bfloat16 (nearest even) once, after the division by l.
 *  Arithmetic: scores and all statistics in fp32; P is rounded to bfloat16
 *  for the P V product, and l sums that same rounded P, so each output row is
 *  a convex combination of V rows.  The maximum subtracted before
 *  exponentiation is a reference that moves to the running row maximum only
 *  when that has grown by more than a factor 2^8; since O and l carry the
 *  same factor, O / l and lse do not depend on when it moves.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Same contract with IEEE half-precision Q/K/V/O. */
int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Causal attention forward with structured masks as tile skips (sliding
 * windows and document boundaries, the structured-mask paragraph of "Online
 * Softmax: Tiling Across a Reduction"), bfloat16 operands: query i of batch b
 * sees keys j with lo_i <= j <= i, where
 *   lo_i = max(doc_start[b * N + i], i - window + 1)     (clamped to 0 .. i).
 *  doc_start  [B, N] int32, 4-byte aligned, read only: the first position of the
 *             document that position i belongs to (packed sequences), shared
 *             by every head; NULL = one document per batch row.
 *  window     keys per query including itself; 0 = unbounded.
 *  Key tiles wholly before a query block's smallest lo_i or after its
 *  diagonal are never read; tiles crossing a bound are masked element by
 *  element.  Every other argument, layout, error and the arithmetic are those
 *  of fa_fwd with causal = 1; lse is over the visible keys.
 */
int fa_fwd_local(const void* q, const void* k, const void* v, void* o, float* lse,
                 const int* doc_start, int window, int B, int H, int N, int d, float scale,
                 hipStream_t stream);

/* Same contract with IEEE half-precision Q/K/V/O. */
int fa_fwd_local_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                     const int* doc_start, int window, int B, int H, int N, int d, float scale,
                     hipStream_t stream);

/*
 * Attention forward under a block-sparse pattern, the block-level skip of the
 * structured-sparsity paragraph of "Online Softmax: Tiling Across a Reduction",
 * bfloat16 operands.  Queries are grouped in blocks of 256 rows (query block qb
 * = rows 256 qb .. 256 qb + 255) and keys in blocks of 128; query i of every
 * batch and head sees the keys of the key blocks listed for its query block,
 *   blk_idx[blk_ptr[qb]] .. blk_idx[blk_ptr[qb + 1] - 1],   qb = i / 256,
 * keys j < N only, and with causal = 1 only keys j <= i.
 *  blk_ptr  int32[ceil(N / 256) + 1], device, 4-byte aligned, read only:
 *           CSR row offsets, blk_ptr[0] = 0, non-decreasing, last = nnz.
 *  blk_idx  int32[nnz], device, 4-byte aligned, read only: key-block indices
 *           in 0 .. ceil(N / 128) - 1, ascending and distinct within a query
 *           block (may be NULL when nnz = 0).
 *  nnz      number of listed (query block, key block) pairs, >= 0.
 *  Only listed key blocks are read from memory.  A query that sees no key
 *  (an empty list, or causal with every listed key after it) gets O = 0 and
 *  lse = -inf.  Row offsets are clamped to 0 .. nnz, and a block index outside
 *  0 .. ceil(N / 128) - 1 contributes no keys, so no pattern makes the kernel
 *  read or write outside its buffers; a block listed twice is counted twice.
 *  Every other argument, layout, error and the arithmetic are those of fa_fwd;
 *  blk_ptr and blk_idx may not overlap o or lse (FA_ERR_INVALID_ARG).
 */
int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int* blk_ptr, const int* blk_idx, int nnz, int B, int H, int N,
                       int d, float scale, int causal, hipStream_t stream);

/* Same contract with IEEE half-precision Q/K/V/O. */
int fa_fwd_blocksparse_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int* blk_ptr, const int* blk_idx, int nnz, int B, int H, int N,
                           int d, float scale, int causal, hipStream_t stream);

/*
 * Attention forward with fp8 operands: Q, K, V hold OCP fp8 E4M3 codes (1 byte;
 * sign, 4-bit exponent with bias 7, 3-bit mantissa, largest finite 448, no
 * infinities), and the value of an element is its tensor's descale times the
 * code's value.  O = softmax(scale * Qv Kv^T) Vv is written in bf16 and the
 * logsumexp of the scaled scores in fp32, as for fa_fwd.  Both products run on
 * the fp8 MFMA with fp32 accumulation; P is rounded to E4M3 (as 2^7 P, with a
 * reference maximum that trails the row maximum by at most 1.5 in log2 units,
 * so every stored weight stays below 448) and the row sum is taken over the
 * rounded values.  fp8 as the next precision step
 * is the one the "100 Days of GPU, Day 97" page names for its follow-up.
 *
 *  q, k, v    [B, H, N, d] E4M3 codes, 16-byte aligned, read only.
 *  o          [B, H, N, d] bf16, 16-byte aligned, written.
 *  lse        [B, H, N] fp32 or NULL.
 *  q_descale, k_descale, v_descale  finite, > 0 (else FA_ERR_INVALID_ARG).
 *  d = 64 or 128 (else FA_ERR_UNSUPPORTED).  Every other argument, layout and
 *  error is that of fa_fwd.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
               int N, int d, float scale, float q_descale, float k_descale, float v_descale,
               int causal, hipStream_t stream);

/* Same contract with fp32 Q/K/V/O: products and sums in fp32 throughout, no
 * reduced-precision operand anywhere (the fp32 workloads' path). */
int fa_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * Decode-shaped attention: Nq queries against Nk keys, the queries being the
 * last Nq positions of the key sequence (one new token per head, a few
 * speculative tokens, or a prefill chunk over a cached prefix).  The key range
 * of each head is cut into chunks that separate waves process with the
 * online-softmax recurrence; each leaves a partial (m, l, unnormalised O) per
 * query in `workspace`, and a second kernel merges a query's partials with the
 * associative rule of two partial results, each with its own maximum, rescaled
 * to the larger one ("100 Days of GPU, Day 97", Solution).  Split-KV keeps
 * about 2048 waves busy even when B*H*Nq is small.
 *
 *  q          [B, H, Nq, d] bf16, read only.
 *  k, v       [B, H, Nk, d] bf16, read only.
 *  o          [B, H, Nq, d] bf16, written.
 *  lse        [B, H, Nq] fp32 natural-log logsumexp over the visible keys, or NULL.
 *  workspace  device memory of at least fa_decode_workspace_bytes(B, H, Nq,
 *             Nk, d) bytes, 16-byte aligned, owned by the caller; contents
 *             on entry ignored, scratch on exit.  Calls that share it must be
 *             ordered (the same stream does that).
 *  workspace_bytes  its size; a smaller value returns FA_ERR_INVALID_ARG.
 *  causal     1: query i (0-based) sees keys 0 .. Nk - Nq + i, and needs
 *             Nq <= Nk; 0: every query sees all Nk keys (any Nq).
 *  d in {64, 128} (else FA_ERR_UNSUPPORTED); Nk * d * 2 < 2^31.
 *  q, k, v, o 16-byte aligned (FA_ERR_ALIGNMENT); o, lse and workspace overlap
 *  neither each other nor an input (FA_ERR_INVALID_ARG).  Every other
 *  convention and the arithmetic (fp32 scores, P rounded to 16 bits, the
 *  trailing reference maximum) are those of fa_fwd.
 */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d);
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, float* workspace,
              size_t workspace_bytes, int B, int H, int Nq, int Nk, int d, float scale, int causal,
              hipStream_t stream);

/* Same contract with IEEE half-precision Q/K/V/O. */
int fa_decode_f16(const void* q, const void* k, const void* v, void* o, float* lse,
                  float* workspace, size_t workspace_bytes, int B, int H, int Nq, int Nk, int d,
                  float scale, int causal, hipStream_t stream);

/*
 * fa_decode without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine) and clears nothing; the partials live in a
 * static device array of FA_DECODE_STATIC_SCRATCH_BYTES that the library holds
 * on every GPU it runs on until the process ends (its address is looked up
 * once per device, on the first call there).
 *
 *  Arguments, layouts, arithmetic and results are those of fa_decode (bf16)
 *  with the workspace taken from that array.
 *  FA_ERR_SCRATCH_LIMIT when fa_decode_workspace_bytes(B, H, Nq, Nk, d)
 *  exceeds FA_DECODE_STATIC_SCRATCH_BYTES (every other error as fa_decode).
 *  Every call on one GPU shares that GPU's array and leaves its partials
 *  there: calls that overlap in time on one GPU (different streams, or other
 *  host threads, without ordering between them) race on it and give wrong
 *  results.  Calls ordered on one stream are safe.
 */
#define FA_DECODE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
int fa_decode_static(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Nq, int Nk, int d, float scale, int causal, hipStream_t stream);

/*
 * Attention backward: the gradients dQ, dK, dV of O = softmax(scale * Q K^T) V
 * for an upstream gradient dO, bfloat16 operands, fp32 accumulation.
 *
 * The N x N weights are not stored by the forward pass; they are recomputed
 * tile by tile from Q and K and normalised in one step with the saved per-row
 * statistic (the backward-pass paragraphs of "Online Softmax: Tiling Across
 * a Reduction"): P = exp(scale * q_i . k_j - lse_i).  With D_i = <dO_i, O_i>:
 *   dV = P^T dO,  dS = P o (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 *  q, k, v, o, dout [B, H, N, d] bfloat16, 16-byte aligned, read only; o is
 *           the forward output for these q, k, v (it enters through D only).
 *  lse      [B, H, N] fp32, 4-byte aligned, read only: the natural-log
 *           logsumexp that fa_fwd writes.
 *  dq, dk, dv [B, H, N, d] bfloat16, 16-byte aligned, written; they must not
 *           overlap each other, the workspace or any input.
 *  workspace  fp32, 16-byte aligned, at least fa_bwd_workspace_bytes(B, H, N)
 *           bytes, owned by the caller, overwritten (it carries D between the
 *           two kernels of the call; no state survives the call).
 *  B, H, N, d, scale, causal: as for fa_fwd (d is 64 or 128).
 *  Arithmetic: scores, P, dP, dS and all sums in fp32; P and dS are rounded
 *  to bfloat16 for their matrix products; outputs are rounded once.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H, int N,
           int d, float scale, int causal, hipStream_t stream);

/* Same contract with IEEE half-precision q, k, v, o, dout, dq, dk, dv. */
int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, float* workspace, int B, int H,
               int N, int d, float scale, int causal, hipStream_t stream);

/* Workspace bytes fa_bwd needs for these sizes (4 B H N), 0 if a size is < 1
 * or the product overflows. */
size_t fa_bwd_workspace_bytes(int B, int H, int N);

/*
 * Row softmax: y[r, :] = exp(x[r, :] - max_r) / sum_j exp(x[r, j] - max_r).
 *
 *  x     [rows, cols] fp32, 4-byte aligned, read only.
 *  y     [rows, cols] fp32, 4-byte aligned, written; must not overlap x.
 *  rows, cols >= 1; rows*cols must fit in 63 bits.
 *  Rows of up to 32768 columns (with cols a multiple of 4 and both pointers
 *  16-byte aligned) are read from device memory once and written once; longer
 *  or unaligned rows take a two-read path.  Inputs must be finite.
 */
int online_softmax_rows(const float* x, float* y, int rows, int cols, hipStream_t stream);

/*
 * Row softmax for few, very long rows: the same result as online_softmax_rows,
 * with each row cut into chunks that separate workgroups reduce to a partial
 * (maximum, sum) pair, which are then merged with the associative rescaling
 * rule.  Follows the infra-guide page "5.2 CUDA Online Softmax": the merge of
 * two partial results (section 4.1) and its remark that a tiny row count with
 * huge rows needs several blocks per row in a two-phase launch (section 7.1).  Phase 1 writes one (m, l) pair per chunk to `workspace`;
 * phase 2 merges the row's pairs in every workgroup and normalises its chunk.
 * Each element is read twice and written once (12 bytes per element); no
 * workgroup waits on another.
 *
 *  x, y       as for online_softmax_rows (y must not overlap x).
 *  workspace  device memory of at least online_softmax_split_workspace_bytes
 *             (rows, cols) bytes, 8-byte aligned, overlapping neither x nor
 *             y; owned by the caller, contents on entry ignored, scratch on
 *             exit.  Calls that share a workspace must be ordered (the same
 *             stream does that).
 *  workspace_bytes  its size; a smaller value returns FA_ERR_INVALID_ARG.
 *  Chunks hold at least 4096 columns and the launch aims at about 2048
 *  workgroups; rows * chunks must fit in a 31-bit grid.  Inputs must be finite.
 */
size_t online_softmax_split_workspace_bytes(int rows, int cols);
int online_softmax_rows_split(const float* x, float* y, int rows, int cols, float* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * Measurement utility: y[0 .. bytes) = x[0 .. bytes) with 16-byte non-temporal
 * loads and stores, the practical HBM ceiling of a streaming kernel (one read
 * and one write per byte, as the register-cached row softmax moves; "5.2 CUDA
 * Online Softmax", section 6).  Benchmarks time it beside the softmax and use
 * it as the kernel of known size that calibrates byte counters.
 *  x, y   device pointers, 16-byte aligned (FA_ERR_ALIGNMENT), not overlapping.
 *  bytes  a positive multiple of 16 (else FA_ERR_INVALID_ARG).
 */
int fa_stream_copy(const void* x, void* y, size_t bytes, hipStream_t stream);

/*
 * Measurement utility: a stream of 32x32x16 bf16 matrix-unit products with
 * operands held in registers, the ceiling of a dense contraction on this part
 * for the given operand data (the attention forward is one: "Online Softmax:
 * Tiling Across a Reduction", the matrix-unit paragraphs).  The matrix units'
 * power draw depends on how many operand bits switch, and the clock falls with
 * it, so benchmarks run this on operands drawn like the attention inputs.
 * blocks workgroups of 512 threads; every wave runs iters * 8 products
 * (iters * 8 * 32768 FLOP per wave, blocks * 8 waves).
 *  operands  device pointer to FA_MFMA_STREAM_OPERAND_BYTES bytes of bf16 values
 *            (16 sets of 64 lanes x 16 fragments x 16 bytes; a wave uses set
 *            (global wave index % 16); fragments 0-7 are the A operands, 8-15
 *            the B operands), 16-byte aligned (FA_ERR_ALIGNMENT);
 *            operand_bytes its size (smaller: FA_ERR_INVALID_ARG).
 *  out       device pointer to out_floats >= blocks * 512 floats, 4-byte aligned,
 *            not overlapping operands: each thread's sum of its accumulators.
 *  blocks, iters  in [1, 2^20] (else FA_ERR_INVALID_ARG).
 */
#define FA_MFMA_STREAM_OPERAND_BYTES ((size_t)16 * 16 * 64 * 16)
int fa_mfma_stream(const void* operands, size_t operand_bytes, float* out, size_t out_floats,
                   int blocks, int iters, hipStream_t stream);

/* Static description of an fa_status value (never NULL). */
const char* fa_status_string(int status);

/*
 * Resources of the kernel an entry point would launch for a shape, for
 * reports: registers per lane (arch + accumulation VGPRs as the runtime
 * reports them), LDS bytes per workgroup, private (spill) bytes per lane,
 * threads per workgroup and resident workgroups per compute unit.
 *  op: 0 = fa_fwd, 1 = fa_fwd_f16, 2 = fa_fwd_f32, 3 = online_softmax_rows,
 *  4 = fa_bwd's dQ kernel, 5 = fa_bwd's dK/dV kernel, 6 = fa_decode's
 *  chunk kernel, 7 = fa_fwd_fp8, 8 = fa_fwd_blocksparse, 9 = fa_fwd_local
 *  (causal = 1 only)
 *  (for op 3, `d` carries cols and `causal` is ignored).
 */
typedef struct {
  int regs_per_lane;
  int lds_bytes;
  int private_bytes;
  int threads_per_block;
  int blocks_per_cu;
} fa_kernel_attrs;

int fa_kernel_attributes(int op, int d, int causal, fa_kernel_attrs* out);

#ifdef __cplusplus
}
#endif

#endif /* ONLINE_SOFTMAX_04_AMD_FA_H */
