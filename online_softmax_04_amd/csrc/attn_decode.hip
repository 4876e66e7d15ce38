// Split-KV attention for few queries against many keys (decode, speculative
// decode, chunked prefill): O = softmax(scale * Q K^T) V for Nq queries that sit
// at the last Nq positions of an Nk-key sequence, bf16 / fp16 operands on the
// 32x32x16 MFMA, fp32 accumulation.
//
// Why split.  With one workgroup per (batch*head, query block), a decode step
// (Nq = 1) gives B*H workgroups, each streaming the head's whole K and V: 256
// heads cannot fill 256 CUs with enough loads in flight.  The key range of a
// head is cut into chunks instead; each wave runs the online-softmax recurrence
// over its chunk and leaves a partial result (m, l, unnormalised O), and a
// second kernel merges the partials of each query.  The merge is associative:
// each partial's l and O are taken from its own reference m to the largest m
// of the query by one factor 2^(m_s - M), then summed (the merge of partial
// results in "100 Days of GPU, Day 97", section "Solution"):
//     M = max_s m_s,  l = sum_s l_s 2^(m_s - M),  O = sum_s O_s 2^(m_s - M) / l.
// No wave waits on another; the kernel boundary orders the two phases.
//
// Per chunk the arithmetic is the forward kernel's: S^T = K Q^T with the wave's
// 32 queries (lane = query) as the B operand held in VGPRs, the online update of
// "Online softmax, and the register that can't move" (section "Online softmax")
// with a reference maximum trailing the running one by at most 2^8, P rounded to
// 16 bits and summed as rounded, O^T += V^T P^T.  Causal (query i sees keys
// 0 .. Nk - Nq + i) masks element by element only in the tiles that reach past
// the first query's last key, and tiles wholly past the last query's are never
// read ("Online Softmax: Tiling Across a Reduction", causal paragraphs).
//
// Memory.  Every K/V byte is used by one wave only (a query group of 32), so a
// wave stages its own 32-key tiles: direct buffer loads into a private
// double-buffered LDS ring (K and V separately), the next tile in flight while
// the current one is computed, no workgroup barrier anywhere.  The workgroup is
// one wave; the LDS ring (32 KiB at d = 128) sets how many waves share a CU.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace osm {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
// acc + x.lo + x.hi for a word holding two 16-bit values (one dot2 instruction)
template <typename T>
__device__ __forceinline__ float add_pair16(unsigned x, float acc);
template <>
__device__ __forceinline__ float add_pair16<__bf16>(unsigned x, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                         __builtin_bit_cast(bf16x2, 0x3f803f80u), acc, false);
}
template <>
__device__ __forceinline__ float add_pair16<_Float16>(unsigned x, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, 0x3c003c00u),
                                acc, false);
}

typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr float kSlack = 8.f;   // how far (log2 units) the running maximum may pass m
constexpr int kTileKeys = 32;   // keys per tile

// Phase 1.  Workgroup = one wave = (batch*head, chunk, 32-query group).
// Writes, for each of its valid queries q: part_o[(bh, chunk, q), :] = O (not
// normalised, against reference m) and part_ml[(bh, chunk, q)] = (m, l), m in
// units of log2 (scale already folded in).
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(64) void attn_decode_partial(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int Nq, int Nk, int n_qg, int n_chunks, int chunk_tiles, float c) {
  using v8 = typename Mma<T>::v8;
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kTileKeys * ROW_BYTES;  // one K or V tile
  constexpr int ND = D / 32;                         // 32-dim blocks of O^T
  constexpr int NK = D / 16;                         // 16-deep MFMA steps of K Q^T
  constexpr int CPR = D / 8;                         // 16-byte chunks per row
  constexpr int RPI = 1024 / ROW_BYTES;              // rows per 1 KiB wave-wide load
  constexpr int NI = TILE_BYTES / 1024;              // such loads per tile
  // One array per stage and operand, always indexed with a compile-time stage:
  // the compiler then knows which array each pending direct load writes, and a
  // read of one stage does not wait for the loads into the other.
  __shared__ __attribute__((aligned(1024))) unsigned char k0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char k1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char v1[TILE_BYTES];

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hf = lane >> 5;
  const int id = blockIdx.x;
  const int qg = id % n_qg;
  const int chunk = (id / n_qg) % n_chunks;
  const int bh = id / (n_qg * n_chunks);
  const int qw0 = qg * 32;          // first query of this wave
  const int qi = qw0 + l32;         // this lane's query
  const int off_q = Nk - Nq;        // position of query 0 in the key sequence

  // key tiles of this chunk, cut at the last key any of the wave's queries sees
  const int n_tiles = (Nk + kTileKeys - 1) / kTileKeys;
  const int t_begin = chunk * chunk_tiles;
  int t_end = min(n_tiles, t_begin + chunk_tiles);
  if (CAUSAL) t_end = min(t_end, (off_q + min(qw0 + 31, Nq - 1)) / kTileKeys + 1);

  // ---- Q^T fragments: B operand, lane = query, 8 consecutive head dims; queries
  // past Nq fall outside the buffer and read as zero
  const size_t qbase = (size_t)bh * Nq * D;
  v8 qf[NK];
  {
    const auto rq = make_rsrc(Q + qbase + (size_t)qw0 * D, (int64_t)(Nq - qw0) * ROW_BYTES);
    const int off = l32 * ROW_BYTES + 16 * hf;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
      qf[kb] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 32 * kb, 0, 0));
  }

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  const size_t kvbase = (size_t)bh * Nk * D;
  const uint16_t* Kh = K + kvbase;
  const uint16_t* Vh = V + kvbase;
  // loader: lane i's 16 bytes land at LDS + 16 i of each 1 KiB piece; it fetches
  // the global chunk that its LDS slot holds under the swizzle.  Rows past Nk
  // fall outside the buffer and land as zeros.
  int kgoff[NI], vgoff[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int row = j * RPI + lane / CPR;
    const int p = lane % CPR;
    kgoff[j] = row * ROW_BYTES + (p ^ kswz<D>(row)) * 16;
    vgoff[j] = row * ROW_BYTES + (p ^ vswz<D>(row)) * 16;
  }
  // (a tile with `real` false is an empty buffer: its loads fetch nothing and
  // land as zeros, so every step issues the same loads and waits the same counts)
  auto load_tile = [&](int t, bool real, unsigned char* kdst, unsigned char* vdst) {
    const int64_t rest = real ? (int64_t)(Nk - t * kTileKeys) * ROW_BYTES : 0;
    const auto rk = make_rsrc(Kh + (size_t)t * kTileKeys * D, rest);
#pragma unroll
    for (int j = 0; j < NI; ++j) load16_to_lds_nt(rk, kdst + j * 1024, kgoff[j]);
    const auto rv = make_rsrc(Vh + (size_t)t * kTileKeys * D, rest);
#pragma unroll
    for (int j = 0; j < NI; ++j) load16_to_lds_nt(rv, vdst + j * 1024, vgoff[j]);
  };

  // operand read offsets, as in the forward kernel (K: row l32, logical chunk
  // 2 kb + hf; V^T: transposed 8-byte reads, keys in the P^T permutation)
  int kroff[NK];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) kroff[kb] = l32 * ROW_BYTES + ((2 * kb + hf) ^ kswz<D>(l32)) * 16;
  int vroff[ND];
  {
    const int q = lane & 15;
    const int row = 4 * hf + (q >> 2);
    const int col = 16 * ((lane >> 4) & 1) + 4 * (q & 3);
#pragma unroll
    for (int db = 0; db < ND; ++db)
      vroff[db] = row * ROW_BYTES + (((col + 32 * db) >> 3) ^ vswz<D>(row)) * 16 + (col & 7) * 2;
  }

  // One tile from stage S (0: k0/v0, 1: k1/v1), the next one loading into the other.
  auto step = [&](int t, auto stage_tag) {
    constexpr int S = decltype(stage_tag)::value;
    const unsigned char* Kt = S == 0 ? k0 : k1;
    const unsigned char* Vt = S == 0 ? v0 : v1;
    // the next tile goes into the other stage, whose reads (tile t - 1) were all
    // consumed by MFMAs of the previous step
    load_tile(t + 1, t + 1 < t_end, S == 0 ? k1 : k0, S == 0 ? v1 : v0);
    // K(t) landed: at most V(t) and the next tile's loads still outstanding
    wait_vmem<3 * NI>();

    // S^T = K(t) Q^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      const v8 kf = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(Kt + kroff[kb]));
      s = Mma<T>::run(kf, qf[kb], s);
    }

    // online softmax of the tile
    const int j0 = t * kTileKeys;
    if (j0 + kTileKeys > Nk || (CAUSAL && j0 + kTileKeys - 1 > off_q + qw0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (key >= Nk || (CAUSAL && key > off_q + qi)) s[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_halves(mx);
    const float m_cand = fmaxf(m_run, mx * c);
    const float m_new = (m_cand > m_run + kSlack) ? m_cand : m_run;
    const float m_sub = (m_new == kNegInf) ? 0.f : m_new;  // a fully masked row stays empty
    const float alpha = exp2_fast(m_run - m_sub);
    v8 pf[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) pf[r >> 3][r & 7] = (T)exp2_fast(fmaf(s[r], c, -m_sub));
    float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const u32x4 w = __builtin_bit_cast(u32x4, pf[kb]);
#pragma unroll
      for (int e = 0; e < 4; ++e) ls[e] = add_pair16<T>(w[e], ls[e]);
    }
    l_run = fmaf(l_run, alpha, (ls[0] + ls[1]) + (ls[2] + ls[3]));
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
    }

    // V(t) landed: at most the next tile's loads outstanding
    wait_vmem<2 * NI>();
    // O^T += V^T(t) P^T(t)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const unsigned char* pa = Vt + vroff[db] + 16 * kb * ROW_BYTES;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 8 * ROW_BYTES));
        const v8 vf = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = Mma<T>::run(vf, pf[kb], o[db]);
      }
    }
  };

  if (t_begin < t_end) load_tile(t_begin, true, k0, v0);
  for (int t = t_begin; t < t_end; t += 2) {
    step(t, StageTag<0>{});
    if (t + 1 < t_end) step(t + 1, StageTag<1>{});
  }
  wait_vmem<0>();  // the last step's empty loads

  // ---- the partial result of each valid query (a chunk without visible keys
  // leaves m = -inf, l = 0, O = 0, which the merge weighs by zero)
  const float l_tot = sum_halves(l_run);
  if (qi < Nq) {
    const size_t row = ((size_t)bh * n_chunks + chunk) * Nq + qi;
    float* po = part_o + row * D;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4v w = {o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
        *reinterpret_cast<f32x4v*>(po + 32 * db + 8 * g + 4 * hf) = w;
      }
    }
    if (hf == 0) part_ml[row] = make_float2(m_run, l_tot);
  }
}

// Phase 2.  One workgroup of D threads per (batch*head, query): the threads
// first find M over the chunks together, then take the chunks D at a time --
// thread i turns pair i into its weight 2^(m - M) in LDS -- and thread e sums
// head dim e of O over them.  Every load of a step is independent of the others,
// so the partials stream in parallel rather than one chunk after another.
// Thread e writes O[e] in the storage type; thread 0 the natural-log logsumexp
// ln 2 * (M + log2 l).
template <typename T, int D>
__global__ __launch_bounds__(D) void attn_decode_merge(const float* __restrict__ part_o,
                                                       const float2* __restrict__ part_ml,
                                                       uint16_t* __restrict__ O,
                                                       float* __restrict__ LSE, int Nq,
                                                       int n_chunks) {
  __shared__ float red[D / 64];
  __shared__ float wgt[D], lw[D];
  const int e = threadIdx.x;
  const int bh = blockIdx.x / Nq, q = blockIdx.x - bh * Nq;
  const size_t row0 = (size_t)bh * n_chunks * Nq + q;  // chunk s at row0 + s * Nq
  float M = kNegInf;
  for (int s = e; s < n_chunks; s += D) M = fmaxf(M, part_ml[row0 + (size_t)s * Nq].x);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((e & 63) == 0) red[e >> 6] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int w = 1; w < D / 64; ++w) M = fmaxf(M, red[w]);
  float l = 0.f, acc = 0.f;
  for (int s0 = 0; s0 < n_chunks; s0 += D) {
    const int cnt = min(D, n_chunks - s0);
    __syncthreads();  // the previous step's weights are no longer read
    if (e < cnt) {
      const float2 ml = part_ml[row0 + (size_t)(s0 + e) * Nq];
      const float w = exp2_fast(ml.x - M);  // 0 for a chunk that saw no key
      wgt[e] = w;
      lw[e] = ml.y * w;
    }
    __syncthreads();
    const float* po = part_o + (row0 + (size_t)s0 * Nq) * D + e;
#pragma unroll 8
    for (int i = 0; i < cnt; ++i) {
      acc = fmaf(po[(size_t)i * Nq * D], wgt[i], acc);
      l += lw[i];
    }
  }
  const size_t out = ((size_t)bh * Nq + q) * D + e;
  O[out] = __builtin_bit_cast(uint16_t, (T)(acc / l));
  if (LSE != nullptr && e == 0) LSE[(size_t)bh * Nq + q] = (M + log2f(l)) * kLn2;
}

template <typename T, int D, bool C>
hipError_t launch_typed(const void* q, const void* k, const void* v, void* o, float* lse,
                        float* workspace, int BH, int Nq, int Nk, float c, hipStream_t stream) {
  int n_chunks, chunk_tiles;
  decode_split_plan(BH, Nq, Nk, &n_chunks, &chunk_tiles);
  const int n_qg = (Nq + 31) / 32;
  const size_t rows = (size_t)BH * n_chunks * Nq;
  float* part_o = workspace;
  float2* part_ml = reinterpret_cast<float2*>(workspace + rows * D);
  const float2* cpart_ml = part_ml;
  const float* cpart_o = part_o;
  const uint16_t* Qp = static_cast<const uint16_t*>(q);
  const uint16_t* Kp = static_cast<const uint16_t*>(k);
  const uint16_t* Vp = static_cast<const uint16_t*>(v);
  uint16_t* Op = static_cast<uint16_t*>(o);
  void* a1[] = {(void*)&Qp, (void*)&Kp, (void*)&Vp, (void*)&part_o, (void*)&part_ml, (void*)&Nq,
                (void*)&Nk, (void*)&n_qg, (void*)&n_chunks, (void*)&chunk_tiles, (void*)&c};
  hipError_t e = hipLaunchKernel((const void*)attn_decode_partial<T, D, C>,
                                 dim3(BH * n_chunks * n_qg), dim3(64), a1, 0, stream);
  if (e != hipSuccess) return e;
  void* a2[] = {(void*)&cpart_o, (void*)&cpart_ml, (void*)&Op, (void*)&lse, (void*)&Nq,
                (void*)&n_chunks};
  return hipLaunchKernel((const void*)attn_decode_merge<T, D>, dim3(BH * Nq), dim3(D), a2, 0,
                         stream);
}

template <typename T>
hipError_t launch_elem(int d, bool causal, const void* q, const void* k, const void* v, void* o,
                       float* lse, float* workspace, int BH, int Nq, int Nk, float c,
                       hipStream_t stream) {
  if (d == 64)
    return causal ? launch_typed<T, 64, true>(q, k, v, o, lse, workspace, BH, Nq, Nk, c, stream)
                  : launch_typed<T, 64, false>(q, k, v, o, lse, workspace, BH, Nq, Nk, c, stream);
  return causal ? launch_typed<T, 128, true>(q, k, v, o, lse, workspace, BH, Nq, Nk, c, stream)
                : launch_typed<T, 128, false>(q, k, v, o, lse, workspace, BH, Nq, Nk, c, stream);
}

}  // namespace

// Chunks per head: 32 tiles (1024 keys) each, or fewer tiles (down to 4) when
// that leaves the grid with fewer than about 2048 waves.
void decode_split_plan(int BH, int Nq, int Nk, int* n_chunks, int* chunk_tiles) {
  const int64_t tiles = ((int64_t)Nk + kTileKeys - 1) / kTileKeys;
  const int64_t groups = (int64_t)BH * ((Nq + 31) / 32);
  int64_t ct = 32;
  while (ct > 4 && groups * ((tiles + ct - 1) / ct) < 2048) ct >>= 1;
  *chunk_tiles = (int)ct;
  *n_chunks = (int)((tiles + ct - 1) / ct);
}

hipError_t launch_attn_decode(Elem elem, const void* q, const void* k, const void* v, void* o,
                              float* lse, float* workspace, int B, int H, int Nq, int Nk, int d,
                              float scale, bool causal, hipStream_t stream) {
  const float c = scale * kLog2e;
  const int BH = B * H;
  if (elem == Elem::bf16)
    return launch_elem<__bf16>(d, causal, q, k, v, o, lse, workspace, BH, Nq, Nk, c, stream);
  return launch_elem<_Float16>(d, causal, q, k, v, o, lse, workspace, BH, Nq, Nk, c, stream);
}

hipError_t attn_decode_attributes(int d, bool causal, hipFuncAttributes* attr, int* threads,
                                  int* blocks_per_cu) {
  const void* fn = d == 64 ? (causal ? (const void*)attn_decode_partial<__bf16, 64, true>
                                     : (const void*)attn_decode_partial<__bf16, 64, false>)
                           : (causal ? (const void*)attn_decode_partial<__bf16, 128, true>
                                     : (const void*)attn_decode_partial<__bf16, 128, false>);
  *threads = 64;
  hipError_t e = hipFuncGetAttributes(attr, fn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, 64, 0);
}

}  // namespace osm
