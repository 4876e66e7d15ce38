// Attention forward for gfx950: O = softmax(scale * Q K^T) V with the online-softmax
// recurrence, bf16 / fp16 operands on the 32x32x16 MFMA, fp32 accumulation.
//
// Method.  Query blocks are the outer loop and key/value tiles the inner loop
// ("Online Softmax: Tiling Across a Reduction", loop-order paragraphs).  Each
// query row carries (m, l, O); per key tile, following the update equations of
// "Online softmax, and the register that can't move" (section "Online
// softmax"):
//     m_new = max(m_old, rowmax S)
//     l     = l * exp(m_old - m_new) + rowsum exp(S - m_new)
//     O     = O * exp(m_old - m_new) + exp(S - m_new) V
// and O / l once after the last tile.  m starts at -inf, so the first rescale
// factor is exactly 0 ("Day 97", Solution).  Exponentials run in base 2 with
// c = scale * log2(e) folded into one FMA per score, so m is kept in units of
// c * score; the logsumexp written out is ln 2 * (m + log2 l).
//
// Work decomposition.  A workgroup of 4 waves owns 128 consecutive queries of
// one (batch, head); each wave owns 32 of them.  Key tiles are 64 keys.
//
// Orientation.  The score tile is computed transposed, S^T = K Q^T, with K from
// LDS as the A operand and the wave's Q^T held in VGPRs for the whole loop as
// the B operand.  In the 32x32 MFMA accumulator layout, lane l holds column
// l % 32 -- one query -- and 16 of the 32 rows (keys); lane l ^ 32 holds the
// other 16.  So a query's row maximum is an in-lane max over 32 values plus
// one v_permlane32_swap exchange, the rescale factor is per lane, and the
// output accumulator O^T = V^T P^T (rows = head dims, columns = queries) also
// has one query per lane: O *= alpha is a plain per-lane multiply of VGPRs.
// The accumulator never leaves registers during the loop.
//
// P repack.  P^T is the B operand of the second MFMA straight from the score
// registers (fp32 -> bf16/fp16, round to nearest even).  The keys a lane holds
// in the accumulator layout are not the keys the B layout assigns to it; the
// mismatch is absorbed by storing V^T in LDS with the same key permutation
// (within each 16-key group, bits 2 and 3 of the key index are swapped), since
// the sum over keys does not depend on their order.
//
// Loader.  K and V tiles are double-buffered in LDS: while tile t is consumed,
// tile t+1 is fetched into registers and written to the other buffers after
// the MFMAs of tile t; one barrier per tile.
//
// Loader.  Global traffic uses buffer loads whose base is advanced by whole
// tiles on the scalar unit, so each load needs no vector address arithmetic,
// and rows past N fall outside the buffer's range and read as zero (their
// scores are masked).  K rows are padded by 16 bytes in LDS; V is transposed
// in registers (4 keys x D/16 dims per thread) and stored as V^T rows padded
// by 16 bytes, 16 lanes per row so the stores do not collide in LDS banks.
//
// Causal.  Key tiles wholly after the query block are never visited, tiles
// wholly before it run without a mask, and only tiles straddling the diagonal
// (or the ragged end of the sequence) mask element by element ("Online Softmax:
// Tiling Across a Reduction", causal paragraphs).  A wave stops computing at
// the last tile holding a key visible to one of its queries.  Query blocks are
// handed out longest first.
#include "common.h"
#include "kernels.h"

namespace osm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format,
// no swizzle): out-of-range loads return zero and out-of-range stores are dropped.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kBufferWord3);
}

template <typename T>
struct Mma;
template <>
struct Mma<__bf16> {
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mma<_Float16> {
  using v8 = f16x8;
  static __device__ __forceinline__ f32x16 run(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  return (unsigned)__builtin_bit_cast(unsigned short, (T)a) |
         ((unsigned)__builtin_bit_cast(unsigned short, (T)b) << 16);
}

constexpr int kBM = 128;  // queries per workgroup
constexpr int kBN = 64;   // keys per tile
constexpr int kThreads = 256;

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int BH,
    int N, int n_mtiles, float c, int xcd_groups) {
  using v8 = typename Mma<T>::v8;
  constexpr int KS = D + 8;            // K tile row stride in LDS (elements)
  constexpr int VS = kBN + 8;          // V^T tile row stride in LDS (elements)
  constexpr int K_ELEMS = kBN * KS;
  constexpr int V_ELEMS = D * VS;
  constexpr int ND = D / 32;           // 32-dim blocks of O^T per wave
  constexpr int NK = D / 16;           // 16-deep MFMA steps of K Q^T
  constexpr int CPR = D / 8;           // 16-byte chunks per K row
  constexpr int KCH = kBN * CPR / kThreads;  // K rows per thread
  constexpr int VD = D / 16;           // head dims per thread in the V transpose
  constexpr int ROW_BYTES = D * 2;
  static_assert(KCH >= 1 && VD % 2 == 0 && 4 * ROW_BYTES < 4096, "tile shape");
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2 * K_ELEMS];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2 * V_ELEMS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // ---- which (batch*head, query block) this workgroup owns ---------------------
  int id = blockIdx.x, bh, mt;
  if (xcd_groups) {
    // consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD a
    // contiguous run of heads so the blocks sharing a head's K/V share its L2
    const int per = gridDim.x >> 3;
    id = (id & 7) * per + (id >> 3);
    bh = id / n_mtiles;
    mt = n_mtiles - 1 - (id - bh * n_mtiles);
  } else {
    bh = id % BH;
    mt = n_mtiles - 1 - id / BH;
  }
  const int i0 = mt * kBM;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint16_t* Kh = K + base;
  const uint16_t* Vh = V + base;
  const int qw0 = i0 + wave * 32;  // first query of this wave
  const int qi = qw0 + l32;        // this lane's query

  // ---- Q^T fragments: B operand, lane = query, 8 consecutive head dims -------------
  v8 qf[NK];
  {
    const auto rq = make_rsrc(Q + base + (size_t)qw0 * D, (int64_t)(N - qw0) * ROW_BYTES);
    const int off = l32 * ROW_BYTES + 16 * hf;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
      qf[kb] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 32 * kb, 0, 0));
  }

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;

  const int nk_all = (N + kBN - 1) / kBN;
  const int n_kt = CAUSAL ? min(nk_all, (i0 + kBM - 1) / kBN + 1) : nk_all;
  // tiles holding a key visible to some query of this wave
  const int n_kt_w = CAUSAL ? min(n_kt, (qw0 + 31) / kBN + 1) : n_kt;

  // ---- loader: registers <- global (tile t), LDS buffer <- registers ----------------
  const int krow = (tid / CPR) * KCH;  // K rows krow .. krow+KCH-1 of the tile
  const int kcol = (tid % CPR) * 8;
  const int kgoff = krow * ROW_BYTES + kcol * 2;
  // V: keys 4*va .. 4*va+3 of the tile, head dims vb*VD .. vb*VD+VD-1.  The key
  // group is the fast index so that 16 consecutive lanes store their 8-byte
  // V^T pieces into 128 contiguous (permuted) bytes of one V^T row: distinct
  // banks.  (With the head-dim group fast, the lanes' rows sit 8 rows apart,
  // a multiple of 128 bytes, and all 16 hit the same banks.)
  const int va = tid & 15, vb = tid >> 4;
  const int vgoff = 4 * va * ROW_BYTES + vb * VD * 2;
  const int vpos = 4 * ((va & ~3) | ((va & 1) << 1) | ((va >> 1) & 1));  // permuted key slot
  u32x4 kreg[KCH];
  unsigned vreg[4][VD / 2];

  auto load_k = [&](int t) {
    const auto r = make_rsrc(Kh + (size_t)t * kBN * D, (int64_t)(N - t * kBN) * ROW_BYTES);
#pragma unroll
    for (int i = 0; i < KCH; ++i)
      kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(r, kgoff + i * ROW_BYTES, 0, 0);
  };
  auto store_k = [&](int b) {
    uint16_t* Ks = kbuf + b * K_ELEMS;
#pragma unroll
    for (int i = 0; i < KCH; ++i) *reinterpret_cast<u32x4*>(Ks + (krow + i) * KS + kcol) = kreg[i];
  };
  auto load_v = [&](int t) {
    const auto r = make_rsrc(Vh + (size_t)t * kBN * D, (int64_t)(N - t * kBN) * ROW_BYTES);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      if constexpr (VD == 8) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, vgoff + rr * ROW_BYTES, 0, 0);
        vreg[rr][0] = x[0]; vreg[rr][1] = x[1]; vreg[rr][2] = x[2]; vreg[rr][3] = x[3];
      } else {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, vgoff + rr * ROW_BYTES, 0, 0);
        vreg[rr][0] = x[0]; vreg[rr][1] = x[1];
      }
    }
  };
  auto store_v = [&](int b) {
    uint16_t* Vt = vbuf + b * V_ELEMS;
#pragma unroll
    for (int cc = 0; cc < VD; ++cc) {
      const int w = cc >> 1;
      unsigned k01, k23;  // keys (4va, 4va+1) and (4va+2, 4va+3) of head dim vb*VD+cc
      if ((cc & 1) == 0) {
        k01 = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
        k23 = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
      } else {
        k01 = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
        k23 = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
      }
      *reinterpret_cast<u32x2*>(Vt + (vb * VD + cc) * VS + vpos) = u32x2{k01, k23};
    }
  };
  // S^T = K Q^T for the tile in K buffer b: two 32-key halves
  auto qk = [&](int b, f32x16 (&s)[2]) {
    const uint16_t* Ks = kbuf + b * K_ELEMS;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const v8 kf = __builtin_bit_cast(
            v8, *reinterpret_cast<const u32x4*>(Ks + (kh * 32 + l32) * KS + kb * 16 + 8 * hf));
        s[kh] = Mma<T>::run(kf, qf[kb], s[kh]);
      }
    }
  };

  // One tile: S = K Q^T, then m, l and O updated with P = 2^(c S - m_new).
  auto step = [&](int t) {
    const int j0 = t * kBN;
    f32x16 s[2];
    qk(t & 1, s);
    // keys past N, and keys after the query when causal (wave-uniform test)
    if ((j0 + kBN > N) || (CAUSAL && j0 + kBN - 1 > qw0)) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * kh + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key >= N || (CAUSAL && key > qi)) s[kh][r] = kNegInf;
        }
      }
    }
    // ---- online softmax: m, l, O rescaled by 2^(m_old - m_new) ---------------------
    float mx = kNegInf;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
    mx = max_halves(mx);
    const float m_new = fmaxf(m_run, mx * c);
    const float m_sub = (m_new == kNegInf) ? 0.f : m_new;  // a fully masked row stays empty
    const float alpha = exp2_fast(m_run - m_sub);
    float ls = 0.f;
    v8 pf[2][2];  // P^T as 16-bit B operands: [32-key half][16-key step]
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2_fast(fmaf(s[kh][r], c, -m_sub));
        ls += p;
        pf[kh][r >> 3][r & 7] = (T)p;
      }
    }
    l_run = fmaf(l_run, alpha, ls);
    m_run = m_new;
    if (__any(alpha != 1.f)) {  // wave-uniform; skipped while no row's max moves
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
    }
    // ---- O^T += V^T P^T ---------------------------------------------------------------
    const uint16_t* Vt = vbuf + (t & 1) * V_ELEMS;
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {  // ND independent accumulators in flight
          const v8 vf = __builtin_bit_cast(
              v8, *reinterpret_cast<const u32x4*>(Vt + (db * 32 + l32) * VS + 32 * kh + 16 * kb +
                                                  8 * hf));
          o[db] = Mma<T>::run(vf, pf[kh][kb], o[db]);
        }
      }
    }
  };

  // ---- prologue: tile 0 into LDS --------------------------------------------------------
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  __syncthreads();
  // Retire the Q loads here.  Left pending, they would make the first MFMA that
  // reads Q inside the loop wait on the vector-memory counter, which by then
  // also counts the next tile's prefetch.
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) asm volatile("" ::"v"(qf[kb]));

  for (int t = 0; t < n_kt; ++t) {
    if (t + 1 < n_kt) {  // prefetch tile t+1 into registers while tile t computes
      load_k(t + 1);
      load_v(t + 1);
    }
    if (t < n_kt_w) step(t);
    if (t + 1 < n_kt) {  // the other buffers were last read in iteration t-1
      store_k((t + 1) & 1);
      store_v((t + 1) & 1);
    }
    __syncthreads();
  }

  // ---- epilogue: O / l, logsumexp --------------------------------------------------
  const float l_tot = sum_halves(l_run);
  const float inv = 1.f / l_tot;
  {
    // rows past N fall outside the buffer and are dropped
    const auto ro = make_rsrc(O + base + (size_t)qw0 * D, (int64_t)(N - qw0) * ROW_BYTES);
    const int off = l32 * ROW_BYTES + 8 * hf;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const u32x2 w = u32x2{pack2<T>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                              pack2<T>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, off + (db * 32 + 8 * g) * 2, 0, 0);
      }
    }
  }
  if (LSE != nullptr && hf == 0 && qi < N)
    LSE[(size_t)bh * N + qi] = (m_run + log2f(l_tot)) * kLn2;
}

// ------------------------------------------------------------------------------------
// fp32 operands: one query per lane (two lanes per query at d = 128), fp32 FMA dot
// products on the vector ALU, the same recurrence, 32-key tiles in LDS.
// ------------------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_fwd_f32(const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     float* __restrict__ O,
                                                     float* __restrict__ LSE, int BH, int N,
                                                     int n_mtiles, float c) {
  constexpr int LPQ = D / 64;         // lanes per query
  constexpr int DL = D / LPQ;         // head dims per lane
  constexpr int QPW = 64 / LPQ;       // queries per wave
  constexpr int BMF = 4 * QPW;        // queries per workgroup
  constexpr int BNF = 32;             // keys per tile
  __shared__ __attribute__((aligned(16))) float Ks[BNF * D];
  __shared__ __attribute__((aligned(16))) float Vs[BNF * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x % BH;
  const int mt = n_mtiles - 1 - blockIdx.x / BH;
  const int i0 = mt * BMF;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int qw0 = i0 + wave * QPW;
  const int qi = qw0 + lane % QPW;
  const int part = lane / QPW;

  float q[DL], o[DL];
  {
    const float* qp = Q + base + (size_t)min(qi, N - 1) * D + part * DL;
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      q[e] = qp[e];
      o[e] = 0.f;
    }
  }
  float m_run = kNegInf, l_run = 0.f;
  const int nk_all = (N + BNF - 1) / BNF;
  const int n_kt = CAUSAL ? min(nk_all, (i0 + BMF - 1) / BNF + 1) : nk_all;

  for (int t = 0; t < n_kt; ++t) {
    const int j0 = t * BNF;
    __syncthreads();  // previous tile fully consumed
    for (int idx = tid; idx < BNF * D / 4; idx += 256) {
      const int row = idx / (D / 4), col = (idx % (D / 4)) * 4;
      const size_t g = (size_t)min(j0 + row, N - 1) * D + col;
      *reinterpret_cast<float4*>(&Ks[row * D + col]) = *reinterpret_cast<const float4*>(K + base + g);
      *reinterpret_cast<float4*>(&Vs[row * D + col]) = *reinterpret_cast<const float4*>(V + base + g);
    }
    __syncthreads();
    if (CAUSAL && j0 > qw0 + QPW - 1) continue;  // wave-uniform: whole tile hidden
    float s[BNF];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) acc = fmaf(q[e], Ks[j * D + part * DL + e], acc);
      if constexpr (LPQ == 2) acc += __shfl_xor(acc, 32);
      const int key = j0 + j;
      if (key >= N || (CAUSAL && key > qi)) acc = kNegInf;
      s[j] = acc;
      mx = fmaxf(mx, acc);
    }
    const float m_new = fmaxf(m_run, mx * c);
    const float m_sub = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = exp2_fast(m_run - m_sub);
    float ls = 0.f;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      s[j] = exp2_fast(fmaf(s[j], c, -m_sub));
      ls += s[j];
    }
    l_run = fmaf(l_run, alpha, ls);
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < DL; ++e) {
      float acc = o[e] * alpha;
#pragma unroll
      for (int j = 0; j < BNF; ++j) acc = fmaf(s[j], Vs[j * D + part * DL + e], acc);
      o[e] = acc;
    }
  }
  if (qi < N) {
    const float inv = 1.f / l_run;
    float* op = O + base + (size_t)qi * D + part * DL;
#pragma unroll
    for (int e = 0; e < DL; ++e) op[e] = o[e] * inv;
    if (LSE != nullptr && part == 0) LSE[(size_t)bh * N + qi] = (m_run + log2f(l_run)) * kLn2;
  }
}

template <typename T, int D, bool C>
const void* mfma_fn() {
  return (const void*)attn_fwd_mfma<T, D, C>;
}

const void* pick_attn(Elem elem, int d, bool causal, int* threads, int* rows_per_block) {
  *threads = 256;
  if (elem == Elem::f32) {
    *rows_per_block = 4 * (64 / (d / 64));
    if (d == 64) return causal ? (const void*)attn_fwd_f32<64, true> : (const void*)attn_fwd_f32<64, false>;
    return causal ? (const void*)attn_fwd_f32<128, true> : (const void*)attn_fwd_f32<128, false>;
  }
  *rows_per_block = kBM;
  if (elem == Elem::bf16) {
    if (d == 64) return causal ? mfma_fn<__bf16, 64, true>() : mfma_fn<__bf16, 64, false>();
    return causal ? mfma_fn<__bf16, 128, true>() : mfma_fn<__bf16, 128, false>();
  }
  if (d == 64) return causal ? mfma_fn<_Float16, 64, true>() : mfma_fn<_Float16, 64, false>();
  return causal ? mfma_fn<_Float16, 128, true>() : mfma_fn<_Float16, 128, false>();
}

}  // namespace

hipError_t launch_attn_fwd(Elem elem, const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
  int threads, rows_per_block;
  const void* fn = pick_attn(elem, d, causal, &threads, &rows_per_block);
  int BH = B * H;
  int n_mtiles = (N + rows_per_block - 1) / rows_per_block;
  float c = scale * kLog2e;
  const int grid = BH * n_mtiles;
  if (elem == Elem::f32) {
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse,
                    (void*)&BH, (void*)&N, (void*)&n_mtiles, (void*)&c};
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
  }
  int xcd_groups = (BH % 8 == 0) ? 1 : 0;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&BH,
                  (void*)&N, (void*)&n_mtiles, (void*)&c, (void*)&xcd_groups};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
}

hipError_t attn_fwd_attributes(Elem elem, int d, bool causal, hipFuncAttributes* attr,
                               int* threads, int* blocks_per_cu) {
  int rows_per_block;
  const void* fn = pick_attn(elem, d, causal, threads, &rows_per_block);
  hipError_t e = hipFuncGetAttributes(attr, fn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, *threads, 0);
}

}  // namespace osm
