// Attention forward with fp8 operands on gfx950: Q, K and V stored as OCP fp8
// E4M3 codes with one descale per tensor (value = descale * code), both products
// on the 32x32x64 fp8 MFMA (twice the bf16 rate), fp32 accumulation, O in bf16.
//
// Method.  The online-softmax recurrence of "Online softmax, and the register
// that can't move" (section "Online softmax"), tile by tile, O / l once at the
// end, as in the bf16 kernel: per key tile, m_new = max(m_old, rowmax S), l and
// O rescaled by 2^(m_old - m_new), P = 2^(c S - m_new).  The descales of Q and
// K fold into c = scale * q_descale * k_descale * log2(e); the descale of V
// multiplies O once in the epilogue.  fp8 as the next precision step after
// 16 bits is the one the "100 Days of GPU, Day 97" page names for its
// follow-up.
//
// P in fp8.  P is the B operand of the second product, so it is rounded to
// E4M3 (3 mantissa bits, largest value 448).  It is stored as 2^7 P, and the
// reference maximum m trails the row maximum by at most 1.5 (log2 units), so a
// stored weight is at most 2^8.5 = 362: O and l are rescaled only on the tiles
// where some row's maximum passes m by more than that.  E4M3 is normal from
// 2^-6, so weights down to 2^-13 keep 3 mantissa bits and smaller ones fall
// into subnormal steps of 2^-9 (2^-16 in units of P).  2^7 is exact and costs
// nothing (2^(c S - m + 7)).  As in the 16-bit kernels, l sums the rounded
// values that multiply V, so O / l is a convex combination of the V rows with
// the rounded weights; that sum runs on the matrix unit as one more MFMA per
// tile, with an all-ones row in place of V^T (the softmax, not the matrix
// unit, bounds this kernel).
//
// Layout.  The same decomposition and slot schedule as the bf16 kernel: 8 waves
// own 256 queries of one (batch, head) in two groups that run half a tile apart
// (one issues MFMAs while the other runs the softmax), 64-key tiles, one
// barrier per tile, direct buffer loads into LDS with one array per stage
// (StageTag).  Rows are 128 bytes (d = 128 fp8).  Unlike the bf16 kernel, only
// group 0 issues the tile loads, in slot Y where it runs the products: the fp8
// products take about a third of the softmax's time, so that wave has room for
// the load instructions, whose issue would otherwise lengthen the softmax wave
// that bounds the slot.
//  * S^T = K Q^T: A = K rows from LDS (lane = key, 32 bytes of head dims per
//    lane half), B = Q^T in VGPRs (lane = query).  Two MFMAs per 32 keys.
//  * O^T += V^T P^T: A = V^T through ds_read_b64_tr_b8 (in each 16-lane group
//    lane q receives column q of the 8 rows the group addresses), B = P^T.  The
//    32 keys a lane's P holds after the score MFMAs come in runs of 4 (keys
//    8g + 4 h + 0..3 of each 32-key block, h the lane half); one
//    v_permlane32_swap per pair of runs turns them into runs of 8 consecutive
//    keys (16 i + 8 h + 0..7, i = 0..3), which is what four transposed reads of
//    8 rows deliver.  One MFMA per 32 head dims covers the 64 keys of a tile.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace osm {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// 32x32x64 MFMA with E4M3 A and B (format codes 0, no block scales)
__device__ __forceinline__ f32x16 mma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Wait states after a chain of fp8 MFMAs, before anything may read their results.
// The compiler's own wait after the 32x32x64 fp8 MFMA is short on this part: a
// register copy it placed 17 wait states after the last MFMA of a chain read the
// last two result registers before the MFMA had written them.  The scheduling
// barriers keep every reader of the results below the padding.
__device__ __forceinline__ void mfma_settle() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 15\n s_nop 15" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

constexpr int kBM = 256;        // queries per workgroup
constexpr int kBN = 64;         // keys per tile
constexpr int kThreads = 512;   // two groups of 4 waves
constexpr float kPScale = 7.f;  // P is stored as 2^7 P
constexpr float kSlack = 1.5f;  // how far (log2 units) the row maximum may pass m: 2^(7 + 1.5) < 448

// 16-byte chunk swizzles of D-byte rows (physical chunk = logical ^ swizzle):
// K is read as 16-byte pieces of 32 consecutive rows at one chunk position,
// V^T as 8 rows x 32 bytes per 32 lanes; both spread over all 64 banks.  With
// 128-byte rows, rows 2 apart share a bank line; with 64-byte rows, rows 4 apart.
// Rows 32 (K) and 16 (V) apart keep their swizzle, as the operand reads assume.
template <int D>
__device__ __forceinline__ int kswz8(int row) { return D == 128 ? (row >> 1) & 7 : (row >> 2) & 3; }
template <int D>
__device__ __forceinline__ int vswz8(int row) {
  return D == 128 ? 2 * ((row >> 1) & 3) : 2 * ((row >> 2) & 1);
}

// The kernel body for head dim kD (64 or 128); the kernels below instantiate it.
template <int kD, bool CAUSAL>
__device__ __forceinline__ void fp8_forward(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int N, int n_mtiles, float c,
    float v_descale, int xcd_groups) {
  constexpr int ROW_BYTES = kD;
  constexpr int TILE_BYTES = kBN * ROW_BYTES;  // 8 KiB
  constexpr int ND = kD / 32;                  // 32-dim blocks of O^T
  constexpr int NK = kD / 64;                  // 64-deep MFMA steps of K Q^T
  constexpr int NH = kBN / 32;                 // 32-key blocks of a tile
  constexpr int CPR = ROW_BYTES / 16;          // 16-byte chunks per row
  constexpr int RPI = 1024 / ROW_BYTES;        // rows per 1 KiB wave-wide load
  constexpr int NI = TILE_BYTES / 1024 / 4;    // such loads per group-0 wave per tile
  static_assert(NI >= 1 && NH == 2, "tile shape");
  __shared__ __attribute__((aligned(1024))) unsigned char kb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char kb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char vb1[TILE_BYTES];
  auto kbuf = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return kb0; else return kb1;
  };
  auto vbuf = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return vb0; else return vb1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int group = wave >> 2;

  // ---- which (batch*head, query blocks) this workgroup owns (as the bf16 kernel:
  // causal workgroups take blocks mt and n_mtiles - 1 - mt, which together hold
  // as many key tiles as any other pair)
  int id = blockIdx.x, bh, mt_a, mt_b = 0;
  const int n_units = CAUSAL ? (n_mtiles + 1) >> 1 : n_mtiles;
  if (xcd_groups) {
    const int per = gridDim.x >> 3;
    id = (id & 7) * per + (id >> 3);
    bh = id / n_units;
    mt_a = n_units - 1 - (id - bh * n_units);
  } else {
    bh = id % BH;
    mt_a = n_units - 1 - id / BH;
  }
  if (CAUSAL) {
    mt_b = mt_a;
    mt_a = n_mtiles - 1 - mt_b;
  }

  // Q^T fragments of query block mt: lane = query, 32 consecutive head dims per
  // 64-deep step
  auto load_q = [&](const int mt, i32x8 (&qf)[NK]) __attribute__((always_inline)) {
    const int qw0_s = __builtin_amdgcn_readfirstlane(mt * kBM + 32 * (2 * (wave & 3) + group));
    const auto rq = make_rsrc(Q + (size_t)bh * (size_t)N * kD + (size_t)qw0_s * kD,
                              (int64_t)(N - qw0_s) * ROW_BYTES);
    const int off = l32 * ROW_BYTES + 32 * hf;
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 64 * kb, 0, 0);
      const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 64 * kb + 16, 0, 0);
      qf[kb] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
    }
  };

  // one query block; inlined once per block of the pair.  after_loop runs once
  // the block's last Q^T read is done.
  auto block = [&](const int mt, i32x8 (&qf)[NK], auto&& after_loop) __attribute__((always_inline)) {
    const int i0 = mt * kBM;
    const size_t base = (size_t)bh * (size_t)N * kD;  // bytes = elements
    const uint8_t* Kh = K + base;
    const uint8_t* Vh = V + base;
    const int qw0 = i0 + 32 * (2 * (wave & 3) + group);
    const int qi = qw0 + l32;
    const int qw0_s = __builtin_amdgcn_readfirstlane(qw0);


    f32x16 o[ND];
  #pragma unroll
    for (int db = 0; db < ND; ++db) o[db] = f32x16{};
    f32x16 s[NH];
    // row sums of the rounded P on the matrix unit: a V^T block whose row 0 is all
    // ones, so element 0 of the lane-half-0 accumulator is l for the lane's query
    // (the other 31 rows are zero and stay zero)
    f32x16 lacc = f32x16{};
    const int one8 = l32 == 0 ? 0x38383838 : 0;  // E4M3 1.0 in every byte of row 0
    const i32x8 ones = {one8, one8, one8, one8, one8, one8, one8, one8};
    i32x8 pf;  // P^T (2^7 P in E4M3) as the B operand: bytes 8 i .. 8 i + 7 = keys 16 i + 8 hf + 0..7
    float m_run = kNegInf;

    const int nk_all = (N + kBN - 1) / kBN;
    const int n_kt = CAUSAL ? min(nk_all, (i0 + kBM - 1) / kBN + 1) : nk_all;
    int n_w = CAUSAL ? min(n_kt, (qw0 + 31) / kBN + 1) : n_kt;
    asm volatile("" : "+v"(n_w));
    auto act = [&](int t) { return t < n_w; };

    // ---- loader: global -> LDS directly, by the four group-0 waves (2 KiB each per tile)
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    int kgoff[NI], vgoff[NI];
  #pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = ((wave & 3) * NI + j) * RPI + lane / CPR;
      const int p = lane % CPR;
      kgoff[j] = row * ROW_BYTES + (p ^ kswz8<kD>(row)) * 16;
      vgoff[j] = row * ROW_BYTES + (p ^ vswz8<kD>(row)) * 16;
    }
    auto load_k = [&](int t, auto st) __attribute__((always_inline)) {
      const auto r = make_rsrc(Kh + (size_t)t * kBN * kD, (int64_t)(N - t * kBN) * ROW_BYTES);
  #pragma unroll
      for (int j = 0; j < NI; ++j) load16_to_lds(r, kbuf(st) + ((wave_s & 3) * NI + j) * 1024, kgoff[j]);
    };
    auto load_v = [&](int t, auto st) __attribute__((always_inline)) {
      const auto r = make_rsrc(Vh + (size_t)t * kBN * kD, (int64_t)(N - t * kBN) * ROW_BYTES);
  #pragma unroll
      for (int j = 0; j < NI; ++j) load16_to_lds(r, vbuf(st) + ((wave_s & 3) * NI + j) * 1024, vgoff[j]);
    };
    auto loads_landed = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    // ---- operand read offsets
    // K: row l32 (+32 per key block), logical chunks 4 kb + 2 hf and 4 kb + 2 hf + 1
    int kroff[NK][2];
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb)
  #pragma unroll
      for (int h = 0; h < 2; ++h)
        kroff[kb][h] = l32 * ROW_BYTES + ((4 * kb + 2 * hf + h) ^ kswz8<kD>(l32)) * 16;
    // V^T: read i of head-dim block db takes rows 16 i + 8 hf + (q >> 1), bytes
    // 32 db + 16 ((lane >> 4) & 1) + 8 (q & 1) (q = lane % 16); rows 16 i apart share
    // the swizzle, so one offset per db serves all four reads
    int vroff[ND];
    {
      const int q = lane & 15;
      const int row = 8 * hf + (q >> 1);
  #pragma unroll
      for (int db = 0; db < ND; ++db)
        vroff[db] = row * ROW_BYTES + ((2 * db + ((lane >> 4) & 1)) ^ vswz8<kD>(row)) * 16 + 8 * (q & 1);
    }

    auto qk = [&](auto st) __attribute__((always_inline)) {
      const unsigned char* Kt = kbuf(st);
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh) s[kh] = f32x16{};
  #pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
  #pragma unroll
        for (int kh = 0; kh < NH; ++kh) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(Kt + kroff[kb][0] + kh * 32 * ROW_BYTES);
          const u32x4 b = *reinterpret_cast<const u32x4*>(Kt + kroff[kb][1] + kh * 32 * ROW_BYTES);
          const i32x8 kf = {(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                            (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
          s[kh] = mma_fp8(kf, qf[kb], s[kh]);
        }
      }
      mfma_settle();
    };
    auto sm = [&](int t) __attribute__((always_inline)) {
      const int j0 = t * kBN;
      if ((j0 + kBN > N) || (CAUSAL && j0 + kBN - 1 > qw0)) {
  #pragma unroll
        for (int kh = 0; kh < NH; ++kh) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * kh + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= N || (CAUSAL && key > qi)) s[kh][r] = kNegInf;
          }
        }
      }
      float mx = kNegInf;
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh)
  #pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kh][r]);
      mx = max_halves(mx);
      const float m_cand = fmaxf(m_run, mx * c);
      const float m_new = (m_cand > m_run + kSlack) ? m_cand : m_run;  // -inf moves to any finite max
      const float m_sub = (m_new == kNegInf) ? 0.f : m_new;  // a fully masked row stays empty
      const float alpha = exp2_fast(m_run - m_sub);
      const float shift = kPScale - m_sub;
      // 2^7 P rounded to E4M3: word g of block kh holds keys 32 kh + 8 g + 4 hf + 0..3
      unsigned w[NH][4];
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float p0 = exp2_fast(fmaf(s[kh][4 * g], c, shift));
          const float p1 = exp2_fast(fmaf(s[kh][4 * g + 1], c, shift));
          const float p2 = exp2_fast(fmaf(s[kh][4 * g + 2], c, shift));
          const float p3 = exp2_fast(fmaf(s[kh][4 * g + 3], c, shift));
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, x, true);
          w[kh][g] = (unsigned)x;
        }
      }
      m_run = m_new;
      // runs of 4 keys -> runs of 8: swap word 2j + 1 of the low half with word 2j
      // of the high half
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh) {
  #pragma unroll
        for (int j = 0; j < 2; ++j) {
          const auto r = __builtin_amdgcn_permlane32_swap(w[kh][2 * j], w[kh][2 * j + 1], false, false);
          pf[4 * kh + 2 * j] = (int)r[0];
          pf[4 * kh + 2 * j + 1] = (int)r[1];
        }
      }
      if (__any(alpha != 1.f)) {
  #pragma unroll
        for (int db = 0; db < ND; ++db) o[db] *= alpha;
        lacc[0] *= alpha;
      }
    };
    auto pv_chain = [&](auto st) __attribute__((always_inline)) {
      const unsigned char* Vt = vbuf(st);
  #pragma unroll
      for (int db = 0; db < ND; ++db) {
        i32x2 r[4];
  #pragma unroll
        for (int i = 0; i < 4; ++i)
          r[i] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(Vt + vroff[db] + 16 * i * ROW_BYTES));
        const i32x8 vf = {r[0][0], r[0][1], r[1][0], r[1][1], r[2][0], r[2][1], r[3][0], r[3][1]};
        o[db] = mma_fp8(vf, pf, o[db]);
      }
      lacc = mma_fp8(ones, pf, lacc);  // l += sum of the rounded P
    };
    auto pv = [&](auto st) __attribute__((always_inline)) {
      pv_chain(st);
      mfma_settle();
    };
    auto pv_qk = [&](auto stp, auto stq) __attribute__((always_inline)) {
      pv_chain(stp);
      qk(stq);
      constexpr int kAhead = 2;  // MFMAs whose operands are read ahead
      constexpr int kPv = ND + 1, kQk = NH * NK;
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * kAhead, 0);  // DS reads
  #pragma unroll
      for (int i = 0; i < kPv + kQk; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        const int j = i + kAhead;
        if (j < kPv - 1) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
        else if (j < kPv + kQk) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
    };

    // One tile t in stage S = t & 1: slot X(t), the barrier, slot Y(t) (the bf16
    // kernel's schedule: group 0 runs SM(t) then PV(t), QK(t+1); group 1 runs
    // PV(t-1), QK(t) then SM(t)).
    auto tile = [&](int t, auto st) __attribute__((always_inline)) {
      constexpr int S = decltype(st)::value;
      const StageTag<S> cur;
      const StageTag<S ^ 1> other;
      if (group == 0) {
        if (act(t)) sm(t);
      } else {
        __builtin_amdgcn_s_setprio(1);
        if (t > 0 && act(t - 1) && act(t)) {
          pv_qk(other, cur);
        } else {
          if (t > 0 && act(t - 1)) pv(other);
          if (act(t)) qk(cur);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      loads_landed();
      __syncthreads();
      if (group == 0) {
        if (t + 2 < n_kt) load_k(t + 2, cur);
        if (t + 1 < n_kt) load_v(t + 1, other);
        __builtin_amdgcn_s_setprio(1);
        if (act(t) && act(t + 1)) {
          pv_qk(cur, other);
        } else {
          if (act(t)) pv(cur);
          if (act(t + 1)) qk(other);
        }
        __builtin_amdgcn_s_setprio(0);
      } else {
        if (act(t)) sm(t);
      }
    };

    if (group == 0) load_k(0, StageTag<0>{});
    loads_landed();
    __syncthreads();
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb) asm volatile("" ::"v"(qf[kb]));
    if (group == 0) {
      if (1 < n_kt) load_k(1, StageTag<1>{});
      load_v(0, StageTag<0>{});
    }
    if (group == 0 && act(0)) {
      __builtin_amdgcn_s_setprio(1);
      qk(StageTag<0>{});
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    for (int t = 0; t < n_kt; t += 2) {
      tile(t, StageTag<0>{});
      if (t + 1 < n_kt) tile(t + 1, StageTag<1>{});
    }
    after_loop();
    if (group == 1 && act(n_kt - 1)) {
      if (((n_kt - 1) & 1) == 0) pv(StageTag<0>{}); else pv(StageTag<1>{});
    }

    // ---- epilogue: O = v_descale * O / l in bf16, logsumexp = ln 2 (m + log2(l / 2^7))
    const float l_tot = sum_halves(lacc[0]);  // the high half's element 0 is row 4: zero
    const float inv = v_descale / l_tot;
    {
      const auto ro = make_rsrc(O + (size_t)bh * N * kD + (size_t)qw0_s * kD, (int64_t)(N - qw0_s) * kD * 2);
      const int off = l32 * kD * 2 + 8 * hf;
  #pragma unroll
      for (int db = 0; db < ND; ++db) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 wv = u32x2{pack2<__bf16>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                 pack2<__bf16>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
          __builtin_amdgcn_raw_buffer_store_b64(wv, ro, off + (db * 32 + 8 * g) * 2, 0, 0);
        }
      }
    }
    if (LSE != nullptr && hf == 0 && qi < N)
      LSE[(size_t)bh * N + qi] = (m_run + log2f(l_tot) - kPScale) * kLn2;
  };

  // the second block's Q loads go out while the first block finishes
  const bool two = CAUSAL && mt_b != mt_a;
  i32x8 qa[NK], qb[NK];
  load_q(mt_a, qa);
  block(mt_a, qa, [&]() __attribute__((always_inline)) { if (two) load_q(mt_b, qb); });
  if (two) {
    __syncthreads();  // the first block's LDS stages are read no more
    block(mt_b, qb, []() {});
  }
}

#define FP8_KERNEL_ARGS                                                                         \
  const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,  \
      uint16_t* __restrict__ O, float* __restrict__ LSE, int BH, int N, int n_mtiles, float c, \
      float v_descale, int xcd_groups
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_d128(FP8_KERNEL_ARGS) {
  fp8_forward<128, CAUSAL>(Q, K, V, O, LSE, BH, N, n_mtiles, c, v_descale, xcd_groups);
}
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_fp8_d64(FP8_KERNEL_ARGS) {
  fp8_forward<64, CAUSAL>(Q, K, V, O, LSE, BH, N, n_mtiles, c, v_descale, xcd_groups);
}
#undef FP8_KERNEL_ARGS

}  // namespace

static const void* pick_fp8(int d, bool causal) {
  if (d == 64) return causal ? (const void*)attn_fwd_fp8_d64<true> : (const void*)attn_fwd_fp8_d64<false>;
  return causal ? (const void*)attn_fwd_fp8_d128<true> : (const void*)attn_fwd_fp8_d128<false>;
}

hipError_t launch_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                               int B, int H, int N, int d, float scale, float q_descale,
                               float k_descale, float v_descale, bool causal, hipStream_t stream) {
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  int BH = B * H;
  int n_mtiles = (N + kBM - 1) / kBM;
  float c = scale * q_descale * k_descale * kLog2e;
  int xcd_groups = (BH % 8 == 0) ? 1 : 0;
  const int grid = BH * (causal ? (n_mtiles + 1) / 2 : n_mtiles);  // causal: paired blocks
  const void* fn = pick_fp8(d, causal);
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&BH,
                  (void*)&N, (void*)&n_mtiles, (void*)&c, (void*)&v_descale, (void*)&xcd_groups};
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, stream);
}

hipError_t attn_fwd_fp8_attributes(int d, bool causal, hipFuncAttributes* attr, int* threads,
                                   int* blocks_per_cu) {
  const void* fn = pick_fp8(d, causal);
  *threads = kThreads;
  hipError_t e = hipFuncGetAttributes(attr, fn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, *threads, 0);
}

}  // namespace osm
