// Attention backward for gfx950: dQ, dK, dV of O = softmax(scale * Q K^T) V for
// an upstream gradient dO, bf16 / fp16 operands on the 32x32x16 MFMA, fp32
// accumulation.
//
// Method.  The backward pass recomputes the scores instead of storing the
// N x N weights: with the saved per-row statistic lse_i (natural-log
// logsumexp of the scaled scores), every score tile is rebuilt from Q and K and
// normalised in one step, P = exp(scale * s - lse), with no running update
// (backward-pass paragraphs of "Online Softmax: Tiling Across a Reduction").  The gradients are the chain rule through the forward definition:
//     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_j P_ij dP_ij,
//     dQ = scale dS K,  dK = scale dS^T Q,
// and D_i = <dO_i, O_i> because O = P V.  Exponentials run in base 2 with
// c = scale * log2(e) folded into one FMA, P = 2^(c s - lse log2 e).
//
// Two kernels, each owning one side of the score matrix so that every
// gradient row is accumulated in registers by one wave and written once:
//
//  * attn_bwd_dq: a workgroup owns 256 queries (32 per wave), as in the
//    forward kernel, and walks the key tiles.  Per 32-key block:
//    S^T = K Q^T and dP^T = V dO^T (K and V from LDS as A operands, Q^T and
//    dO^T in VGPRs as B operands), so each lane holds one query, whose lse and
//    D are per-lane constants; dS^T = P^T o (dP^T - D) is packed to 16 bits and
//    dQ^T += K^T dS^T takes K^T from LDS through transposing reads.  The lane
//    also forms D_i = <dO_i, O_i> from its rows and writes it to the workspace.
//
//  * attn_bwd_dkdv: a workgroup owns 128 keys (32 per wave pair) and walks the
//    query tiles (64 queries; each wave of a pair takes 32 of them).  Its K and
//    V rows stay in LDS for the whole loop.  S = Q K^T and dP = dO V^T put one
//    key per lane; P and dS = P o (dP - D) are packed to 16 bits and
//    dV^T += dO^T P, dK^T += Q^T dS take dO^T and Q^T through transposing
//    reads.  The two waves of a pair add their partial sums through LDS at
//    the end.
//
// The 16-bit packing of P and dS uses the same trick as the forward kernel:
// the accumulator layout gives a lane its rows in an order that differs from
// the B-operand order by a swap of bits 2 and 3 of the row index; the
// transposing reads of the other operand use the same permutation, since the
// contraction sum does not depend on order.
//
// Causal: key tiles after a query block (dQ) and query tiles before a key
// block (dK, dV) are never visited; tiles straddling the diagonal or the
// ragged end mask element by element (P = dS = 0 there).
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

namespace osm {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;  // 8 waves
constexpr int kQB = 256;       // queries per dQ workgroup
constexpr int kKT = 64;        // keys per dQ key tile
constexpr int kKB = 128;       // keys per dK/dV workgroup
constexpr int kQT = 64;        // queries per dK/dV query tile

// 16-byte chunk swizzle of the backward's LDS tiles (physical chunk = logical ^
// bswz(row)).  The tiles are read two ways: as 16-byte row pieces, 16 lanes
// taking 16 consecutive rows at one logical chunk, and through the transposing
// reads, 32 lanes taking 4 consecutive rows (aligned to 4) x 4 consecutive
// chunks.  With the LDS as 64 banks of 4 bytes, the first needs the swizzles of
// 16 consecutive rows to differ (d = 128; at d = 64, where two 128-byte rows
// share a bank line, those of the 8 rows of each parity), the second needs the
// swizzles of 4 aligned consecutive rows to differ in their high two bits
// (d = 64: rows r and r + 2 in bit 2).  The forward's K-style swizzle (row & 15)
// meets only the first, and its transposing reads then hit 4 banks 4 times over
// (2 times at d = 64).
template <int D>
__device__ __forceinline__ int bswz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Offsets of the transposing reads (ds_read_b64_tr_b16) of a row-major tile in
// the bswz swizzle, for the A operand X^T of X^T Y with X rows = the
// contraction index.  Within each group of 16 lanes the lane at position q
// supplies the address of row R + q/4, columns C + 4 (q % 4) .. +3, and receives
// X[R + k][C + q] for k = 0..3; with R = 4 hf (+ 16-row step, + 32-row block) and
// C = 32 db + 16 ((lane >> 4) & 1) the lane gets its column (32 db + lane % 32)
// at B-operand positions 8 hf .. 8 hf + 3, and a second read 8 rows further
// gives 8 hf + 4 .. 8 hf + 7.  The swizzle of row r + 8 is that of row
// r with one more bit flipped, so the second read has its own offset.
template <int D>
struct TrOffsets {
  static constexpr int ND = D / 32;
  int lo[ND], hi[ND];
  __device__ __forceinline__ explicit TrOffsets(int lane) {
    constexpr int ROW_BYTES = D * 2;
    constexpr int kFlip8 = 2;  // bswz(r + 8) = bswz(r) ^ 2 for rows r with r & 8 == 0
    const int hf = lane >> 5, q = lane & 15;
    const int row = 4 * hf + (q >> 2);
    const int col = 16 * ((lane >> 4) & 1) + 4 * (q & 3);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int ch = (col + 32 * db) >> 3;
      lo[db] = row * ROW_BYTES + (ch ^ bswz<D>(row)) * 16 + (col & 7) * 2;
      hi[db] = (row + 8) * ROW_BYTES + (ch ^ bswz<D>(row) ^ kFlip8) * 16 + (col & 7) * 2;
    }
  }
};

// A operand X^T(16 rows of the contraction starting at tile row `r0`) for column block db.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::v8 read_tr(const unsigned char* tile, const TrOffsets<D>& o,
                                                       int db, int r0) {
  constexpr int ROW_BYTES = D * 2;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + o.lo[db] + r0 * ROW_BYTES));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + o.hi[db] + r0 * ROW_BYTES));
  return __builtin_bit_cast(typename Mma<T>::v8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Row-major tile of `ROWS` rows loaded straight into LDS by all 8 waves, 16-byte
// chunks in the bswz swizzle.  Rows past the buffer's range land as zeros.
template <int D, int ROWS>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t r, unsigned char* lds, int wave_s, int lane) {
  constexpr int ROW_BYTES = D * 2, CPR = D / 8, RPI = 1024 / ROW_BYTES;
  constexpr int NI = ROWS * ROW_BYTES / 1024 / 8;
  static_assert(NI >= 1, "tile shape");
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int row = (wave_s * NI + j) * RPI + lane / CPR;
    const int p = lane % CPR;
    load16_to_lds(r, lds + (wave_s * NI + j) * 1024, row * ROW_BYTES + (p ^ bswz<D>(row)) * 16);
  }
}

// Store a transposed accumulator block set acc[ND] (rows = head dims, column =
// this lane's row of the output) as 16-bit values times `mul`, through LDS: a
// lane holds 4 consecutive head dims of its row per accumulator group, so
// stores straight from the accumulators write 16 bytes into each of 32 rows per
// instruction.  The wave writes its 32 rows into `stage` (32 * D * 2 bytes of
// its own, swizzled like K) and stores whole rows from there, 16 bytes per
// lane.  Every wave of the workgroup calls it (one barrier inside); rows of the
// output past the buffer's range are dropped.
template <typename T, int D>
__device__ __forceinline__ void store_rows(const f32x16* acc, __amdgpu_buffer_rsrc_t r,
                                           unsigned char* stage, int lane, float mul) {
  constexpr int ROW_BYTES = D * 2, ND = D / 32, CPR = D / 8, RPS = 64 / CPR;
  const int l32 = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int db = 0; db < ND; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x2 w = u32x2{pack2<T>(acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul),
                            pack2<T>(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul)};
      *reinterpret_cast<u32x2*>(stage + l32 * ROW_BYTES + (((4 * db + g) ^ (l32 & (CPR - 1))) * 16) + 8 * hf) = w;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 32 / RPS; ++j) {
    const int row = j * RPS + lane / CPR, c = lane % CPR;
    const u32x4 w = *reinterpret_cast<const u32x4*>(stage + row * ROW_BYTES + ((c ^ (row & (CPR - 1))) * 16));
    __builtin_amdgcn_raw_buffer_store_b128(w, r, row * ROW_BYTES + c * 16, 0, 0);
  }
}

// Workgroup id -> (batch*head, block); consecutive ids go round-robin over the
// 8 XCDs, so with xcd_groups each XCD gets a contiguous run of heads (their K/V
// or Q/dO share its L2).  `reverse` hands out the last block of a head first.
__device__ __forceinline__ void block_of(int BH, int n_blocks, int xcd_groups, bool reverse, int* bh,
                                         int* blk) {
  int id = blockIdx.x;
  if (xcd_groups) {
    const int per = gridDim.x >> 3;
    id = (id & 7) * per + (id >> 3);
    *bh = id / n_blocks;
    const int b = id - *bh * n_blocks;
    *blk = reverse ? n_blocks - 1 - b : b;
  } else {
    *bh = id % BH;
    const int b = id / BH;
    *blk = reverse ? n_blocks - 1 - b : b;
  }
}

// ------------------------------------------------------------------------------------
// dQ (and D) : workgroup = 256 queries of one head, key tiles of 64
// ------------------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dq(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO, const float* __restrict__ LSE,
    uint16_t* __restrict__ dQ, float* __restrict__ Dws, int BH, int N, int n_qblocks, float c,
    float scale, int xcd_groups) {
  using v8 = typename Mma<T>::v8;
  constexpr int ROW_BYTES = D * 2;
  constexpr int TILE_BYTES = kKT * ROW_BYTES;
  constexpr int ND = D / 32, NK = D / 16;
  // K and V tiles, two stages each, one array per stage (StageTag)
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

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // causal: blocks qb and n_qblocks - 1 - qb, one after the other, so that every
  // workgroup visits as many key tiles as any other
  int bh, qb_a, qb_b = 0;
  block_of(BH, CAUSAL ? (n_qblocks + 1) >> 1 : n_qblocks, xcd_groups, true, &bh, &qb_b);
  qb_a = CAUSAL ? n_qblocks - 1 - qb_b : qb_b;

  // With rev (the second block of a pair) the key tiles are walked from the
  // diagonal down, so that the second blocks of a head, which start 4 tile times
  // apart, read the same key tile at the same time (as in the forward kernel).
  auto block = [&](const int qb, const bool rev) __attribute__((always_inline)) {
    const int i0 = qb * kQB;
    const size_t base = (size_t)bh * (size_t)N * D;
    const int qw0 = i0 + 32 * wave;  // first query of this wave
    const int qw0_s = __builtin_amdgcn_readfirstlane(qw0);
    const int qi = qw0 + l32;

    // Q^T and dO^T as B operands: lane = query, 8 consecutive head dims per step;
    // D_i = <dO_i, O_i> from the same rows (each lane half holds half the dims)
    v8 qf[NK], dof[NK];
    float Di;
    {
      const int64_t bytes = (int64_t)(N - qw0_s) * ROW_BYTES;
      const auto rq = make_rsrc(Q + base + (size_t)qw0_s * D, bytes);
      const auto rdo = make_rsrc(dO + base + (size_t)qw0_s * D, bytes);
      const auto ro = make_rsrc(O + base + (size_t)qw0_s * D, bytes);
      const int off = l32 * ROW_BYTES + 16 * hf;
      float acc = 0.f;
  #pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        qf[kb] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 32 * kb, 0, 0));
        dof[kb] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rdo, off + 32 * kb, 0, 0));
        const v8 of = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(ro, off + 32 * kb, 0, 0));
  #pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)dof[kb][e], (float)of[e], acc);
      }
      Di = sum_halves(acc);
    }
    const float lse2 = qi < N ? LSE[(size_t)bh * N + qi] * kLog2e : 0.f;
    if (hf == 0 && qi < N) Dws[(size_t)bh * N + qi] = Di;

    f32x16 dq[ND];
  #pragma unroll
    for (int db = 0; db < ND; ++db) dq[db] = f32x16{};

    const int nk_all = (N + kKT - 1) / kKT;
    const int n_kt = CAUSAL ? min(nk_all, (i0 + kQB - 1) / kKT + 1) : nk_all;
    const int n_w = CAUSAL ? min(n_kt, (qw0 + 31) / kKT + 1) : n_kt;  // this wave's last tile + 1

    // K and V rows (A operands, rows = keys) through 16-byte reads
    int kroff[NK];
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb) kroff[kb] = l32 * ROW_BYTES + ((2 * kb + hf) ^ bswz<D>(l32)) * 16;
    const TrOffsets<D> tro(lane);
    const uint16_t* Kh = K + base;
    const uint16_t* Vh = V + base;
    auto load_kv = [&](int t, auto st) __attribute__((always_inline)) {
      const int64_t bytes = (int64_t)(N - t * kKT) * ROW_BYTES;
      load_tile<D, kKT>(make_rsrc(Kh + (size_t)t * kKT * D, bytes), kbuf(st), wave_s, lane);
      load_tile<D, kKT>(make_rsrc(Vh + (size_t)t * kKT * D, bytes), vbuf(st), wave_s, lane);
    };

    auto kt = [&](int i) { return rev ? n_kt - 1 - i : i; };  // key tile at list position i
    // list position i from stage st; the next position loads into the other
    // stage, whose reads (position i - 1) ended at the previous barrier
    auto tile = [&](int i, auto st) __attribute__((always_inline)) {
      if (i + 1 < n_kt) load_kv(kt(i + 1), StageTag<decltype(st)::value ^ 1>{});
      const int t = kt(i);
      if (t < n_w) {
        const unsigned char* Kt = kbuf(st);
        const unsigned char* Vt = vbuf(st);
        const int j0 = t * kKT;
        const bool masked = (j0 + kKT > N) || (CAUSAL && j0 + kKT - 1 > qw0);
  #pragma unroll
        for (int kh = 0; kh < kKT / 32; ++kh) {
          f32x16 s = f32x16{}, dp = f32x16{};
  #pragma unroll
          for (int kb = 0; kb < NK; ++kb) {
            const int o = kroff[kb] + kh * 32 * ROW_BYTES;
            const v8 kf = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(Kt + o));
            const v8 vf = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(Vt + o));
            s = Mma<T>::run(kf, qf[kb], s);
            dp = Mma<T>::run(vf, dof[kb], dp);
          }
          v8 dsf[2];
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(fmaf(s[r], c, -lse2));
            float ds = p * (dp[r] - Di);
            if (masked) {
              const int key = j0 + 32 * kh + 8 * (r >> 2) + 4 * hf + (r & 3);
              if (key >= N || (CAUSAL && key > qi)) ds = 0.f;
            }
            dsf[r >> 3][r & 7] = (T)ds;
          }
  #pragma unroll
          for (int kb = 0; kb < 2; ++kb)
  #pragma unroll
            for (int db = 0; db < ND; ++db)
              dq[db] = Mma<T>::run(read_tr<T, D>(Kt, tro, db, 32 * kh + 16 * kb), dsf[kb], dq[db]);
        }
      }
      vmem_landed();  // tile t + 1
      __syncthreads();
    };

    load_kv(kt(0), StageTag<0>{});
    vmem_landed();
    __syncthreads();
    for (int i = 0; i < n_kt; i += 2) {
      tile(i, StageTag<0>{});
      if (i + 1 < n_kt) tile(i + 1, StageTag<1>{});
    }
    // the last tile's barrier freed the stage arrays: each wave stages its rows
    // in its own half of one of them
    {
      static_assert(TILE_BYTES == 2 * 32 * ROW_BYTES, "dQ staging space");
      // lane rederived here: left to the compiler, the staging addresses would be
      // shared by both blocks of a pair and held through the second
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int arr = wave_s >> 1;
      unsigned char* stg = (arr == 0 ? kb0 : arr == 1 ? kb1 : arr == 2 ? vb0 : vb1) + (wave_s & 1) * 32 * ROW_BYTES;
      store_rows<T, D>(dq, make_rsrc(dQ + base + (size_t)qw0_s * D, (int64_t)(N - qw0_s) * ROW_BYTES), stg, ln, scale);
    }
  };

  block(qb_a, false);
  if (CAUSAL && qb_b != qb_a) {
    __syncthreads();  // the first block's tiles are read no more
    block(qb_b, true);
  }
}

// ------------------------------------------------------------------------------------
// dK, dV : workgroup = 128 keys of one head, query tiles of 64
// ------------------------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_dkdv(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dws,
    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int BH, int N, int n_kblocks, float c,
    float scale, int xcd_groups) {
  using v8 = typename Mma<T>::v8;
  constexpr int ROW_BYTES = D * 2;
  constexpr int ND = D / 32, NK = D / 16;
  constexpr int BLK_BYTES = kKB * ROW_BYTES;   // the workgroup's K (or V) rows
  constexpr int TILE_BYTES = kQT * ROW_BYTES;  // one Q (or dO) tile
  constexpr int STAT_BYTES = kQT * 4;          // one tile of lse (or D)
  // kvblk = the workgroup's K rows then its V rows, loaded once; after the loop
  // it holds the partial sums of the second wave of each pair, dK then dV.  The
  // per-tile Q, dO, lse and D have two stages each, one array per stage
  // (StageTag).
  constexpr int OFF_V = BLK_BYTES;
  constexpr int RED_BYTES = 4 * 64 * ND * 16 * 4;  // one of dK, dV for the four pairs
  static_assert(RED_BYTES <= 2 * BLK_BYTES, "reduction space");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * BLK_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char qb0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char qb1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char db0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) unsigned char db1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lb0[STAT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lb1[STAT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char eb0[STAT_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char eb1[STAT_BYTES];
  auto qbuf = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return qb0; else return qb1;
  };
  auto dobuf = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return db0; else return db1;
  };
  auto lbuf = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return lb0; else return lb1;
  };
  auto dbuf = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return eb0; else return eb1;
  };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  // wave-uniform indices in scalar registers: the accumulators leave few vector ones
  const int kg = wave_s & 3;   // 32-key group of this wave
  const int qh = wave_s >> 2;  // which 32 queries of each tile
  // (key blocks are not paired the way dQ pairs its query blocks: at
  // B8 H32 N8192 d128 causal that measured no faster here)
  int bh, kbk;
  block_of(BH, n_kblocks, xcd_groups, false, &bh, &kbk);
  const int k0 = kbk * kKB;
  const size_t base = (size_t)bh * (size_t)N * D;
  const int key = k0 + 32 * kg + l32;  // this lane's key (column of S)
  const int kw0 = k0 + 32 * kg;        // first key of this wave

  {
    const int64_t bytes = (int64_t)(N - k0) * ROW_BYTES;
    load_tile<D, kKB>(make_rsrc(K + base + (size_t)k0 * D, bytes), smem, wave_s, lane);
    load_tile<D, kKB>(make_rsrc(V + base + (size_t)k0 * D, bytes), smem + OFF_V, wave_s, lane);
  }

  f32x16 dk[ND], dv[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) dk[db] = dv[db] = f32x16{};

  const int n_qt = (N + kQT - 1) / kQT;
  const int qt_first = CAUSAL ? k0 / kQT : 0;
  // 16-byte operand reads: Q / dO rows (A operands, rows = queries) and K / V
  // rows (B operands, column = this lane's key)
  int qroff[NK], kboff[NK];
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) {
    qroff[kb] = (32 * qh + l32) * ROW_BYTES + ((2 * kb + hf) ^ bswz<D>(l32)) * 16;
    kboff[kb] = (32 * kg + l32) * ROW_BYTES + ((2 * kb + hf) ^ bswz<D>(l32)) * 16;
  }
  const TrOffsets<D> tro(lane);
  auto load_qtile = [&](int t, auto st) __attribute__((always_inline)) {
    const int64_t bytes = (int64_t)(N - t * kQT) * ROW_BYTES;
    load_tile<D, kQT>(make_rsrc(Q + base + (size_t)t * kQT * D, bytes), qbuf(st), wave_s, lane);
    load_tile<D, kQT>(make_rsrc(dO + base + (size_t)t * kQT * D, bytes), dobuf(st), wave_s, lane);
    const int64_t sbytes = (int64_t)(N - t * kQT) * 4;
    if (wave_s == 0) load4_to_lds(make_rsrc(LSE + (size_t)bh * N + (size_t)t * kQT, sbytes), lbuf(st), lane * 4);
    if (wave_s == 1) load4_to_lds(make_rsrc(Dws + (size_t)bh * N + (size_t)t * kQT, sbytes), dbuf(st), lane * 4);
  };

  // query tile t from stage st; the next tile loads into the other stage, whose
  // reads (tile t - 1) ended at the previous barrier
  auto tile = [&](int t, auto st) __attribute__((always_inline)) {
    if (t + 1 < n_qt) load_qtile(t + 1, StageTag<decltype(st)::value ^ 1>{});
    const int qa0 = t * kQT + 32 * qh;    // first query of this wave's half
    // skip when every query of the half is before every key of the wave
    if (!CAUSAL || qa0 + 31 >= kw0) {
      const unsigned char* Qt = qbuf(st);
      const unsigned char* dOt = dobuf(st);
      const float* Lt = reinterpret_cast<const float*>(lbuf(st));
      const float* Dt = reinterpret_cast<const float*>(dbuf(st));
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
        const v8 qa = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(Qt + qroff[kb]));
        const v8 da = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(dOt + qroff[kb]));
        const v8 kf = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(smem + kboff[kb]));
        const v8 vf = __builtin_bit_cast(v8, *reinterpret_cast<const u32x4*>(smem + OFF_V + kboff[kb]));
        s = Mma<T>::run(qa, kf, s);
        dp = Mma<T>::run(da, vf, dp);
      }
      const bool masked = (qa0 + 32 > N) || (CAUSAL && qa0 < kw0 + 31);
      v8 pf[2], dsf[2];
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // rows 4j .. 4j + 3: queries 32 qh + 8 j + 4 hf + 0..3
        const int qr = 32 * qh + 8 * j + 4 * hf;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + qr);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dt + qr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          float p = exp2_fast(fmaf(s[r], c, -l4[i] * kLog2e));
          if (masked) {
            const int qa = t * kQT + qr + i;
            if (qa >= N || (CAUSAL && qa < key)) p = 0.f;
          }
          const float ds = p * (dp[r] - d4[i]);
          pf[r >> 3][r & 7] = (T)p;
          dsf[r >> 3][r & 7] = (T)ds;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int db = 0; db < ND; ++db) {
          dv[db] = Mma<T>::run(read_tr<T, D>(dOt, tro, db, 32 * qh + 16 * kb), pf[kb], dv[db]);
          dk[db] = Mma<T>::run(read_tr<T, D>(Qt, tro, db, 32 * qh + 16 * kb), dsf[kb], dk[db]);
        }
      }
    }
    vmem_landed();  // tile t + 1
    __syncthreads();
  };

  if (qt_first < n_qt) load_qtile(qt_first, StageTag<0>{});
  vmem_landed();
  __syncthreads();
  for (int t = qt_first; t < n_qt; t += 2) {
    tile(t, StageTag<0>{});
    if (t + 1 < n_qt) tile(t + 1, StageTag<1>{});
  }

  // The two waves of a pair (qh = 0, 1) hold partial sums over different
  // queries.  The qh = 1 waves leave theirs in LDS (dK in the K/V block, dV in
  // the stage arrays, key group kg in stage array kg), the qh = 0 waves add
  // them and write the 16-bit rows of dK and dV into the K/V block, and all
  // eight waves store whole rows from there (16 bytes per lane, RPS rows per
  // instruction) rather than 16 bytes into each of 32 rows per instruction.
  {
    static_assert(ND * 64 * 64 == TILE_BYTES && 4 * ND * 64 * 64 <= 2 * BLK_BYTES, "staging space");
    f32x16* red_k = reinterpret_cast<f32x16*>(smem) + kg * ND * 64;
    f32x16* red_v = reinterpret_cast<f32x16*>(kg == 0 ? qb0 : kg == 1 ? qb1 : kg == 2 ? db0 : db1);
    if (qh == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        red_k[db * 64 + lane] = dk[db];
        red_v[db * 64 + lane] = dv[db];
      }
    }
    __syncthreads();
    if (qh == 0) {
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        dk[db] += red_k[db * 64 + lane];
        dv[db] += red_v[db * 64 + lane];
      }
    }
    __syncthreads();  // the partial sums are read
    constexpr int CPR = D / 8;  // 16-byte chunks per row
    if (qh == 0) {
      const int kr = 32 * kg + l32;  // this lane's key row in the block
#pragma unroll
      for (int db = 0; db < ND; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int off = kr * ROW_BYTES + (((4 * db + g) ^ (kr & (CPR - 1))) * 16) + 8 * hf;
          *reinterpret_cast<u32x2*>(smem + off) =
              u32x2{pack2<T>(dk[db][4 * g] * scale, dk[db][4 * g + 1] * scale),
                    pack2<T>(dk[db][4 * g + 2] * scale, dk[db][4 * g + 3] * scale)};
          *reinterpret_cast<u32x2*>(smem + BLK_BYTES + off) =
              u32x2{pack2<T>(dv[db][4 * g], dv[db][4 * g + 1]), pack2<T>(dv[db][4 * g + 2], dv[db][4 * g + 3])};
        }
      }
    }
    __syncthreads();  // the rows are in LDS
    // waves 0-3 store the 128 rows of dK, waves 4-7 those of dV
    constexpr int RPS = 64 / CPR;  // rows per store instruction
    const int half = wave_s >> 2, r0 = 32 * (wave_s & 3);
    const int64_t bytes = (int64_t)(N - k0) * ROW_BYTES;
    const auto r = make_rsrc((half ? dV : dK) + base + (size_t)k0 * D, bytes);
    const unsigned char* src = smem + half * BLK_BYTES;
#pragma unroll
    for (int j = 0; j < 32 / RPS; ++j) {
      const int row = r0 + j * RPS + lane / CPR, c = lane % CPR;
      const u32x4 w = *reinterpret_cast<const u32x4*>(src + row * ROW_BYTES + ((c ^ (row & (CPR - 1))) * 16));
      __builtin_amdgcn_raw_buffer_store_b128(w, r, row * ROW_BYTES + c * 16, 0, 0);
    }
  }
}

template <typename T, int D>
struct BwdKernels {
  static const void* dq(bool causal) {
    return causal ? (const void*)attn_bwd_dq<T, D, true> : (const void*)attn_bwd_dq<T, D, false>;
  }
  static const void* dkdv(bool causal) {
    return causal ? (const void*)attn_bwd_dkdv<T, D, true> : (const void*)attn_bwd_dkdv<T, D, false>;
  }
};

void pick_bwd(Elem elem, int d, bool causal, const void** fdq, const void** fdkdv) {
  if (elem == Elem::bf16) {
    *fdq = d == 64 ? BwdKernels<__bf16, 64>::dq(causal) : BwdKernels<__bf16, 128>::dq(causal);
    *fdkdv = d == 64 ? BwdKernels<__bf16, 64>::dkdv(causal) : BwdKernels<__bf16, 128>::dkdv(causal);
  } else {
    *fdq = d == 64 ? BwdKernels<_Float16, 64>::dq(causal) : BwdKernels<_Float16, 128>::dq(causal);
    *fdkdv = d == 64 ? BwdKernels<_Float16, 64>::dkdv(causal) : BwdKernels<_Float16, 128>::dkdv(causal);
  }
}

}  // namespace

hipError_t launch_attn_bwd(Elem elem, const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* workspace, int B, int H, int N, int d, float scale, bool causal,
                           hipStream_t stream) {
  const void *fdq, *fdkdv;
  pick_bwd(elem, d, causal, &fdq, &fdkdv);
  int BH = B * H;
  float c = scale * kLog2e;
  int xcd_groups = (BH % 8 == 0) ? 1 : 0;
  int n_qblocks = (N + kQB - 1) / kQB;
  const int dq_grid = BH * (causal ? (n_qblocks + 1) / 2 : n_qblocks);  // causal: paired blocks
  void* a1[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&dout, (void*)&lse, (void*)&dq,
                (void*)&workspace, (void*)&BH, (void*)&N, (void*)&n_qblocks, (void*)&c, (void*)&scale,
                (void*)&xcd_groups};
  hipError_t e = hipLaunchKernel(fdq, dim3(dq_grid), dim3(kThreads), a1, 0, stream);
  if (e != hipSuccess) return e;
  int n_kblocks = (N + kKB - 1) / kKB;
  const float* dws = workspace;
  void* a2[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&dout, (void*)&lse, (void*)&dws, (void*)&dk,
                (void*)&dv, (void*)&BH, (void*)&N, (void*)&n_kblocks, (void*)&c, (void*)&scale,
                (void*)&xcd_groups};
  return hipLaunchKernel(fdkdv, dim3(BH * n_kblocks), dim3(kThreads), a2, 0, stream);
}

hipError_t attn_bwd_attributes(Elem elem, int d, bool causal, int which, hipFuncAttributes* attr,
                               int* threads, int* blocks_per_cu) {
  const void *fdq, *fdkdv;
  pick_bwd(elem, d, causal, &fdq, &fdkdv);
  const void* fn = which == 0 ? fdq : fdkdv;
  *threads = kThreads;
  hipError_t e = hipFuncGetAttributes(attr, fn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, *threads, 0);
}

}  // namespace osm
