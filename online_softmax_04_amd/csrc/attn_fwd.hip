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
// c * score; the logsumexp written out is ln 2 * (m + log2 l).  The row sum
// in l runs on the matrix unit over P after its rounding to 16 bits, the same
// values that multiply V: O / l then weights V by exactly the rounded P
// normalised to 1, and a rounding error d of one weight moves O by
// d p (v - O) / l, not by d p v / l.
//
// The m carried here is a reference point that trails the running maximum by
// at most kSlack = 8 (a factor 2^8): it moves to the new maximum only when
// that exceeds it by more than kSlack.  Any reference gives the same O / l and
// m + log2 l, because l and O are scaled by the same 2^(-m); the eager rule
// above is the case kSlack = 0.  Every exponential stays at or below 2^8, far
// from fp32 and bf16/fp16 overflow, and the rescale of O (D/2 multiplies per
// lane) runs only on the rare tiles where some row's reference moves.
//
// Work decomposition.  A workgroup of 8 waves owns 256 consecutive queries of
// one (batch, head); each wave owns 32 of them, and all 8 share each K/V tile
// staged in LDS.  Key tiles are 64 keys at d = 128 and 128 keys at d = 64.  The
// waves form two groups of four that run half a tile apart (slot schedule in
// the kernel): in every phase one
// wave per SIMD issues MFMAs while the other runs the softmax on the vector
// ALU, so the matrix unit is not left idle during the softmax.
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
// Loader.  K and V tiles go from global memory straight into LDS with buffer
// loads that write LDS directly (no register staging), 16 bytes per lane.  The
// buffer base is advanced by whole tiles on the scalar unit, so a load needs no
// vector address arithmetic, and rows past N fall outside the buffer's range
// and read as zero (their scores are masked).  Half the waves issue the loads,
// spread between their MFMAs (slot schedule in the kernel).  K and V have
// separate double buffers.  Both are stored row-major with 16-byte chunks XOR-swizzled by row
// so that the MFMA operand reads spread over the LDS banks; V^T operands are
// read with the transposing ds_read_b64_tr_b16.
//
// Causal.  Key tiles wholly after the query block are never visited, tiles
// wholly before it run without a mask, and only tiles straddling the diagonal
// (or the ragged end of the sequence) mask element by element ("Online Softmax:
// Tiling Across a Reduction", causal paragraphs).  A wave stops computing at
// the last tile holding a key visible to one of its queries.  With 16-bit
// operands a workgroup takes two query blocks, one near each end of the
// sequence, so that every workgroup holds the same number of key tiles;
// otherwise query blocks are handed out longest first.
#include "common.h"
#include "kernels.h"
#include "mfma_tile.h"

#include <type_traits>

namespace osm {
namespace {

// Wave-wide minimum and maximum of an int: prefix steps through DPP row shifts
// (1, 2, 4, 8 lanes) leave each 16-lane row's result in its last lane, two row
// broadcasts carry those on to lane 63, which is read out (wave-uniform).
// Lanes a shift or broadcast does not reach keep the identity.
__device__ __forceinline__ int wave_min_i32(int v) {
  constexpr int kId = 0x7fffffff;
  v = min(v, __builtin_amdgcn_update_dpp(kId, v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = min(v, __builtin_amdgcn_update_dpp(kId, v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = min(v, __builtin_amdgcn_update_dpp(kId, v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = min(v, __builtin_amdgcn_update_dpp(kId, v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = min(v, __builtin_amdgcn_update_dpp(kId, v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = min(v, __builtin_amdgcn_update_dpp(kId, v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  constexpr int kId = (int)0x80000000;
  v = max(v, __builtin_amdgcn_update_dpp(kId, v, 0x111, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(kId, v, 0x112, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(kId, v, 0x114, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(kId, v, 0x118, 0xf, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(kId, v, 0x142, 0xa, 0xf, false));
  v = max(v, __builtin_amdgcn_update_dpp(kId, v, 0x143, 0xc, 0xf, false));
  return __builtin_amdgcn_readlane(v, 63);
}

// two 16-bit ones in one word
template <typename T>
constexpr unsigned kOnePair = sizeof(T) == 2 && __is_same(T, __bf16) ? 0x3f803f80u : 0x3c003c00u;

constexpr float kSlack = 8.f;  // how far (log2 units) the running maximum may pass m
constexpr int kBM = 256;       // queries per workgroup
// keys per tile: 128 at d = 64, where the per-tile fixed costs weigh most and the
// registers allow it (222 VGPRs); 64 at d = 128 (217 VGPRs, 128 would need 250+).
// The causal kernels, with two query blocks inlined, take 226 and 237.
template <int D>
constexpr int kBN = D == 64 ? 128 : 64;
constexpr int kThreads = 512;  // 8 waves: two groups of 4, one wave of each group per SIMD


// MASK: kMaskNone, kMaskLocal or kMaskSparse (kernels.h)
template <typename T, int D, bool CAUSAL, int MASK>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int BH,
    int N, int n_mtiles, float c, int xcd_groups, int H, const int* __restrict__ doc_start,
    int window, const int* __restrict__ blk_ptr, const int* __restrict__ blk_idx, int nnz,
    int pairs) {
  constexpr bool LOCAL = MASK == kMaskLocal;
  constexpr bool SPARSE = MASK == kMaskSparse;
  using v8 = typename Mma<T>::v8;
  constexpr int ROW_BYTES = D * 2;
  constexpr int BN = kBN<D>;                  // keys per tile
  constexpr int TILE_BYTES = BN * ROW_BYTES;   // one K or V tile
  constexpr int ND = D / 32;                   // 32-dim blocks of O^T per wave
  constexpr int NK = D / 16;                   // 16-deep MFMA steps of K Q^T
  constexpr int NH = BN / 32;                  // 32-key blocks of a tile
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int RPI = 1024 / ROW_BYTES;        // rows per 1 KiB wave-wide load
  // Only group 0 loads, in slot Y where it runs the products, with its loads
  // spread between the MFMAs.  A wave-wide load occupies the texture unit for
  // several cycles, and a wave that issues one while the unit is busy stalls:
  // eight waves each issuing their loads at the top of a slot held the softmax
  // waves up for hundreds of cycles.
  constexpr bool LG = true;
  constexpr int NI = TILE_BYTES / 1024 / (LG ? 4 : 8);  // such loads per loading wave per tile
  static_assert(NI >= 1, "tile shape");
  // One array per stage and operand, always named at compile time: the compiler
  // tracks the pending direct loads per array, so a read of one stage does not
  // wait for the loads into the other.  The tile at list position i (below)
  // lives in stage i & 1.
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
  // Waves w and w + 4 share a SIMD; they belong to different groups, which run
  // half a tile apart (see the slot schedule below).
  const int group = wave >> 2;

  // ---- which (batch*head, query blocks) this workgroup owns --------------------
  // With pairs, a workgroup takes two query blocks of one head, mt and
  // n_mtiles - 1 - mt, one after the other: under the causal mask every such
  // pair holds the same number of key tiles.  The dispatcher hands workgroups to
  // the compute units of an XCD in order, so with one block per workgroup the
  // unequal causal blocks left compute units idle between workgroups (9% of
  // the time at B8 H32 N8192, measured from per-workgroup timestamps).
  const bool paired = CAUSAL && MASK == kMaskNone && pairs;  // compiled out elsewhere
  int id = blockIdx.x, bh, mt_a, mt_b = 0;
  const int n_units = paired ? (n_mtiles + 1) >> 1 : n_mtiles;
  if (xcd_groups) {
    // consecutive workgroup ids go round-robin over the 8 XCDs; give each XCD a
    // contiguous run of heads so the blocks sharing a head's K/V share its L2
    const int per = gridDim.x >> 3;
    id = (id & 7) * per + (id >> 3);
    bh = id / n_units;
    mt_a = n_units - 1 - (id - bh * n_units);
    if constexpr (LOCAL) {
      // document boundaries differ between batch rows, so a run of one row's
      // heads per XCD left the XCDs unequal work (they finished up to 8% apart
      // at B8 H32 N8192); give each XCD the same heads of every batch row
      const int nb = BH / H;
      bh = (bh % nb) * H + bh / nb;
    }
  } else {
    bh = id % BH;
    mt_a = n_units - 1 - id / BH;
  }
  if (paired) {
    mt_b = mt_a;
    mt_a = n_mtiles - 1 - mt_b;
  }

  // the window kernel's first K tile depends on the document bounds of the
  // block's queries: their load goes out ahead of the Q loads
  int doc_first = 0;
  if constexpr (LOCAL) {
    if (doc_start) {
      const int q = min(mt_a * kBM + 32 * (2 * (wave & 3) + group) + l32, N - 1);
      doc_first = doc_start[(size_t)(bh / H) * N + q];
    }
  }

  // Q^T fragments of query block mt: B operand, lane = query, 8 consecutive head dims
  auto load_q = [&](const int mt, v8 (&qf)[NK]) __attribute__((always_inline)) {
    const int qw0 = mt * kBM + 32 * (2 * (wave & 3) + group);
    const int qw0_s = __builtin_amdgcn_readfirstlane(qw0);
    const auto rq = make_rsrc(Q + (size_t)bh * (size_t)N * D + (size_t)qw0_s * D,
                              (int64_t)(N - qw0_s) * ROW_BYTES);
    const int off = l32 * ROW_BYTES + 16 * hf;
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb)
      qf[kb] = __builtin_bit_cast(v8, __builtin_amdgcn_raw_buffer_load_b128(rq, off + 32 * kb, 0, 0));
  };

  // one query block; called twice when paired (inlined twice: a loop around it
  // spilled registers).  after_loop runs once the block's last Q^T read is done.
  // With rev (the second block of a pair), the key tiles are walked from the
  // diagonal down to tile 0.  Pair j ends its first block 4 tile times after pair
  // j + 1, whose second block is 4 tiles longer: walked downwards, all second
  // blocks of a head read the same key tile at the same time and share it in L2;
  // walked upwards they would read tiles 4 apart.
  auto block = [&](const int mt, v8 (&qf)[NK], auto&& after_loop, const bool rev) __attribute__((always_inline)) {
    const int i0 = mt * kBM;
    const size_t base = (size_t)bh * (size_t)N * D;
    const uint16_t* Kh = K + base;
    const uint16_t* Vh = V + base;
    // 32-query blocks of the workgroup interleave between the groups, so both
    // groups reach the causal diagonal at nearly the same key tile
    const int qw0 = i0 + 32 * (2 * (wave & 3) + group);  // first query of this wave
    const int qi = qw0 + l32;                             // this lane's query
    // qw0 is uniform across the wave; the buffer descriptors built from it must
    // be scalar, or every access through them becomes a per-lane loop
    const int qw0_s = __builtin_amdgcn_readfirstlane(qw0);


    f32x16 o[ND];
  #pragma unroll
    for (int db = 0; db < ND; ++db) o[db] = f32x16{};
    f32x16 s[NH];
    // The row sum of P runs on the matrix unit, one 16x16x32 MFMA per 16-key step
    // (half the cycles of a 32x32x16 one): on the vector ALU the sum of the
    // 16-bit P takes two-term dot products, which wait for the matrix unit while
    // the other wave of the SIMD keeps it busy (measured slower at both head
    // dims).  Read as the 16x16x32 B operand, P^T's register puts column c of
    // lane group g = l / 16 in lane c + 16 g, i.e. query c + 16 (g % 2), keys of
    // half g / 2.  An A operand with ones in rows 0 and 8 for the even groups and
    // rows 4 and 12 for the odd ones (zeros elsewhere) makes accumulator row
    // 4 (l / 16) of lane l -- its register 0 -- the step's sum for query l % 32,
    // in both lane halves; the other registers stay zero.
    f32x4v lacc = f32x4v{};
    v8 ones;
    {
      const int r16 = lane & 15, g16 = lane >> 4;
      const unsigned w = ((r16 & 3) == 0 && ((r16 >> 2) & 1) == (g16 & 1)) ? kOnePair<T> : 0u;
      ones = __builtin_bit_cast(v8, u32x4{w, w, w, w});
    }
    v8 pf[NH][2];  // P^T as 16-bit B operands: [32-key block][16-key step]
    float m_run = kNegInf;

    const int nk_all = (N + BN - 1) / BN;
    const int n_kt = CAUSAL ? min(nk_all, (i0 + kBM - 1) / BN + 1) : nk_all;
    // tiles holding a key visible to some query of this wave
    int n_w = CAUSAL ? min(n_kt, (qw0 + 31) / BN + 1) : n_kt;
    // Without the causal limit the compiler would prove n_w == n_kt, drop the
    // per-wave tests and merge the slots into blocks it schedules with more
    // values live than fit in registers; keep the tests in place.
    asm volatile("" : "+v"(n_w));

    // LOCAL (with CAUSAL): query i sees keys lo_i .. i, lo_i = max(document start,
    // i - window + 1).  Whole tiles before a wave's smallest lo_i are skipped (tw0),
    // the workgroup loads from the smallest over its waves (t0), and tiles reaching
    // below a wave's largest lo_i are masked element by element.
    int lo_i = 0, lo_max_w = 0, tw0 = 0, t0 = 0;
    if constexpr (LOCAL) {
      const int qc = min(qi, N - 1);
      int lo = doc_first;
      asm volatile("" : "+v"(lo));  // consumed here, after the Q loads went out
      lo = min(max(lo, 0), qc);
      if (window > 0) lo = max(lo, qc - window + 1);
      lo_i = lo;
      lo_max_w = wave_max_i32(lo);
      tw0 = wave_min_i32(lo) / BN;
      __shared__ int wave_first[kThreads / 64];
      if (lane == 0) wave_first[wave] = tw0;
      __syncthreads();
      t0 = wave_first[0];
  #pragma unroll
      for (int w = 1; w < kThreads / 64; ++w) t0 = min(t0, wave_first[w]);
    }
    // tile t holds keys this wave computes with
    auto act = [&](int t) { return (!LOCAL || t >= tw0) && t < n_w; };

    // The workgroup walks a list of key tiles: position i holds tile t0 + i for the
    // dense and sliding-window kernels; for block-sparse, the tiles of the key
    // blocks listed for this query block (ascending, as the pattern lists them).
    // Causal masking and the key count N apply on top.
    constexpr int kTilesPerBlock = kSparseKBlock / BN;
    const int nkb = (N + kSparseKBlock - 1) / kSparseKBlock;  // key blocks
    int n_list = n_kt - t0, p0 = 0;
    if constexpr (SPARSE) {
      static_assert(kBM == kSparseQBlock && kSparseKBlock % BN == 0, "pattern blocks");
      // the row's range, clamped into [0, nnz]
      p0 = min(max(blk_ptr[mt], 0), nnz);
      n_list = (min(max(blk_ptr[mt + 1], p0), nnz) - p0) * kTilesPerBlock;
    }
    auto tile_of = [&](int i) -> int {
      if constexpr (SPARSE) {
        // a block index outside [0, nkb) maps past the last key: no load, no compute
        const unsigned b = (unsigned)blk_idx[p0 + i / kTilesPerBlock];
        return (int)min(b, (unsigned)nkb) * kTilesPerBlock + i % kTilesPerBlock;
      } else {
        return rev ? n_kt - 1 - i : t0 + i;
      }
    };
    // last key a tile may start at and still hold a key this wave computes with;
    // opaque to the compiler for the reason n_w is
    int j0_max = CAUSAL ? min(qw0 + 31, N - 1) : N - 1;
    if constexpr (SPARSE) asm volatile("" : "+v"(j0_max));
    // list position i holds keys this wave computes with
    auto act_at = [&](int i) {
      if constexpr (SPARSE) {
        return tile_of(i) * BN <= j0_max;
      } else {
        return act(tile_of(i));
      }
    };

    // ---- loader: global -> LDS directly, no registers ------------------------------------
    // A wave-wide 16-byte-per-lane buffer load with the LDS flag writes lane i's
    // 16 bytes at (LDS base + 16 i): each of the wave's NI loads fills RPI whole
    // rows, and each lane fetches the global chunk that its LDS slot holds under
    // the swizzle.  Rows past N fall outside the buffer and land as zeros.
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    int kgoff[NI], vgoff[NI];
  #pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int row = ((LG ? wave & 3 : wave) * NI + j) * RPI + lane / CPR;
      const int p = lane % CPR;
      kgoff[j] = row * ROW_BYTES + (p ^ kswz<D>(row)) * 16;
      vgoff[j] = row * ROW_BYTES + (p ^ vswz<D>(row)) * 16;
    }
    // valid = false gives an empty buffer: the loads then read nothing and write
    // zeros into the stage
    auto load_k = [&](int t, auto st, bool valid = true) __attribute__((always_inline)) {
      const auto r = make_rsrc(Kh + (size_t)t * BN * D, valid ? (int64_t)(N - t * BN) * ROW_BYTES : 0);
  #pragma unroll
      for (int j = 0; j < NI; ++j)
        load16_to_lds(r, kbuf(st) + ((LG ? wave_s & 3 : wave_s) * NI + j) * 1024, kgoff[j]);
    };
    auto load_v = [&](int t, auto st, bool valid = true) __attribute__((always_inline)) {
      const auto r = make_rsrc(Vh + (size_t)t * BN * D, valid ? (int64_t)(N - t * BN) * ROW_BYTES : 0);
  #pragma unroll
      for (int j = 0; j < NI; ++j)
        load16_to_lds(r, vbuf(st) + ((LG ? wave_s & 3 : wave_s) * NI + j) * 1024, vgoff[j]);
    };
    // direct loads write LDS behind the compiler's back: wait for them explicitly
    auto loads_landed = [&]() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    // ---- operand read offsets -------------------------------------------------------------
    // K (A operand of S^T = K Q^T): row l32 (+32 for the second key half), logical
    // chunk 2 kb + hf.  Rows 32 apart share a swizzle.
    int kroff[NK];
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb) kroff[kb] = l32 * ROW_BYTES + ((2 * kb + hf) ^ kswz<D>(l32)) * 16;
    // V^T (A operand of O^T = V^T P^T) through ds_read_b64_tr_b16: within each
    // group of 16 lanes, the lane at position q supplies the address of row
    // R + q/4, head dims C + 4 (q % 4) .. +3, and receives V[R + k][C + q] for
    // k = 0..3.  With R = 32 kh + 16 kb + 4 hf and C = 32 db + 16 ((lane >> 4) & 1)
    // the lane gets its head dim (32 db + lane % 32) at the keys of B-operand
    // positions 8 hf .. 8 hf + 3; a second read 8 rows further gives 8 hf + 4 ..
    // 8 hf + 7 (the P^T key permutation).  Row steps of 4 keep the swizzle.
    int vroff[ND];
    {
      const int q = lane & 15;
      const int row = 4 * hf + (q >> 2);
      const int col = 16 * ((lane >> 4) & 1) + 4 * (q & 3);
  #pragma unroll
      for (int db = 0; db < ND; ++db)
        vroff[db] = row * ROW_BYTES + (((col + 32 * db) >> 3) ^ vswz<D>(row)) * 16 + (col & 7) * 2;
    }

    // ---- the three pieces of a tile --------------------------------------------------------
    // QK: S^T = K Q^T, one accumulator per 32-key block, from K stage st.
    auto qk = [&](auto st) __attribute__((always_inline)) {
      const unsigned char* Kt = kbuf(st);
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh) s[kh] = f32x16{};
  #pragma unroll
      for (int kb = 0; kb < NK; ++kb) {
  #pragma unroll
        for (int kh = 0; kh < NH; ++kh) {
          const v8 kf = __builtin_bit_cast(
              v8, *reinterpret_cast<const u32x4*>(Kt + kroff[kb] + kh * 32 * ROW_BYTES));
          s[kh] = Mma<T>::run(kf, qf[kb], s[kh]);
        }
      }
    };
    // SM(t): online softmax of S(t): m, l and O rescaled by 2^(m_old - m_new),
    // P = 2^(c S - m_new) packed to 16 bits, with m the trailing reference.
    auto sm = [&](int t) __attribute__((always_inline)) {
      const int j0 = t * BN;
      // keys past N, and keys after the query when causal (wave-uniform test)
      if ((j0 + BN > N) || (CAUSAL && j0 + BN - 1 > qw0) || (LOCAL && j0 < lo_max_w)) {
  #pragma unroll
        for (int kh = 0; kh < NH; ++kh) {
  #pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * kh + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key >= N || (CAUSAL && key > qi) || (LOCAL && key < lo_i)) s[kh][r] = kNegInf;
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
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh) {
  #pragma unroll
        for (int r = 0; r < 16; ++r) pf[kh][r >> 3][r & 7] = (T)exp2_fast(fmaf(s[kh][r], c, -m_sub));
      }
      m_run = m_new;
      if (__any(alpha != 1.f)) {  // wave-uniform; skipped while no row's reference moves
  #pragma unroll
        for (int db = 0; db < ND; ++db) o[db] *= alpha;
        lacc[0] *= alpha;
      }
    };
    // PV: O^T += V^T P^T, from V stage st.
    // the row sums of P alone: l += rowsum P over the tile's four 16-key steps
    auto rowsums = [&]() __attribute__((always_inline)) {
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh)
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) lacc = Mma<T>::run16(ones, pf[kh][kb], lacc);
    };
    auto pv = [&](auto st, bool with_rowsums = true) __attribute__((always_inline)) {
      const unsigned char* Vt = vbuf(st);
  #pragma unroll
      for (int kh = 0; kh < NH; ++kh) {
  #pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
  #pragma unroll
          for (int db = 0; db < ND; ++db) {  // ND independent accumulators in flight
            const unsigned char* pa = Vt + vroff[db] + (32 * kh + 16 * kb) * ROW_BYTES;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(pa + 8 * ROW_BYTES));
            const v8 vf = __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[db] = Mma<T>::run(vf, pf[kh][kb], o[db]);
          }
          if (with_rowsums) lacc = Mma<T>::run16(ones, pf[kh][kb], lacc);
        }
      }
    };

    // Row sums, PV(tp), then QK(tq) in one block, with the LDS operand reads running
    // a fixed distance ahead of the MFMAs that consume them: enough reads in flight
    // to cover LDS latency, few enough registers to avoid spilling.  The row sums
    // read only registers, so they go first and run while the first PV operands
    // are read (in slot Y the stages were published by the barrier just before).
    // Their order, and so l, is that of the PV loop.  nld (a compile-time count)
    // direct loads issued by loads() are spread evenly between the MFMAs.
    auto pv_qk = [&](auto stp, auto stq, auto nld, auto&& loads) __attribute__((always_inline)) {
      constexpr int NL = decltype(nld)::value;
      loads();
      rowsums();
      pv(stp, false);
      qk(stq);
      constexpr int kAhead = 4;  // operand-reading MFMAs whose reads are issued ahead
      constexpr int kRs = 2 * NH, kPv = 2 * NH * ND, kQk = NH * NK;
      constexpr int kTot = kRs + kPv + kQk;
      // operand-reading MFMA k: PV (two transposed reads) for k < kPv, then QK (one read)
  #pragma unroll
      for (int k = 0; k < kAhead; ++k) {
        if (k < kPv) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
        else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      constexpr int kEvery = NL ? kTot / (NL + 1) : 1;
  #pragma unroll
      for (int i = 0; i < kTot; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        if (NL && i % kEvery == kEvery - 1 && i / kEvery < NL)
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one direct load
        if (i >= kRs) {
          const int k = i - kRs + kAhead;
          if (k < kPv) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          else if (k < kPv + kQk) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    };

    // The tile at list position i, in stage S = i & 1: slot X, the barrier, slot Y.
    auto tile = [&](int i, auto st) __attribute__((always_inline)) {
      constexpr int S = decltype(st)::value;
      const StageTag<S> cur;
      const StageTag<S ^ 1> other;
      const bool a_cur = act_at(i);
      // ---- slot X
      if (group == 0) {
        if (a_cur) sm(tile_of(i));
      } else {
        __builtin_amdgcn_s_setprio(1);
        const bool a_prev = i > 0 && act_at(i - 1);
        if (a_prev && a_cur) {
          pv_qk(other, cur, std::integral_constant<int, 0>{}, [] {});
        } else {
          if (a_prev) pv(other);
          if (a_cur) qk(cur);
        }
        __builtin_amdgcn_s_setprio(0);
      }
      loads_landed();  // K of position i + 1, V of position i
      __syncthreads();
      // ---- slot Y
      if (group == 0) {
        __builtin_amdgcn_s_setprio(1);
        const bool a_next = i + 1 < n_list && act_at(i + 1);
        // K(i + 2) into the stage K(i) leaves, V(i + 1) into the one V(i - 1) left;
        // past the end of the list the loads are empty, and the zeros they write
        // land in stages that no later read uses.  Unconditional loads keep the
        // block straight, so the schedule can spread them.
        const bool k_ok = i + 2 < n_list, v_ok = i + 1 < n_list;
        const int tk = k_ok ? tile_of(i + 2) : 0, tv = v_ok ? tile_of(i + 1) : 0;
        auto loads = [&]() __attribute__((always_inline)) {
          load_k(tk, cur, k_ok);
          load_v(tv, other, v_ok);
        };
        if (a_cur && a_next) {
          pv_qk(cur, other, std::integral_constant<int, 2 * NI>{}, loads);
        } else {
          loads();
          if (a_cur) pv(cur);
          if (a_next) qk(other);
        }
        __builtin_amdgcn_s_setprio(0);
      } else {
        if (a_cur) sm(tile_of(i));
      }
    };

    // ---- slot schedule ----------------------------------------------------------------
    // Each tile t takes two slots:
    //   slot X(t): group 0 runs SM(t)          group 1 runs PV(t-1), QK(t)
    //   slot Y(t): group 0 runs PV(t), QK(t+1) group 1 runs SM(t)
    // so on every SIMD one wave keeps the matrix unit busy while the other runs
    // the vector-ALU softmax.  K(t+1) and V(t) are read from Y(t) to X(t+1); group
    // 0 issues their loads between its MFMAs in Y(t-1) (into the stages of K(t-1)
    // and V(t-1), last read in X(t-1)), they land during Y(t-1) and X(t), and the
    // workgroup barrier that ends X(t) publishes them.  That barrier is the only one per tile: no LDS stage changes
    // hands between Y(t) and X(t+1), and meeting once per tile keeps the two
    // groups in opposite phases.  The dense kernel starts at tile t0 = 0; the
    // LOCAL one at the workgroup's first visible tile, each wave computing from
    // its own first tile tw0.
    const bool loader = !LG || group == 0;
    if (loader && n_list > 0) load_k(tile_of(0), StageTag<0>{});
    loads_landed();
    __syncthreads();
    // Retire the Q loads here.  Left pending, they would make the first MFMA that
    // reads Q wait on the vector-memory counter, which then also counts the tile
    // loads in flight.
  #pragma unroll
    for (int kb = 0; kb < NK; ++kb) asm volatile("" ::"v"(qf[kb]));
    // slot Y(t0 - 1): load K(t0+1), V(t0); group 0 computes S(t0)
    if (loader && 1 < n_list) load_k(tile_of(1), StageTag<1>{});
    if (loader && n_list > 0) load_v(tile_of(0), StageTag<0>{});
    if (group == 0 && n_list > 0 && act_at(0)) {
      __builtin_amdgcn_s_setprio(1);
      qk(StageTag<0>{});
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
    for (int i = 0; i < n_list; i += 2) {
      tile(i, StageTag<0>{});
      if (i + 1 < n_list) tile(i + 1, StageTag<1>{});
    }
    after_loop();
    // slot X after the last tile: group 1 finishes the last PV
    if (group == 1 && n_list > 0 && act_at(n_list - 1)) {
      if (((n_list - 1) & 1) == 0) pv(StageTag<0>{}); else pv(StageTag<1>{});
    }

    // ---- epilogue: O / l, logsumexp --------------------------------------------------
    const float l_tot = lacc[0];
    // a block-sparse row can see no key at all: O = 0 and logsumexp -inf there
    const float inv = (SPARSE && l_tot == 0.f) ? 0.f : 1.f / l_tot;
    if constexpr (D == 128) {
      // O leaves through LDS: a lane holds 4 consecutive dims of its query per
      // accumulator group, so storing from registers writes 16 bytes into each of
      // 32 rows per instruction; staged row-major, every store writes whole rows.
      // Each wave stages its 32 rows in its own part of the stage arrays, free
      // once every wave is past its last product.
      constexpr int WAVE_BYTES = 32 * ROW_BYTES;
      constexpr int PER_ARRAY = TILE_BYTES / WAVE_BYTES;  // waves per stage array
      static_assert(PER_ARRAY >= 2 && kThreads / 64 / PER_ARRAY <= 4, "O staging space");
      const int arr = wave_s / PER_ARRAY;
      unsigned char* stg = (arr == 0 ? kb0 : arr == 1 ? kb1 : arr == 2 ? vb0 : vb1) +
                           (wave_s % PER_ARRAY) * WAVE_BYTES;
      // lane indices rederived here: left to the compiler, the addresses below
      // would be shared by both blocks of a pair and held through the second
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int lr = ln & 31, lh = ln >> 5;
      __syncthreads();  // group 1 has run the last PV
  #pragma unroll
      for (int db = 0; db < ND; ++db) {
  #pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x2 w = u32x2{pack2<T>(o[db][4 * g] * inv, o[db][4 * g + 1] * inv),
                                pack2<T>(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv)};
          const int ch = (4 * db + g) ^ (lr & (CPR - 1));
          *reinterpret_cast<u32x2*>(stg + lr * ROW_BYTES + ch * 16 + 8 * lh) = w;
        }
      }
      __syncthreads();  // the wave's rows are in LDS
      // rows past N fall outside the buffer and are dropped
      const auto ro = make_rsrc(O + base + (size_t)qw0_s * D, (int64_t)(N - qw0_s) * ROW_BYTES);
      constexpr int RPS = 64 / CPR;  // rows per store
  #pragma unroll
      for (int j = 0; j < 32 / RPS; ++j) {
        const int row = j * RPS + ln / CPR, c = ln % CPR;
        const u32x4 w = *reinterpret_cast<const u32x4*>(stg + row * ROW_BYTES + ((c ^ (row & (CPR - 1))) * 16));
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, row * ROW_BYTES + c * 16, 0, 0);
      }
    } else {
      // (at d = 64 staging through LDS measured no faster)
      // rows past N fall outside the buffer and are dropped
      const auto ro = make_rsrc(O + base + (size_t)qw0_s * D, (int64_t)(N - qw0_s) * ROW_BYTES);
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
      LSE[(size_t)bh * N + qi] = (SPARSE && l_tot == 0.f) ? kNegInf : (m_run + log2f(l_tot)) * kLn2;
  };

  // the second block's Q loads go out while the first block finishes
  const bool two = paired && mt_b != mt_a;
  v8 qa[NK], qb[NK];
  load_q(mt_a, qa);
  block(mt_a, qa, [&]() __attribute__((always_inline)) { if (two) load_q(mt_b, qb); }, false);
  if (two) {
    __syncthreads();  // the first block's LDS stages are read no more
    block(mt_b, qb, []() {}, true);
  }
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
const void* mfma_fn(int mask) {
  if (mask == kMaskSparse) return (const void*)attn_fwd_mfma<T, D, C, kMaskSparse>;
  if constexpr (C) {
    if (mask == kMaskLocal) return (const void*)attn_fwd_mfma<T, D, true, kMaskLocal>;
  }
  return (const void*)attn_fwd_mfma<T, D, C, kMaskNone>;
}

// mask: kMaskNone, kMaskLocal (requires causal) or kMaskSparse; 16-bit operands
// only for the last two
const void* pick_attn(Elem elem, int d, bool causal, int* threads, int* rows_per_block,
                      int mask = kMaskNone) {
  if (elem == Elem::f32) {
    *threads = 256;
    *rows_per_block = 4 * (64 / (d / 64));
    if (d == 64) return causal ? (const void*)attn_fwd_f32<64, true> : (const void*)attn_fwd_f32<64, false>;
    return causal ? (const void*)attn_fwd_f32<128, true> : (const void*)attn_fwd_f32<128, false>;
  }
  *threads = kThreads;
  *rows_per_block = kBM;
  if (elem == Elem::bf16) {
    if (d == 64) return causal ? mfma_fn<__bf16, 64, true>(mask) : mfma_fn<__bf16, 64, false>(mask);
    return causal ? mfma_fn<__bf16, 128, true>(mask) : mfma_fn<__bf16, 128, false>(mask);
  }
  if (d == 64) return causal ? mfma_fn<_Float16, 64, true>(mask) : mfma_fn<_Float16, 64, false>(mask);
  return causal ? mfma_fn<_Float16, 128, true>(mask) : mfma_fn<_Float16, 128, false>(mask);
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
  // causal: two query blocks of unequal length per workgroup (see the kernel)
  int pairs = (causal && elem != Elem::f32) ? 1 : 0;
  const int grid = BH * (pairs ? (n_mtiles + 1) / 2 : n_mtiles);
  if (elem == Elem::f32) {
    void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse,
                    (void*)&BH, (void*)&N, (void*)&n_mtiles, (void*)&c};
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
  }
  int xcd_groups = (BH % 8 == 0) ? 1 : 0;
  const int* doc_start = nullptr;
  int window = 0;
  const int* blk_ptr = nullptr;
  const int* blk_idx = nullptr;
  int nnz = 0;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&BH,
                  (void*)&N, (void*)&n_mtiles, (void*)&c, (void*)&xcd_groups, (void*)&H,
                  (void*)&doc_start, (void*)&window, (void*)&blk_ptr, (void*)&blk_idx,
                  (void*)&nnz, (void*)&pairs};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
}

hipError_t launch_attn_fwd_local(Elem elem, const void* q, const void* k, const void* v, void* o,
                                 float* lse, const int* doc_start, int window, int B, int H, int N,
                                 int d, float scale, hipStream_t stream) {
  int threads, rows_per_block;
  const void* fn = pick_attn(elem, d, true, &threads, &rows_per_block, kMaskLocal);
  int BH = B * H;
  int n_mtiles = (N + rows_per_block - 1) / rows_per_block;
  float c = scale * kLog2e;
  const int grid = BH * n_mtiles;
  int xcd_groups = (BH % 8 == 0) ? 1 : 0;
  const int* blk_ptr = nullptr;
  const int* blk_idx = nullptr;
  int nnz = 0;
  int pairs = 0;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&BH,
                  (void*)&N, (void*)&n_mtiles, (void*)&c, (void*)&xcd_groups, (void*)&H,
                  (void*)&doc_start, (void*)&window, (void*)&blk_ptr, (void*)&blk_idx,
                  (void*)&nnz, (void*)&pairs};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
}

hipError_t launch_attn_fwd_blocksparse(Elem elem, const void* q, const void* k, const void* v,
                                       void* o, float* lse, const int* blk_ptr,
                                       const int* blk_idx, int nnz, int B, int H, int N, int d,
                                       float scale, bool causal, hipStream_t stream) {
  int threads, rows_per_block;
  const void* fn = pick_attn(elem, d, causal, &threads, &rows_per_block, kMaskSparse);
  int BH = B * H;
  int n_mtiles = (N + rows_per_block - 1) / rows_per_block;
  float c = scale * kLog2e;
  const int grid = BH * n_mtiles;
  int xcd_groups = (BH % 8 == 0) ? 1 : 0;
  const int* doc_start = nullptr;
  int window = 0;
  int pairs = 0;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse, (void*)&BH,
                  (void*)&N, (void*)&n_mtiles, (void*)&c, (void*)&xcd_groups, (void*)&H,
                  (void*)&doc_start, (void*)&window, (void*)&blk_ptr, (void*)&blk_idx,
                  (void*)&nnz, (void*)&pairs};
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
}

hipError_t attn_fwd_attributes(Elem elem, int d, bool causal, hipFuncAttributes* attr,
                               int* threads, int* blocks_per_cu, int mask) {
  int rows_per_block;
  const void* fn = pick_attn(elem, d, causal, threads, &rows_per_block, mask);
  hipError_t e = hipFuncGetAttributes(attr, fn);
  if (e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, fn, *threads, 0);
}

}  // namespace osm
