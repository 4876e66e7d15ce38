"""Seeded synthetic inputs for the attention-forward and row-softmax workloads.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no scores, no exponentials, no normalisation), so both the
fp64 oracle and the HIP path can consume what it produces without sharing any
of the computation being checked.

Storage conventions
-------------------
* ``"f32"`` tensors are ``np.float32``.
* ``"f16"`` tensors are ``np.float16`` (numpy's cast rounds to nearest even).
* ``"bf16"`` tensors are ``np.uint16`` arrays holding bfloat16 bit patterns,
  produced from float32 draws by round-to-nearest-even.
* Attention tensors are row-major ``[B, H, N, d]``.

Workloads (sizes and value recipes of the pages' examples):
* ``attn_f32_n256``      -- one head, N=256, d=64, fp32, non-causal, scale 1/8.
* ``attn_f32_n256_last`` -- the same shape with the largest score of every
  query row placed in the final 64-key tile and Q multiplied by 10, so the
  running maximum still moves on the last tile ("Day 97", the loud key N-3).
* ``softmax_4096x32768`` -- row softmax input, fp32, N(0,1) with about 1% of
  entries set to +50.
* ``attn_bf16_n4096``    -- one head, N=4096, d=64, bf16, non-causal.
* ``attn_bf16_b8h32n8192_causal`` -- B=8, H=32, N=8192, d=128, bf16, causal,
  every K row scaled by a U(0.5, 2) factor.
* ``attn_bf16_n131072_causal`` -- one head, N=131072, d=64, bf16, causal.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 97000

__all__ = [
    "AttnWorkload", "SoftmaxWorkload", "DecodeWorkload", "ATTN", "SOFTMAX", "DECODE",
    "decode_head", "decode_full",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "f32_to_e4m3", "cast", "attn_head", "attn_full",
    "attn_sample_rows", "softmax_input", "random_attn", "random_rows",
]


# --------------------------------------------------------------------------
# bit-level storage helpers (no arithmetic of the method)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 rounding helper expects finite inputs")
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _e4m3_table() -> np.ndarray:
    """The 127 non-negative finite values of the OCP fp8 E4M3 format, in code order
    0x00 .. 0x7E (code 0x7F is NaN; there is no infinity): exponent field e (4 bits,
    bias 7) and mantissa field m (3 bits) give m/8 * 2^-6 for e = 0 and
    (1 + m/8) * 2^(e - 7) otherwise."""
    codes = np.arange(127)
    e, m = codes >> 3, codes & 7
    return np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))


_E4M3 = _e4m3_table()


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP fp8 E4M3 codes (nearest, ties to the even code),
    saturating at +-448; returns np.uint8 codes."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("fp8 rounding helper expects finite inputs")
    a = np.minimum(np.abs(x), _E4M3[-1])
    hi = np.clip(np.searchsorted(_E4M3, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - _E4M3[lo], _E4M3[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where((x < 0) & (code != 0), code | np.uint8(0x80), code).astype(np.uint8)


def cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Store float32 draws in the workload's element type."""
    if dtype == "fp8":
        return f32_to_e4m3(x32)
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return np.ascontiguousarray(x32.astype(np.float16))
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


# --------------------------------------------------------------------------
# workload descriptions
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str
    causal: bool
    seed: int
    k_row_scale: tuple | None = None      # (lo, hi) of a per-key-row U(lo, hi) factor
    descales: tuple | None = None         # fp8: (q, k, v) value = descale * stored code
    last_tile_max: bool = False           # loud key N-3 + Q x 10
    sampled_rows: int | None = None       # rows checked per head (None = all)
    scale: float = field(default=0.0)

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """4*N^2*d per head (QK^T and PV, 2 flops per MAC), halved when causal."""
        f = 4.0 * self.N * self.N * self.d * self.B * self.H
        return f / 2.0 if self.causal else f


@dataclass(frozen=True)
class SoftmaxWorkload:
    name: str
    rows: int
    cols: int
    seed: int
    spike_prob: float = 0.01
    spike_value: float = 50.0

    @property
    def algorithmic_bytes(self) -> int:
        """One read of X and one write of Y, fp32."""
        return 8 * self.rows * self.cols


ATTN = {
    w.name: w for w in [
        AttnWorkload("attn_f32_n256", 1, 1, 256, 64, "f32", False, BASE_SEED + 1),
        AttnWorkload("attn_f32_n256_last", 1, 1, 256, 64, "f32", False, BASE_SEED + 11,
                     last_tile_max=True),
        AttnWorkload("attn_bf16_n4096", 1, 1, 4096, 64, "bf16", False, BASE_SEED + 3),
        AttnWorkload("attn_bf16_b8h32n8192_causal", 8, 32, 8192, 128, "bf16", True,
                     BASE_SEED + 4, k_row_scale=(0.5, 2.0), sampled_rows=256),
        AttnWorkload("attn_bf16_n131072_causal", 1, 1, 131072, 64, "bf16", True,
                     BASE_SEED + 5, sampled_rows=256),
        # the B8 H32 N8192 d128 causal recipe stored in fp8 E4M3 with per-tensor
        # descales that keep the draws inside +-448 (|N(0,1)| < 7 x 64, K x 2 < 14 x 32)
        AttnWorkload("attn_fp8_b8h32n8192_causal", 8, 32, 8192, 128, "fp8", True,
                     BASE_SEED + 8, k_row_scale=(0.5, 2.0), sampled_rows=256,
                     descales=(1.0 / 64, 1.0 / 32, 1.0 / 64)),
    ]
}

SOFTMAX = {
    w.name: w for w in [
        SoftmaxWorkload("softmax_4096x32768", 4096, 32768, BASE_SEED + 2),
        # few very long rows (one row per sequence of a batch of 4, 16M positions
        # each); rarer spikes so that each spike carries a visible share (~1/170)
        SoftmaxWorkload("softmax_split_4x16777216", 4, 1 << 24, BASE_SEED + 6, spike_prob=1e-5),
    ]
}


# --------------------------------------------------------------------------
# attention inputs
# --------------------------------------------------------------------------
def _head_f32(w: AttnWorkload, b: int, h: int):
    """float32 draws of one head's Q, K, V before rounding to the storage type."""
    rng = np.random.default_rng([w.seed, b, h])
    q = rng.standard_normal((w.N, w.d), dtype=np.float32)
    k = rng.standard_normal((w.N, w.d), dtype=np.float32)
    v = rng.standard_normal((w.N, w.d), dtype=np.float32)
    if w.k_row_scale is not None:
        lo, hi = w.k_row_scale
        u = rng.uniform(lo, hi, size=(w.N, 1)).astype(np.float32)
        k = k * u
    if w.last_tile_max:
        # Every query gets a large positive first coordinate and key N-3 gets a
        # large first coordinate, so key N-3 (inside the last 64-key tile) is
        # each row's argmax by a wide margin; then Q is scaled by 10 so the
        # scores are O(100) and the final rescale factor is tiny.
        q[:, 0] = np.abs(q[:, 0]) + 1.0
        k[w.N - 3, 0] += 16.0 * math.sqrt(w.d)
        q = q * np.float32(10.0)
    return q, k, v


def attn_head(w: AttnWorkload, b: int = 0, h: int = 0):
    """One head's (q, k, v), each [N, d] in the workload's storage type (fp8: the
    draws divided by the tensor's descale, then rounded)."""
    q, k, v = _head_f32(w, b, h)
    if w.dtype == "fp8":
        sq, sk, sv = w.descales
        return cast(q / sq, "fp8"), cast(k / sk, "fp8"), cast(v / sv, "fp8")
    return cast(q, w.dtype), cast(k, w.dtype), cast(v, w.dtype)


def attn_full(w: AttnWorkload, threads: int = 8):
    """Full (q, k, v), each [B, H, N, d] in the storage type (heads drawn in parallel)."""
    dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "fp8": np.uint8}[w.dtype]
    shape = (w.B, w.H, w.N, w.d)
    q = np.empty(shape, dt)
    k = np.empty(shape, dt)
    v = np.empty(shape, dt)

    def fill(bh):
        b, h = divmod(bh, w.H)
        q[b, h], k[b, h], v[b, h] = attn_head(w, b, h)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(w.B * w.H)))
    return q, k, v


def attn_sample_rows(w: AttnWorkload, b: int, h: int, count: int | None = None) -> np.ndarray:
    """Sorted distinct query rows checked for head (b, h).

    Always includes the tile and diagonal boundaries {0, 1, 63, 64, 127, 128, N-1}
    (those below N); the rest are drawn from a seeded stream of their own.
    """
    count = w.sampled_rows if count is None else count
    if count is None or count >= w.N:
        return np.arange(w.N, dtype=np.int64)
    fixed = {r for r in (0, 1, 63, 64, 127, 128, w.N - 1) if 0 <= r < w.N}
    rng = np.random.default_rng([w.seed, b, h, 7])
    rest = rng.choice(w.N, size=min(w.N, count + len(fixed)), replace=False)
    rows = list(fixed)
    for r in rest:
        if len(rows) >= count:
            break
        if int(r) not in fixed:
            rows.append(int(r))
    return np.array(sorted(rows), dtype=np.int64)


def packed_doc_starts(B: int, N: int, seed: int, min_len: int, max_len: int) -> np.ndarray:
    """[B, N] int32: for each position, the first position of its document, for rows
    packed with documents of seeded lengths uniform in [min_len, max_len] (the
    last one cut at N)."""
    rng = np.random.default_rng([BASE_SEED + 800, seed, B, N])
    out = np.empty((B, N), np.int32)
    for b in range(B):
        p = 0
        while p < N:
            ln = int(rng.integers(min_len, max_len + 1))
            out[b, p:p + ln] = p
            p += ln
    return out


# sliding-window / packed-document forward: the B8 H32 N8192 d128 causal shape with
# a 1024-key window over documents of 512 to 4096 tokens (K rows x U(0.5, 2) as the
# dense workload)
LOCAL_WORKLOAD = dict(name="attn_bf16_b8h32n8192_w1024_docs", base="attn_bf16_b8h32n8192_causal",
                      window=1024, doc_min=512, doc_max=4096, doc_seed=5)


def local_ranges(doc_start_row: np.ndarray, window: int) -> tuple[np.ndarray, np.ndarray]:
    """(lo, hi) of every query of one batch row: keys max(doc start, i - window + 1) .. i."""
    n = doc_start_row.shape[0]
    i = np.arange(n, dtype=np.int64)
    lo = doc_start_row.astype(np.int64)
    if window > 0:
        lo = np.maximum(lo, i - window + 1)
    return np.clip(lo, 0, i), i


def block_sparse_pattern(N: int, seed: int, qblock: int = 256, kblock: int = 128,
                         band: int = 2, sinks: int = 1, p_random: float = 0.1,
                         causal: bool = True) -> tuple[np.ndarray, np.ndarray]:
    """(blk_ptr, blk_idx) int32 CSR over ceil(N / qblock) query blocks: for each
    query block, ascending distinct key-block indices of the first `sinks` key
    blocks, the `band` key blocks ending at the block holding the query block's
    last row together with every key block overlapping the query block, and each
    other key block with probability p_random; with causal, only key blocks that
    start at or before the query block's last row are drawn."""
    rng = np.random.default_rng([BASE_SEED + 900, seed, N, qblock, kblock])
    nqb = (N + qblock - 1) // qblock
    nkb = (N + kblock - 1) // kblock
    ptr = [0]
    idx: list[int] = []
    for qb in range(nqb):
        first_row = qb * qblock
        last_row = min(N, first_row + qblock) - 1
        top = last_row // kblock if causal else nkb - 1   # last key block drawn from
        chosen = set(range(min(sinks, top + 1)))
        diag_hi = last_row // kblock
        chosen.update(range(max(0, min(first_row // kblock, diag_hi - band + 1)), diag_hi + 1))
        if not causal:
            chosen.update(range(first_row // kblock, diag_hi + 1))
        draws = rng.random(nkb) < p_random
        chosen.update(int(b) for b in np.nonzero(draws[:top + 1])[0])
        blocks = sorted(b for b in chosen if 0 <= b < nkb and b <= top)
        idx.extend(blocks)
        ptr.append(len(idx))
    return np.asarray(ptr, np.int32), np.asarray(idx, np.int32)


def block_sparse_pairs(N: int, blk_ptr: np.ndarray, blk_idx: np.ndarray, causal: bool,
                       qblock: int = 256, kblock: int = 128) -> int:
    """Number of (query, key) pairs a pattern lets through (per head), counting
    keys j < N and, with causal, j <= i."""
    total = 0
    for qb in range(len(blk_ptr) - 1):
        r0, r1 = qb * qblock, min(N, (qb + 1) * qblock)
        for b in blk_idx[blk_ptr[qb]:blk_ptr[qb + 1]]:
            j0, j1 = int(b) * kblock, min(N, (int(b) + 1) * kblock)
            if not causal:
                total += (r1 - r0) * (j1 - j0)
                continue
            for i in range(r0, r1):
                total += max(0, min(j1, i + 1) - j0)
    return total


# block-sparse forward: the B8 H32 N8192 d128 causal shape under a pattern of one
# sink block, a two-block band at the diagonal and 10 % random blocks (K rows x
# U(0.5, 2) as the dense workload)
BLOCKSPARSE_WORKLOAD = dict(name="attn_bf16_b8h32n8192_blocksparse", base="attn_bf16_b8h32n8192_causal",
                            band=2, sinks=1, p_random=0.1, pattern_seed=7)


# --------------------------------------------------------------------------
# decode-shaped attention: Nq queries at the end of Nk cached keys
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str
    causal: bool
    seed: int
    k_row_scale: tuple | None = (0.5, 2.0)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def kv_bytes(self) -> int:
        """K and V read once: the algorithmic bytes that dominate (Q and O are Nq / Nk of them)."""
        return 2 * self.B * self.H * self.Nk * self.d * 2

    @property
    def algorithmic_bytes(self) -> int:
        """K and V read once, Q read once, O written once (16-bit), LSE written once (fp32)."""
        return self.kv_bytes + 2 * self.B * self.H * self.Nq * self.d * 2 + 4 * self.B * self.H * self.Nq


# one new token per sequence against a 32768-token cache: the B8 H32 d128 shape of
# the dense workload, N(0, 1) entries with K rows x U(0.5, 2)
DECODE = {
    w.name: w for w in [
        DecodeWorkload("decode_bf16_b8h32_q1_kv32768_d128", 8, 32, 1, 32768, 128, "bf16", True,
                       BASE_SEED + 7),
    ]
}


def decode_head(w: DecodeWorkload, b: int, h: int):
    """One head's (q [Nq, d], k [Nk, d], v [Nk, d]) in the storage type."""
    rng = np.random.default_rng([w.seed, b, h])
    q = rng.standard_normal((w.Nq, w.d), dtype=np.float32)
    k = rng.standard_normal((w.Nk, w.d), dtype=np.float32)
    v = rng.standard_normal((w.Nk, w.d), dtype=np.float32)
    if w.k_row_scale is not None:
        lo, hi = w.k_row_scale
        k = k * rng.uniform(lo, hi, size=(w.Nk, 1)).astype(np.float32)
    return cast(q, w.dtype), cast(k, w.dtype), cast(v, w.dtype)


def decode_full(w: DecodeWorkload, threads: int = 8):
    """Full (q [B, H, Nq, d], k and v [B, H, Nk, d]) in the storage type."""
    dt = {"f16": np.float16, "bf16": np.uint16}[w.dtype]
    q = np.empty((w.B, w.H, w.Nq, w.d), dt)
    k = np.empty((w.B, w.H, w.Nk, w.d), dt)
    v = np.empty((w.B, w.H, w.Nk, w.d), dt)

    def fill(bh):
        b, h = divmod(bh, w.H)
        q[b, h], k[b, h], v[b, h] = decode_head(w, b, h)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, range(w.B * w.H)))
    return q, k, v


# --------------------------------------------------------------------------
# softmax inputs
# --------------------------------------------------------------------------
def softmax_input(w: SoftmaxWorkload, rows: slice | None = None, threads: int = 8) -> np.ndarray:
    """X [rows, cols] fp32: N(0,1) with Bernoulli(spike_prob) entries set to spike_value.

    Each row is drawn from its own seeded stream, so any subset of rows can be
    regenerated alone.
    """
    r0, r1 = (0, w.rows) if rows is None else (rows.start or 0, rows.stop or w.rows)
    x = np.empty((r1 - r0, w.cols), np.float32)

    def fill(chunk):
        for r in chunk:
            rng = np.random.default_rng([w.seed, r])
            row = rng.standard_normal(w.cols, dtype=np.float32)
            mask = rng.random(w.cols) < w.spike_prob
            if not mask.any():            # the recipe asks for at least one spike per row
                mask[rng.integers(w.cols)] = True
            row[mask] = np.float32(w.spike_value)
            x[r - r0] = row

    idx = list(range(r0, r1))
    chunks = [idx[i::max(1, threads)] for i in range(max(1, threads))]
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, chunks))
    return x


# --------------------------------------------------------------------------
# small random cases for edge-case tests
# --------------------------------------------------------------------------
def random_attn(B, H, N, d, dtype, seed, std=1.0):
    """iid N(0, std^2) Q, K, V of shape [B, H, N, d] in the storage type."""
    rng = np.random.default_rng([BASE_SEED + 500, seed, B, H, N, d])
    shape = (B, H, N, d)
    out = []
    for _ in range(3):
        x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
        out.append(cast(x, dtype))
    return tuple(out)


def random_rows(rows, cols, seed, std=1.0, spike_prob=0.0, spike_value=50.0):
    """iid N(0, std^2) fp32 rows, optionally with spikes."""
    rng = np.random.default_rng([BASE_SEED + 600, seed, rows, cols])
    x = rng.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)
    if spike_prob > 0:
        x[rng.random((rows, cols)) < spike_prob] = np.float32(spike_value)
    return x
