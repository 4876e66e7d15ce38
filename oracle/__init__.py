"""fp64 CPU oracle for attention forward and backward and row softmax (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline may import this package; the product path never does.  It shares no
code with the HIP library.

Inputs arrive in their storage type (float32, float16, or bfloat16 bit
patterns held in ``np.uint16``) and are widened exactly to float64 here, by
this package's own decoder.  Every result is float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, IEEE double throughout)."""
    tmp = f"{out}.{os.getpid()}.tmp"  # one per process: parallel test workers build at once
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", src, "-o", tmp, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


class Oracle:
    """Bound view of one compiled oracle library (the real one, or a test build)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lp = ctypes.POINTER(ctypes.c_long)
        L, I, D = ctypes.c_long, ctypes.c_int, ctypes.c_double
        lib.oracle_softmax_rows.argtypes = [dp, dp, L, L, I]
        lib.oracle_softmax_rows.restype = None
        lib.oracle_attention_rows.argtypes = [dp, dp, dp, L, L, D, I, lp, L, dp, dp, I]
        lib.oracle_attention_rows.restype = None
        lib.oracle_attention_ranged.argtypes = [dp, dp, dp, L, L, D, lp, lp, lp, L, dp, dp, I]
        lib.oracle_attention_ranged.restype = None
        lib.oracle_attention_keyset.argtypes = [dp, dp, dp, L, D, lp, lp, lp, L, L, dp, dp, I]
        lib.oracle_attention_keyset.restype = None
        lib.oracle_attention_probs.argtypes = [dp, dp, L, L, D, I, L, dp]
        lib.oracle_attention_probs.restype = None
        lib.oracle_online_normaliser.argtypes = [dp, L, dp, dp]
        lib.oracle_online_normaliser.restype = None
        lib.oracle_attention_tiled_row.argtypes = [dp, dp, dp, L, L, D, I, L, L, dp, dp, dp]
        lib.oracle_attention_tiled_row.restype = L
        lib.oracle_attention_backward.argtypes = [dp, dp, dp, dp, dp, L, L, D, I, dp, dp, dp, dp, dp,
                                                  dp, dp, dp, I]
        lib.oracle_attention_backward.restype = None
        self.lib = lib
        self.path = path

    # -- decoding of the storage types -------------------------------------
    @staticmethod
    def to_f64(x: np.ndarray, dtype: str | None = None) -> np.ndarray:
        """Exact widening to float64.  ``dtype='bf16'`` marks uint16 bit patterns,
        ``dtype='fp8'`` uint8 codes of the OCP fp8 E4M3 format (sign, 4-bit exponent
        with bias 7, 3-bit mantissa; exponent 0 is subnormal, m/8 * 2^-6; codes
        0x7F and 0xFF are NaN; no infinities)."""
        x = np.asarray(x)
        if dtype == "fp8":
            if x.dtype != np.uint8:
                raise TypeError("fp8 data must be np.uint8 codes")
            u = x.astype(np.int64)
            sign = np.where(u & 0x80, -1.0, 1.0)
            e, m = (u >> 3) & 0xF, u & 0x7
            mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                           np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
            mag = np.where((e == 15) & (m == 7), np.nan, mag)
            return np.ascontiguousarray(sign * mag, dtype=np.float64)
        if dtype == "bf16" or (dtype is None and x.dtype == np.uint16):
            if x.dtype != np.uint16:
                raise TypeError("bf16 data must be np.uint16 bit patterns")
            widened = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
            return np.ascontiguousarray(widened, dtype=np.float64)
        return np.ascontiguousarray(x, dtype=np.float64)

    @staticmethod
    def _p(a: np.ndarray):
        return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))

    # -- row softmax ---------------------------------------------------------
    def softmax_rows(self, x, threads: int | None = None) -> np.ndarray:
        x = self.to_f64(x)
        if x.ndim != 2:
            raise ValueError("softmax_rows expects [rows, cols]")
        y = np.empty_like(x)
        self.lib.oracle_softmax_rows(self._p(x), self._p(y), x.shape[0], x.shape[1],
                                     threads or default_threads())
        return y

    # -- attention, one head ---------------------------------------------------
    def attention_head(self, q, k, v, scale: float, causal: bool, rows=None,
                       dtype: str | None = None, threads: int | None = None):
        """O [len(rows), d] and LSE [len(rows)] of one head; q, k, v are [N, d]."""
        q, k, v = (self.to_f64(t, dtype) for t in (q, k, v))
        n, d = q.shape
        if k.shape != (n, d) or v.shape != (n, d):
            raise ValueError("q, k, v must share the shape [N, d]")
        rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= n):
            raise ValueError("row index out of range")
        o = np.empty((rows.size, d), np.float64)
        lse = np.empty(rows.size, np.float64)
        self.lib.oracle_attention_rows(self._p(q), self._p(k), self._p(v), n, d, float(scale),
                                       int(bool(causal)),
                                       rows.ctypes.data_as(ctypes.POINTER(ctypes.c_long)),
                                       rows.size, self._p(o), self._p(lse),
                                       threads or default_threads())
        return o, lse

    def attention_ranged(self, q, k, v, scale: float, lo, hi, rows=None, dtype: str | None = None,
                         threads: int | None = None):
        """O and LSE of one head where query i sees keys lo[i] .. hi[i] (inclusive)."""
        q, k, v = (self.to_f64(t, dtype) for t in (q, k, v))
        n, d = q.shape
        lo = np.ascontiguousarray(lo, dtype=np.int64)
        hi = np.ascontiguousarray(hi, dtype=np.int64)
        if lo.shape != (n,) or hi.shape != (n,) or np.any(lo < 0) or np.any(hi >= n) or np.any(lo > hi):
            raise ValueError("need 0 <= lo[i] <= hi[i] < N for every query")
        rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        o = np.empty((rows.size, d), np.float64)
        lse = np.empty(rows.size, np.float64)
        lp = ctypes.POINTER(ctypes.c_long)
        self.lib.oracle_attention_ranged(self._p(q), self._p(k), self._p(v), n, d, float(scale),
                                         lo.ctypes.data_as(lp), hi.ctypes.data_as(lp),
                                         rows.ctypes.data_as(lp), rows.size, self._p(o),
                                         self._p(lse), threads or default_threads())
        return o, lse

    def attention_keyset(self, q, k, v, scale: float, keysets, rows=None,
                         dtype: str | None = None, threads: int | None = None):
        """O [len(rows), d] and LSE of one head where query rows[r] sees exactly the keys
        keysets[r] (an index array; empty: O = 0, LSE = -inf)."""
        q, k, v = (self.to_f64(t, dtype) for t in (q, k, v))
        n, d = q.shape
        rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        if len(keysets) != rows.size:
            raise ValueError("one key set per row")
        sizes = np.array([len(ks) for ks in keysets], dtype=np.int64)
        ptr = np.zeros(rows.size + 1, np.int64)
        np.cumsum(sizes, out=ptr[1:])
        keys = (np.concatenate([np.asarray(ks, np.int64) for ks in keysets]) if rows.size
                else np.zeros(0, np.int64))
        if keys.size and (keys.min() < 0 or keys.max() >= k.shape[0]):
            raise ValueError("key index out of range")
        keys = np.ascontiguousarray(keys if keys.size else np.zeros(1, np.int64))
        o = np.empty((rows.size, d), np.float64)
        lse = np.empty(rows.size, np.float64)
        lp = ctypes.POINTER(ctypes.c_long)
        self.lib.oracle_attention_keyset(self._p(q), self._p(k), self._p(v), d, float(scale),
                                         ptr.ctypes.data_as(lp), keys.ctypes.data_as(lp),
                                         rows.ctypes.data_as(lp), rows.size,
                                         int(sizes.max()) if sizes.size else 1,
                                         self._p(o), self._p(lse), threads or default_threads())
        return o, lse

    @staticmethod
    def block_sparse_keys(n, i, blk_ptr, blk_idx, qblock, kblock, causal):
        """The keys query i sees under a block-sparse pattern: every key of the key
        blocks listed for its query block (i // qblock) in CSR form (blk_ptr, blk_idx),
        cut at n, and only keys j <= i when causal."""
        qb = i // qblock
        blocks = np.asarray(blk_idx[blk_ptr[qb]:blk_ptr[qb + 1]], np.int64)
        keys = [np.arange(b * kblock, min(n, (b + 1) * kblock)) for b in blocks]
        keys = np.concatenate(keys) if keys else np.zeros(0, np.int64)
        return keys[keys <= i] if causal else keys

    def attention_blocksparse(self, q, k, v, scale: float, causal: bool, blk_ptr, blk_idx,
                              qblock: int, kblock: int, rows=None, dtype: str | None = None,
                              threads: int | None = None):
        """O and LSE of one head under a block-sparse pattern (see block_sparse_keys)."""
        n = q.shape[0]
        rows = np.arange(n, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
        sets = [self.block_sparse_keys(n, int(i), blk_ptr, blk_idx, qblock, kblock, causal)
                for i in rows]
        return self.attention_keyset(q, k, v, scale, sets, rows, dtype=dtype, threads=threads)

    def attention_decode(self, q, k, v, scale: float, causal: bool, dtype: str | None = None,
                         threads: int | None = None):
        """O [Nq, d] and LSE [Nq] of Nq queries against Nk keys, q [Nq, d], k and v [Nk, d].

        The queries are the last Nq positions of the key sequence (decode and
        chunked prefill: query i sits at position Nk - Nq + i); causal lets it
        see keys 0 .. Nk - Nq + i (the causal rule of "Online Softmax: Tiling
        Across a Reduction"), otherwise every key.  Written as the key-range
        oracle over sequences padded to n = max(Nq, Nk) rows: the queries take
        the last Nq rows, padded keys lie outside every range.
        """
        q, k, v = (self.to_f64(t, dtype) for t in (q, k, v))
        nq, d = q.shape
        nk = k.shape[0]
        if k.shape != (nk, d) or v.shape != (nk, d) or nq < 1 or nk < 1:
            raise ValueError("q [Nq, d], k and v [Nk, d] with Nq, Nk >= 1")
        if causal and nq > nk:
            raise ValueError("causal needs Nq <= Nk")
        n = max(nq, nk)
        rows = np.arange(n - nq, n, dtype=np.int64)
        qf = np.zeros((n, d))
        qf[rows] = q
        kf, vf = np.zeros((n, d)), np.zeros((n, d))
        kf[:nk], vf[:nk] = k, v
        lo = np.zeros(n, np.int64)
        hi = np.full(n, nk - 1, np.int64)
        if causal:
            hi[rows] = nk - nq + np.arange(nq)
        return self.attention_ranged(qf, kf, vf, scale, lo, hi, rows, threads=threads)

    def attention(self, q, k, v, scale: float, causal: bool, rows_of=None,
                  dtype: str | None = None, threads: int | None = None):
        """[B, H, N, d] inputs; ``rows_of(b, h)`` picks the checked rows (default all).

        Returns a list over heads of (b, h, rows, O [rows, d], LSE [rows]).
        """
        B, H, N, _ = q.shape
        out = []
        for b in range(B):
            for h in range(H):
                rows = None if rows_of is None else rows_of(b, h)
                o, lse = self.attention_head(q[b, h], k[b, h], v[b, h], scale, causal, rows,
                                             dtype, threads)
                rr = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
                out.append((b, h, rr, o, lse))
        return out

    def attention_probs(self, q, k, scale: float, causal: bool, i: int, dtype=None) -> np.ndarray:
        q, k = self.to_f64(q, dtype), self.to_f64(k, dtype)
        n, d = q.shape
        p = np.empty(n, np.float64)
        self.lib.oracle_attention_probs(self._p(q), self._p(k), n, d, float(scale),
                                        int(bool(causal)), int(i), self._p(p))
        return p

    def attention_backward_head(self, q, k, v, dout, scale: float, causal: bool,
                                dtype: str | None = None, threads: int | None = None, o=None,
                                magnitudes: bool = False):
        """Gradients of one head: (dQ, dK, dV) [N, d] each, plus the row statistic
        lse [N] and D [N] (D_i = sum_j P_ij dP_ij) that the recomputation uses.
        With ``o`` (the forward output as a caller stores it), D_i = <dO_i, o_i>.
        With ``magnitudes``, three more [N, d] arrays follow: the sums of the
        absolute values of the terms of dQ, dK and dV."""
        q, k, v, dout = (self.to_f64(t, dtype) for t in (q, k, v, dout))
        o = None if o is None else self.to_f64(o, dtype)
        n, d = q.shape
        if k.shape != (n, d) or v.shape != (n, d) or dout.shape != (n, d) or (
                o is not None and o.shape != (n, d)):
            raise ValueError("q, k, v, dout (and o) must share the shape [N, d]")
        dq, dk, dv = (np.empty((n, d), np.float64) for _ in range(3))
        lse, dd = np.empty(n, np.float64), np.empty(n, np.float64)
        mags = [np.empty((n, d), np.float64) for _ in range(3)] if magnitudes else [None] * 3
        self.lib.oracle_attention_backward(self._p(q), self._p(k), self._p(v), self._p(dout),
                                           None if o is None else self._p(o), n, d,
                                           float(scale), int(bool(causal)), self._p(dq),
                                           self._p(dk), self._p(dv), self._p(lse), self._p(dd),
                                           *(None if m is None else self._p(m) for m in mags),
                                           threads or default_threads())
        if magnitudes:
            return (dq, dk, dv, lse, dd, *mags)
        return dq, dk, dv, lse, dd

    # -- online forms ----------------------------------------------------------
    def online_normaliser(self, x) -> tuple[float, float]:
        x = self.to_f64(np.ravel(x))
        m = ctypes.c_double()
        s = ctypes.c_double()
        self.lib.oracle_online_normaliser(self._p(x), x.size, ctypes.byref(m), ctypes.byref(s))
        return m.value, s.value

    def attention_tiled_row(self, q, k, v, scale: float, causal: bool, i: int, tile: int,
                            dtype=None):
        """(o [d], lse, alphas [tiles]) of the tile-wise recurrence for query row i."""
        q, k, v = (self.to_f64(t, dtype) for t in (q, k, v))
        n, d = q.shape
        o = np.empty(d, np.float64)
        lse = ctypes.c_double()
        alphas = np.empty(max(1, (n + tile - 1) // tile), np.float64)
        t = self.lib.oracle_attention_tiled_row(self._p(q), self._p(k), self._p(v), n, d,
                                                float(scale), int(bool(causal)), int(i),
                                                int(tile), self._p(o), ctypes.byref(lse),
                                                self._p(alphas))
        return o, lse.value, alphas[:t].copy()


def load(path: str = LIB) -> Oracle:
    """The oracle library, compiled on first use if absent or older than its source."""
    global _lib
    if path == LIB:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = Oracle(LIB)
        return _lib
    return Oracle(path)
