"""Pins of the fp64 oracle to facts fixed outside itself.

Each ``pin_*`` function takes a bound oracle library and raises AssertionError
when the oracle disagrees with a fact that the pages or plain mathematics fix:
hand-derived closed forms (tests/golden/closed_forms.json), special cases,
invariants the pages state (online == three-pass, rows of P sum to one, the
rescale factor never exceeds one, the loud key in the last tile), and a
50-digit brute force on tiny inputs.  The same pins run against deliberately
broken copies of the oracle (test_oracle_mutants.py) to show they would catch
a dropped term, a wrong sign or index, or a transposed operand.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _rng(tag):
    return np.random.default_rng([4242, tag])


# ---------------------------------------------------------------------------
# softmax pins
# ---------------------------------------------------------------------------
def pin_softmax_golden(orc):
    """Hand-derived rows: exp ratios 1:2:3:4, the same shifted by 1000, three spikes."""
    cases = json.load(open(GOLDEN))["softmax"]
    for c in cases:
        y = orc.softmax_rows(np.array([c["x"]], np.float64))[0]
        _close(y, c["y"], c.get("tol", 1e-15), f"softmax golden {c['name']}")


def pin_softmax_constant_row(orc):
    """A row of equal values gives 1/cols everywhere."""
    for cols in (1, 2, 7, 64, 1000):
        x = np.full((3, cols), -3.25)
        _close(orc.softmax_rows(x), np.full((3, cols), 1.0 / cols), 1e-15, f"constant row {cols}")


def pin_softmax_two_element_logistic(orc):
    """softmax([a, b])_0 = 1 / (1 + e^(b - a)), the logistic function."""
    r = _rng(1)
    x = r.normal(0, 5, size=(50, 2))
    y = orc.softmax_rows(x)
    ref = 1.0 / (1.0 + np.exp(x[:, 1] - x[:, 0]))
    _close(y[:, 0], ref, 1e-14, "logistic")
    _close(y[:, 1], 1.0 - ref, 1e-14, "logistic complement")


def pin_softmax_spike_rows(orc):
    """k entries at +50 and the rest <= -1e3: exactly 1/k at the spikes, 0 elsewhere."""
    r = _rng(2)
    x = -1e3 - r.random((6, 300)) * 10
    ks = []
    for i in range(6):
        idx = r.choice(300, size=i + 1, replace=False)
        x[i, idx] = 50.0
        ks.append(idx)
    y = orc.softmax_rows(x)
    for i, idx in enumerate(ks):
        ref = np.zeros(300)
        ref[idx] = 1.0 / len(idx)
        _close(y[i], ref, 1e-15, f"spike row {i}")


def pin_softmax_shift_invariance(orc):
    """softmax(x + t) = softmax(x) for t = 700 (exp(700+) is beyond double range)."""
    x = _rng(3).normal(0, 3, size=(4, 257))
    _close(orc.softmax_rows(x + 700.0), orc.softmax_rows(x), 1e-13, "shift invariance")


def pin_softmax_brute_force(orc):
    """50-digit brute force exp(x_i)/sum exp(x_j) on tiny rows."""
    import mpmath
    mpmath.mp.dps = 50
    x = _rng(4).normal(0, 4, size=(5, 9))
    y = orc.softmax_rows(x)
    for i in range(x.shape[0]):
        e = [mpmath.exp(mpmath.mpf(float(t))) for t in x[i]]
        s = mpmath.fsum(e)
        ref = [float(t / s) for t in e]
        _close(y[i], ref, 1e-15, f"softmax brute force row {i}")


def pin_online_normaliser_equals_three_pass(orc):
    """The scalar recurrence (max, rescaled sum) reproduces the three-pass softmax."""
    r = _rng(5)
    for n in (1, 2, 17, 1000):
        x = r.normal(0, 6, size=n)
        if n > 3:
            x[-1] = x.max() + 20.0       # the maximum arrives last
        m, dsum = orc.online_normaliser(x)
        assert m == float(np.max(x)), "online max differs from the row max"
        y = orc.softmax_rows(x[None, :])[0]
        _close(np.exp(x - m) / dsum, y, 1e-14, f"online normaliser n={n}")


def pin_softmax_rows_sum_to_one(orc):
    """Rows of the spiked workload recipe are non-negative and sum to one."""
    x = workloads.random_rows(8, 4096, seed=6, spike_prob=0.01)
    y = orc.softmax_rows(x)
    assert np.all(y >= 0), "negative probability"
    _close(y.sum(axis=1), np.ones(8), 1e-13, "softmax row sums")


# ---------------------------------------------------------------------------
# attention pins
# ---------------------------------------------------------------------------
def pin_attention_golden(orc):
    """Hand-derived two-key cases (non-causal, causal, scaled)."""
    for c in json.load(open(GOLDEN))["attention"]:
        q, k, v = (np.array(c[t], np.float64) for t in "qkv")
        o, lse = orc.attention_head(q, k, v, c["scale"], c["causal"])
        _close(o, c["o"], 1e-14, f"attention golden {c['name']} O")
        _close(lse, c["lse"], 1e-14, f"attention golden {c['name']} LSE")


def pin_attention_brute_force(orc):
    """50-digit softmax(scale Q K^T) V on tiny non-square inputs, causal and not."""
    import mpmath
    mpmath.mp.dps = 50
    r = _rng(10)
    for n, d, causal in ((1, 3, False), (5, 3, False), (7, 2, True), (8, 4, True), (3, 5, False)):
        q, k, v = (r.normal(0, 1.5, size=(n, d)) for _ in range(3))
        scale = 0.7
        o, lse = orc.attention_head(q, k, v, scale, causal)
        for i in range(n):
            js = range(i + 1) if causal else range(n)
            s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(q[i, e])) * mpmath.mpf(float(k[j, e]))
                                                 for e in range(d)) for j in js]
            w = [mpmath.exp(t) for t in s]
            z = mpmath.fsum(w)
            ref = [float(mpmath.fsum(w[t] * mpmath.mpf(float(v[j, e])) for t, j in enumerate(js)) / z)
                   for e in range(d)]
            _close(o[i], ref, 1e-14, f"attention brute force n={n} d={d} causal={causal} row {i}")
            _close([lse[i]], [float(mpmath.log(z))], 1e-14, f"lse brute force row {i}")


def pin_attention_zero_query(orc):
    """Q = 0: every visible key gets the same weight, so o_i is the mean of the
    visible v_j and lse_i = ln(number of visible keys)."""
    r = _rng(11)
    n, d = 37, 8
    k, v = r.normal(size=(n, d)), r.normal(size=(n, d))
    q = np.zeros((n, d))
    for causal in (False, True):
        o, lse = orc.attention_head(q, k, v, 0.3, causal)
        for i in range(n):
            cnt = i + 1 if causal else n
            _close(o[i], v[:cnt].mean(axis=0), 1e-14, f"zero-q mean causal={causal} row {i}")
            _close([lse[i]], [math.log(cnt)], 1e-14, f"zero-q lse row {i}")


def pin_attention_constant_values(orc):
    """V rows all equal to c: o_i = c whatever the weights."""
    r = _rng(12)
    n, d = 29, 6
    q, k = r.normal(0, 2, size=(n, d)), r.normal(0, 2, size=(n, d))
    c = r.normal(size=d)
    v = np.tile(c, (n, 1))
    for causal in (False, True):
        o, _ = orc.attention_head(q, k, v, 0.5, causal)
        _close(o, np.tile(c, (n, 1)), 1e-13, f"constant V causal={causal}")


def pin_attention_causal_first_row(orc):
    """Causal row 0 sees key 0 only: o_0 = v_0 and lse_0 = scale <q_0, k_0>."""
    r = _rng(13)
    n, d = 16, 5
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    o, lse = orc.attention_head(q, k, v, 0.9, True, rows=[0])
    _close(o[0], v[0], 1e-15, "causal row 0 O")
    _close([lse[0]], [0.9 * float(np.dot(q[0], k[0]))], 1e-14, "causal row 0 LSE")


def pin_attention_key_permutation(orc):
    """Non-causal: permuting K and V rows together leaves O and LSE unchanged."""
    r = _rng(14)
    n, d = 40, 7
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    perm = r.permutation(n)
    o1, l1 = orc.attention_head(q, k, v, 0.4, False)
    o2, l2 = orc.attention_head(q, k[perm], v[perm], 0.4, False)
    _close(o1, o2, 1e-14, "key permutation O")
    _close(l1, l2, 1e-14, "key permutation LSE")


def pin_attention_scale_moves_between_operands(orc):
    """softmax(s Q K^T) = softmax((s/2)(2Q) K^T), and LSE matches too."""
    r = _rng(15)
    n, d = 24, 4
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    o1, l1 = orc.attention_head(q, k, v, 0.8, True)
    o2, l2 = orc.attention_head(2 * q, k, v, 0.4, True)
    o3, l3 = orc.attention_head(q, k, v, 0.4, True)
    _close(o1, o2, 1e-14, "scale O")
    _close(l1, l2, 1e-14, "scale LSE")
    assert np.max(np.abs(o1 - o3)) > 1e-3, "output does not depend on the scale"


def pin_attention_probs(orc):
    """Rows of P are non-negative, sum to one, vanish on hidden keys, and their
    ratios are p_j / p_k = exp(s_j - s_k) (I2 and the definition of softmax)."""
    r = _rng(16)
    n, d = 33, 8
    q, k = r.normal(size=(n, d)), r.normal(size=(n, d))
    for causal in (False, True):
        for i in (0, 5, n - 1):
            p = orc.attention_probs(q, k, 0.35, causal, i)
            vis = i + 1 if causal else n
            assert np.all(p >= 0), "negative probability"
            assert np.all(p[vis:] == 0), "hidden key has weight"
            _close([p.sum()], [1.0], 1e-14, "P row sum")
            s = 0.35 * (k[:vis] @ q[i])
            _close(np.log(p[:vis] / p[0]), s - s[0], 1e-12, "P log-ratios")


def pin_attention_matches_probs_times_v(orc):
    """O = P V with P from the probability routine (a second path through the definition)."""
    r = _rng(17)
    n, d = 21, 6
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    for causal in (False, True):
        o, _ = orc.attention_head(q, k, v, 0.6, causal)
        P = np.stack([orc.attention_probs(q, k, 0.6, causal, i) for i in range(n)])
        _close(o, P @ v, 1e-14, f"O = P V causal={causal}")


def pin_tiled_recurrence_equals_definition(orc):
    """The per-tile (m, l, O) recurrence equals the three-pass result for any tile
    size (exact in exact arithmetic; reassociation only in double)."""
    r = _rng(18)
    n, d = 150, 16
    q, k, v = (r.normal(0, 1.5, size=(n, d)) for _ in range(3))
    for causal in (False, True):
        o_ref, lse_ref = orc.attention_head(q, k, v, 0.25, causal)
        for tile in (1, 7, 64, n):
            for i in (0, 1, 63, 64, 100, n - 1):
                o, lse, alphas = orc.attention_tiled_row(q, k, v, 0.25, causal, i, tile)
                _close(o, o_ref[i], 1e-12, f"tiled O tile={tile} row={i} causal={causal}")
                _close([lse], [lse_ref[i]], 1e-12, f"tiled LSE tile={tile} row={i}")
                vis = i + 1 if causal else n
                assert len(alphas) == -(-vis // tile), "wrong number of tiles visited"


def pin_rescale_factors(orc):
    """Every rescale factor lies in [0, 1]; the first one is exactly 0 (m starts at
    -inf); a factor equals 1 exactly when the running max did not move."""
    r = _rng(19)
    n, d = 200, 8
    q, k, v = (r.normal(0, 2, size=(n, d)) for _ in range(3))
    tile = 16
    for i in (3, 77, 199):
        _, _, alphas = orc.attention_tiled_row(q, k, v, 0.5, False, i, tile)
        assert alphas[0] == 0.0, "first rescale factor is not 0"
        assert np.all((alphas >= 0) & (alphas <= 1)), "rescale factor outside [0, 1]"
        s = 0.5 * (k @ q[i])
        run = np.maximum.accumulate([s[j:j + tile].max() for j in range(0, n, tile)])
        moved = np.r_[True, run[1:] > run[:-1]]
        assert np.array_equal(alphas == 1.0, ~moved), "alpha == 1 does not track a still max"


def pin_last_tile_case(orc):
    """The loud-key workload: every row's largest score lies in the last 64-key
    tile, and the tile-wise run still rescales (alpha < 1) on that last tile."""
    w = workloads.ATTN["attn_f32_n256_last"]
    q, k, v = workloads.attn_head(w)
    o_ref, _ = orc.attention_head(q, k, v, w.sm_scale, w.causal)
    n = w.N
    for i in range(0, n, 5):
        p = orc.attention_probs(q, k, w.sm_scale, w.causal, i)
        assert int(np.argmax(p)) >= n - 64, f"row {i}: argmax not in the last tile"
        o, _, alphas = orc.attention_tiled_row(q, k, v, w.sm_scale, w.causal, i, 64)
        assert alphas[-1] < 1.0, f"row {i}: no rescale on the last tile"
        _close(o, o_ref[i], 1e-12, f"last-tile tiled row {i}")


# ---------------------------------------------------------------------------
# key-range (structured mask) pins
# ---------------------------------------------------------------------------
def pin_ranged_full_ranges_are_causal_and_dense(orc):
    """lo = 0, hi = i is the causal rule; lo = 0, hi = N - 1 is no mask."""
    r = _rng(40)
    n, d = 37, 6
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    for causal, hi in ((True, np.arange(n)), (False, np.full(n, n - 1))):
        o1, l1 = orc.attention_ranged(q, k, v, 0.45, np.zeros(n, np.int64), hi)
        o2, l2 = orc.attention_head(q, k, v, 0.45, causal)
        _close(o1, o2, 1e-14, f"full range O causal={causal}")
        _close(l1, l2, 1e-14, f"full range LSE causal={causal}")


def pin_ranged_window_is_a_slice(orc):
    """A window of keys lo..hi is plain attention of q_i over the sliced K and V."""
    r = _rng(41)
    n, d = 40, 5
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    w = 7
    lo = np.maximum(0, np.arange(n) - w + 1)
    hi = np.arange(n)
    o, lse = orc.attention_ranged(q, k, v, 0.6, lo, hi)
    for i in range(n):
        ks, vs = k[lo[i]:hi[i] + 1], v[lo[i]:hi[i] + 1]
        qs = np.tile(q[i], (ks.shape[0], 1))
        oi, li = orc.attention_head(qs, ks, vs, 0.6, False, rows=[0])
        _close(o[i], oi[0], 1e-14, f"window row {i}")
        _close([lse[i]], li, 1e-14, f"window lse row {i}")


def pin_ranged_documents_are_independent(orc):
    """Packed documents under a causal mask: each document alone, causally."""
    r = _rng(42)
    lens = [5, 1, 12, 9]
    n, d = sum(lens), 4
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    start = np.repeat(np.cumsum([0] + lens[:-1]), lens)
    o, lse = orc.attention_ranged(q, k, v, 0.8, start, np.arange(n))
    for s0, ln in zip(np.cumsum([0] + lens[:-1]), lens):
        oi, li = orc.attention_head(q[s0:s0 + ln], k[s0:s0 + ln], v[s0:s0 + ln], 0.8, True)
        _close(o[s0:s0 + ln], oi, 1e-14, f"document at {s0}")
        _close(lse[s0:s0 + ln], li, 1e-14, f"document lse at {s0}")


def pin_ranged_single_key(orc):
    """lo = hi = j: O_i = v_j and lse_i = scale <q_i, k_j>."""
    r = _rng(43)
    n, d = 11, 3
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    j = r.integers(0, n, size=n)
    o, lse = orc.attention_ranged(q, k, v, 0.3, j, j)
    _close(o, v[j], 1e-15, "single key O")
    _close(lse, 0.3 * np.sum(q * k[j], axis=1), 1e-14, "single key LSE")


# ---------------------------------------------------------------------------
# key-set (block-sparse) pins
# ---------------------------------------------------------------------------
def pin_keyset_full_and_prefix_sets_are_attention(orc):
    """Every key, or keys 0..i, is dense or causal attention."""
    r = _rng(70)
    n, d = 29, 5
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    o1, l1 = orc.attention_keyset(q, k, v, 0.6, [np.arange(n)] * n)
    o2, l2 = orc.attention_head(q, k, v, 0.6, False)
    _close(o1, o2, 1e-14, "full key sets")
    _close(l1, l2, 1e-14, "full key sets LSE")
    o1, l1 = orc.attention_keyset(q, k, v, 0.6, [np.arange(i + 1) for i in range(n)])
    o2, l2 = orc.attention_head(q, k, v, 0.6, True)
    _close(o1, o2, 1e-14, "prefix key sets")
    _close(l1, l2, 1e-14, "prefix key sets LSE")


def pin_keyset_gaps_are_a_slice(orc):
    """A set with gaps is plain attention of q_i over the listed rows of K and V,
    whatever their order."""
    r = _rng(71)
    n, d = 40, 4
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    sets = [np.sort(r.choice(n, size=int(r.integers(1, n)), replace=False)) for _ in range(n)]
    o, lse = orc.attention_keyset(q, k, v, 0.7, sets)
    shuffled = [r.permutation(ks) for ks in sets]
    o2, l2 = orc.attention_keyset(q, k, v, 0.7, shuffled)
    _close(o, o2, 1e-14, "key order")
    _close(lse, l2, 1e-13, "key order LSE")
    for i in (0, 7, 39):
        ks = sets[i]
        oi, li = orc.attention_head(np.tile(q[i], (ks.size, 1)), k[ks], v[ks], 0.7, False, rows=[0])
        _close(o[i], oi[0], 1e-14, f"gapped set row {i}")
        _close([lse[i]], li, 1e-14, f"gapped set LSE row {i}")


def pin_keyset_single_and_empty(orc):
    """One key j: O_i = v_j and LSE_i = scale <q_i, k_j>.  No key: O_i = 0, LSE_i = -inf."""
    r = _rng(72)
    n, d = 9, 3
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    j = r.integers(0, n, size=n)
    sets = [np.array([jj]) for jj in j]
    sets[4] = np.zeros(0, np.int64)
    o, lse = orc.attention_keyset(q, k, v, 0.3, sets)
    for i in range(n):
        if i == 4:
            assert np.all(o[i] == 0.0) and lse[i] == -np.inf
        else:
            _close(o[i], v[j[i]], 1e-15, f"single key {i}")
            _close([lse[i]], [0.3 * float(q[i] @ k[j[i]])], 1e-14, f"single key LSE {i}")


def pin_block_sparse_keys(orc):
    """The block-sparse key rule: listed key blocks of the query's block, cut at N
    and at the diagonal when causal; a full pattern is dense attention."""
    n, qb, kb = 300, 128, 64
    n_qb, n_kb = -(-n // qb), -(-n // kb)
    blk_ptr = np.arange(n_qb + 1) * n_kb
    blk_idx = np.tile(np.arange(n_kb), n_qb)
    assert np.array_equal(orc.block_sparse_keys(n, 299, blk_ptr, blk_idx, qb, kb, False), np.arange(n))
    assert np.array_equal(orc.block_sparse_keys(n, 130, blk_ptr, blk_idx, qb, kb, True), np.arange(131))
    ptr2 = np.array([0, 2, 2, 3])
    idx2 = np.array([1, 3, 4])
    assert np.array_equal(orc.block_sparse_keys(n, 5, ptr2, idx2, qb, kb, False),
                          np.r_[np.arange(64, 128), np.arange(192, 256)])
    assert orc.block_sparse_keys(n, 200, ptr2, idx2, qb, kb, False).size == 0
    assert np.array_equal(orc.block_sparse_keys(n, 290, ptr2, idx2, qb, kb, True), np.arange(256, 291))
    r = _rng(73)
    q, k, v = (r.normal(size=(n, 4)) for _ in range(3))
    o1, l1 = orc.attention_blocksparse(q, k, v, 0.5, True, blk_ptr, blk_idx, qb, kb, rows=[0, 64, 299])
    o2, l2 = orc.attention_head(q, k, v, 0.5, True, rows=[0, 64, 299])
    _close(o1, o2, 1e-14, "full block pattern")
    _close(l1, l2, 1e-14, "full block pattern LSE")


# ---------------------------------------------------------------------------
# fp8 E4M3 decoding (the storage type of the fp8 forward)
# ---------------------------------------------------------------------------
def pin_fp8_decoder_known_codes(orc):
    """Codes whose values the OCP E4M3 definition fixes: 1, 2, -1, the largest
    finite value 448, the smallest normal 2^-6, the subnormals m * 2^-9, 256, zero,
    negative zero and the NaN codes."""
    table = {0x38: 1.0, 0x40: 2.0, 0xB8: -1.0, 0x7E: 448.0, 0xFE: -448.0, 0x08: 2.0 ** -6,
             0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x0F: 1.875 * 2.0 ** -6, 0x78: 256.0,
             0x2B: 0.34375, 0x00: 0.0, 0x80: -0.0, 0x3F: 1.875, 0x30: 0.5}
    codes = np.array(sorted(table), dtype=np.uint8)
    got = orc.to_f64(codes, "fp8")
    for c, g in zip(codes, got):
        assert g == table[int(c)], f"code {int(c):#04x}: {g} != {table[int(c)]}"
    assert np.isnan(orc.to_f64(np.array([0x7F, 0xFF], np.uint8), "fp8")).all()


def pin_fp8_decoder_order(orc):
    """Codes 0x00 .. 0x7E increase strictly, each binade holds 8 evenly spaced
    values, and the sign bit mirrors them."""
    pos = orc.to_f64(np.arange(0x7F, dtype=np.uint8), "fp8")
    assert np.all(np.diff(pos) > 0)
    for e in range(1, 16):
        seg = pos[8 * e: 8 * e + 8]
        steps = np.diff(seg)
        assert np.allclose(steps, steps[0], rtol=0, atol=0), f"binade {e} not evenly spaced"
        assert seg[0] == 2.0 ** (e - 7)
    neg = orc.to_f64(np.arange(0x80, 0xFF, dtype=np.uint8), "fp8")
    assert np.array_equal(neg, -pos)


# ---------------------------------------------------------------------------
# decode-shaped (Nq queries at the end of Nk keys) pins
# ---------------------------------------------------------------------------
def pin_decode_square_is_attention(orc):
    """Nq = Nk: the decode form is plain attention, causal or not."""
    r = _rng(60)
    n, d = 23, 5
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    for causal in (False, True):
        o1, l1 = orc.attention_decode(q, k, v, 0.7, causal)
        o2, l2 = orc.attention_head(q, k, v, 0.7, causal)
        _close(o1, o2, 1e-14, f"square decode O causal={causal}")
        _close(l1, l2, 1e-14, f"square decode LSE causal={causal}")


def pin_decode_query_sees_a_prefix(orc):
    """Causal, Nq < Nk: query i is one query over the keys 0 .. Nk - Nq + i."""
    r = _rng(61)
    nq, nk, d = 4, 19, 6
    q = r.normal(size=(nq, d))
    k, v = r.normal(size=(nk, d)), r.normal(size=(nk, d))
    o, lse = orc.attention_decode(q, k, v, 0.5, True)
    for i in range(nq):
        m = nk - nq + i + 1
        oi, li = orc.attention_head(np.tile(q[i], (m, 1)), k[:m], v[:m], 0.5, False, rows=[0])
        _close(o[i], oi[0], 1e-14, f"prefix query {i}")
        _close([lse[i]], li, 1e-14, f"prefix lse {i}")
    on, _ = orc.attention_decode(q, k, v, 0.5, False)
    _close(on[-1], o[-1], 1e-14, "the last query sees every key either way")
    assert np.max(np.abs(on[0] - o[0])) > 1e-3, "the first query must not see the last keys"


def pin_decode_uniform_scores(orc):
    """q = 0: every visible key weighs the same, O is the mean of the visible V
    rows and LSE = ln(count)."""
    r = _rng(62)
    nq, nk, d = 3, 10, 4
    k, v = r.normal(size=(nk, d)), r.normal(size=(nk, d))
    o, lse = orc.attention_decode(np.zeros((nq, d)), k, v, 1.3, True)
    for i in range(nq):
        cnt = nk - nq + i + 1
        _close(o[i], v[:cnt].mean(axis=0), 1e-15, f"uniform O {i}")
        _close([lse[i]], [math.log(cnt)], 1e-15, f"uniform LSE {i}")


def pin_decode_more_queries_than_keys(orc):
    """Non-causal with Nq > Nk (padding rows exist): each query sees the Nk keys only."""
    r = _rng(63)
    nq, nk, d = 9, 3, 4
    q = r.normal(size=(nq, d))
    k, v = r.normal(size=(nk, d)), r.normal(size=(nk, d))
    o, lse = orc.attention_decode(q, k, v, 0.9, False)
    s = 0.9 * q @ k.T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    _close(o, (p / p.sum(axis=1, keepdims=True)) @ v, 1e-14, "few keys O")
    _close(lse, s.max(axis=1) + np.log(p.sum(axis=1)), 1e-14, "few keys LSE")


# ---------------------------------------------------------------------------
# backward-pass pins
# ---------------------------------------------------------------------------
def _loss(orc, q, k, v, g, scale, causal):
    """L = sum_ie O_ie g_ie, whose gradient with upstream dO = g is the backward pass."""
    o, _ = orc.attention_head(q, k, v, scale, causal)
    return float(np.sum(o * g))


def pin_backward_finite_differences(orc):
    """Every entry of dQ, dK and dV against a central difference of the forward oracle
    (step 1e-5: truncation ~1e-10, rounding ~1e-11)."""
    r = _rng(30)
    n, d, scale = 6, 4, 0.7
    q, k, v, g = (r.normal(size=(n, d)) for _ in range(4))
    h = 1e-5
    for causal in (False, True):
        dq, dk, dv, _, _ = orc.attention_backward_head(q, k, v, g, scale, causal)
        for name, x, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [xp if t is x else t for t in (q, k, v)]
                args_m = [xm if t is x else t for t in (q, k, v)]
                num[idx] = (_loss(orc, *args_p, g, scale, causal) -
                            _loss(orc, *args_m, g, scale, causal)) / (2 * h)
            _close(grad, num, 1e-7, f"{name} finite difference causal={causal}")


def pin_backward_autograd(orc):
    """torch.autograd in float64 on the CPU, an implementation written independently of
    this oracle, on a 40 x 16 head."""
    import torch
    r = _rng(31)
    n, d, scale = 40, 16, 0.25
    q, k, v, g = (r.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
        s = scale * tq @ tk.T
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(n, n, dtype=torch.bool), 1), float("-inf"))
        o = torch.softmax(s, dim=-1) @ tv
        o.backward(torch.tensor(g))
        dq, dk, dv, _, _ = orc.attention_backward_head(q, k, v, g, scale, causal)
        _close(dq, tq.grad.numpy(), 1e-12, f"dQ autograd causal={causal}")
        _close(dk, tk.grad.numpy(), 1e-12, f"dK autograd causal={causal}")
        _close(dv, tv.grad.numpy(), 1e-12, f"dV autograd causal={causal}")


def pin_backward_column_sums(orc):
    """Rows of P sum to one, so sum_j dV_j = sum_i dO_i; rows of dS sum to zero, so
    sum_j dK_j = 0."""
    r = _rng(32)
    n, d = 50, 8
    q, k, v, g = (r.normal(0, 1.5, size=(n, d)) for _ in range(4))
    for causal in (False, True):
        _, dk, dv, _, _ = orc.attention_backward_head(q, k, v, g, 0.6, causal)
        _close(dv.sum(axis=0), g.sum(axis=0), 1e-12, f"sum dV causal={causal}")
        _close(dk.sum(axis=0), np.zeros(d), 1e-12, f"sum dK causal={causal}")


def pin_backward_statistics(orc):
    """D_i equals <dO_i, O_i> (O = P V), and the saved statistic equals the forward LSE."""
    r = _rng(33)
    n, d = 45, 9
    q, k, v, g = (r.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        _, _, _, lse, dd = orc.attention_backward_head(q, k, v, g, 0.35, causal)
        o, lse_f = orc.attention_head(q, k, v, 0.35, causal)
        _close(dd, np.sum(g * o, axis=1), 1e-13, f"D = dO . O causal={causal}")
        _close(lse, lse_f, 1e-14, f"saved statistic causal={causal}")


def pin_backward_given_output(orc):
    """Passing the forward output O gives D_i = <dO_i, O_i>: with the exact O the
    gradients are those of the definition; with O rounded to bf16 only D moves, by
    <dO_i, O_i - round(O_i)>."""
    r = _rng(36)
    n, d, scale = 30, 8, 0.5
    q, k, v, g = (r.normal(size=(n, d)) for _ in range(4))
    for causal in (False, True):
        o, _ = orc.attention_head(q, k, v, scale, causal)
        ref = orc.attention_backward_head(q, k, v, g, scale, causal)
        got = orc.attention_backward_head(q, k, v, g, scale, causal, o=o)
        for a, b, what in zip(got, ref, ("dQ", "dK", "dV", "lse", "D")):
            _close(a, b, 1e-12, f"given exact O {what} causal={causal}")
        orr = workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(o.astype(np.float32))).astype(np.float64)
        got = orc.attention_backward_head(q, k, v, g, scale, causal, o=orr)
        _close(got[4], ref[4] + np.sum(g * (orr - o), axis=1), 1e-13, f"given rounded O D causal={causal}")
        _close(got[2], ref[2], 1e-13, f"given rounded O leaves dV causal={causal}")


def pin_backward_magnitudes(orc):
    """The sums of absolute values bound the sums themselves, change nothing else, and
    equal them where every term is non-negative: with dO >= 0, dV_j = sum_i P_ij dO_i
    has only non-negative terms (P >= 0)."""
    r = _rng(37)
    n, d, scale = 33, 6, 0.4
    q, k, v = (r.normal(size=(n, d)) for _ in range(3))
    g = np.abs(r.normal(size=(n, d)))
    for causal in (False, True):
        plain = orc.attention_backward_head(q, k, v, g, scale, causal)
        dq, dk, dv, lse, dd, mq, mk, mv = orc.attention_backward_head(q, k, v, g, scale, causal,
                                                                       magnitudes=True)
        for a, b, what in zip((dq, dk, dv, lse, dd), plain, ("dQ", "dK", "dV", "lse", "D")):
            _close(a, b, 0.0, f"magnitudes change {what} causal={causal}")
        for m, x, what in ((mq, dq, "dQ"), (mk, dk, "dK"), (mv, dv, "dV")):
            assert np.all(m >= np.abs(x) - 1e-15), f"|{what}| exceeds its magnitude sum"
        _close(mv, dv, 1e-14, f"dV magnitude with dO >= 0 causal={causal}")
        # mixed signs: every magnitude bounds its sum, and the bound is not attained
        gm = r.normal(size=(n, d))
        dq2, dk2, dv2, _, _, mq2, mk2, mv2 = orc.attention_backward_head(q, k, v, gm, scale, causal,
                                                                          magnitudes=True)
        for m, x, what in ((mq2, dq2, "dQ"), (mk2, dk2, "dK"), (mv2, dv2, "dV")):
            assert np.all(m >= np.abs(x) - 1e-15), f"|{what}| exceeds its magnitude sum (mixed signs)"
            assert np.mean(m) > 1.2 * np.mean(np.abs(x)), f"{what} magnitude equals the sum (mixed signs)"
        # dQ_i's terms scale |dS_ij| |k_j|: with k replaced by |k| and dS of one sign per
        # row... simplest exact case: one visible key gives dS = 0, so mq = 0 on causal row 0
        if causal:
            _close(mq[0], np.zeros(d), 1e-15, "magnitude of dQ_0 under the causal mask")


def pin_backward_zero_query(orc):
    """Q = 0: P_ij = 1/n_i over the n_i visible keys, so dK = 0,
    dV_j = sum over the queries i that see j of dO_i / n_i, and
    dQ_i = (scale / n_i) sum_j (dP_ij - mean_j dP_ij) k_j with dP_ij = <dO_i, v_j>."""
    r = _rng(34)
    n, d, scale = 23, 5, 0.45
    k, v, g = (r.normal(size=(n, d)) for _ in range(3))
    q = np.zeros((n, d))
    for causal in (False, True):
        dq, dk, dv, _, _ = orc.attention_backward_head(q, k, v, g, scale, causal)
        cnt = np.arange(1, n + 1) if causal else np.full(n, n)
        dv_ref = np.zeros((n, d))
        dq_ref = np.zeros((n, d))
        for i in range(n):
            vis = cnt[i]
            dv_ref[:vis] += g[i] / vis
            dp = v[:vis] @ g[i]
            dq_ref[i] = scale / vis * ((dp - dp.mean())[:, None] * k[:vis]).sum(axis=0)
        _close(dk, np.zeros((n, d)), 1e-15, f"zero-q dK causal={causal}")
        _close(dv, dv_ref, 1e-14, f"zero-q dV causal={causal}")
        _close(dq, dq_ref, 1e-14, f"zero-q dQ causal={causal}")


def pin_backward_causal_edges(orc):
    """Causal: query 0 sees only key 0 (P = 1, so dS = 0 and dQ_0 = 0), and the last key
    is seen only by the last query: dV_last = P_last,last dO_last."""
    r = _rng(35)
    n, d = 12, 6
    q, k, v, g = (r.normal(size=(n, d)) for _ in range(4))
    dq, _, dv, _, _ = orc.attention_backward_head(q, k, v, g, 0.8, True)
    p_last = orc.attention_probs(q, k, 0.8, True, n - 1)
    _close(dq[0], np.zeros(d), 1e-15, "causal dQ_0")
    _close(dv[n - 1], p_last[n - 1] * g[n - 1], 1e-15, "causal dV_last")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
