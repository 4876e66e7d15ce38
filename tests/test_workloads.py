"""The seeded input generators: determinism, rounding and the recipes' structure."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40], np.float32)])
    mine = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = workloads.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_heads_are_deterministic_and_distinct():
    w = workloads.ATTN["attn_bf16_b8h32n8192_causal"]
    a = workloads.attn_head(w, 3, 7)
    b = workloads.attn_head(w, 3, 7)
    c = workloads.attn_head(w, 3, 8)
    for x, y, z in zip(a, b, c):
        assert x.dtype == np.uint16 and x.shape == (8192, 128)
        assert np.array_equal(x, y)
        assert not np.array_equal(x, z)


def test_k_row_scaling_range():
    w = workloads.ATTN["attn_bf16_b8h32n8192_causal"]
    _, k, _ = workloads.attn_head(w, 0, 0)
    kf = workloads.bf16_bits_to_f32(k)
    rms = np.sqrt((kf.astype(np.float64) ** 2).mean(axis=1))
    # rows are N(0,1) times u ~ U(0.5, 2): the row RMS spans that range up to the
    # sampling spread of a 128-element RMS (about 6% per row, 25% at the extremes)
    assert 0.35 < rms.min() < 0.6 and 1.8 < rms.max() < 2.7


def test_sample_rows():
    w = workloads.ATTN["attn_bf16_n131072_causal"]
    rows = workloads.attn_sample_rows(w, 0, 0)
    assert rows.size == 256 and np.unique(rows).size == 256
    for r in (0, 1, 63, 64, 127, 128, w.N - 1):
        assert r in rows
    assert np.array_equal(rows, workloads.attn_sample_rows(w, 0, 0))
    small = workloads.ATTN["attn_bf16_n4096"]
    assert workloads.attn_sample_rows(small, 0, 0).size == 4096


def test_softmax_input_recipe():
    w = workloads.SOFTMAX["softmax_4096x32768"]
    x = workloads.softmax_input(w, rows=slice(10, 14))
    assert x.dtype == np.float32 and x.shape == (4, 32768)
    spikes = (x == 50.0).sum(axis=1)
    assert np.all(spikes >= 1) and np.all(np.abs(spikes - 327.68) < 80)
    assert np.array_equal(x, workloads.softmax_input(w, rows=slice(10, 14)))
    assert np.array_equal(x[1], workloads.softmax_input(w, rows=slice(11, 12))[0])


def test_e4m3_encoder_round_trips_every_code():
    """The input encoder inverts the oracle's own decoder on every finite code and
    rounds to the nearest code, ties to the even one."""
    import oracle
    orc = oracle.load()
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.to_f64(codes, "fp8")
    finite = ~np.isnan(vals) & (codes != 0x80)
    assert np.array_equal(workloads.f32_to_e4m3(vals[finite].astype(np.float32)), codes[finite])
    # midpoints go to the even code; just above a midpoint goes up
    pos = vals[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    got = workloads.f32_to_e4m3(mid.astype(np.float32)).astype(np.int64)
    lo = np.arange(0x7E)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))
    assert workloads.f32_to_e4m3(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


def test_fp8_workload_stays_in_range():
    """The fp8 recipe's descales keep every draw of a head inside +-448 (no saturation)."""
    w = workloads.ATTN["attn_fp8_b8h32n8192_causal"]
    q, k, v = workloads._head_f32(w, 3, 17)
    sq, sk, sv = w.descales
    assert np.abs(q).max() / sq < 448 and np.abs(k).max() / sk < 448 and np.abs(v).max() / sv < 448
    q8, k8, v8 = workloads.attn_head(w, 3, 17)
    assert q8.dtype == np.uint8 and q8.shape == (w.N, w.d)


@pytest.mark.parametrize("N,causal,p", [(1, True, 0.0), (300, False, 0.3), (1400, True, 0.2),
                                        (8192, True, 0.1)])
def test_block_sparse_pattern_is_valid_csr(N, causal, p):
    """Offsets start at 0 and grow to nnz; each list ascending, distinct, in range,
    holding the sink block and the diagonal block of its query block; causal lists
    hold no block that starts after the query block's last row."""
    ptr, idx = workloads.block_sparse_pattern(N, seed=3, p_random=p, causal=causal)
    nqb, nkb = (N + 255) // 256, (N + 127) // 128
    assert ptr.dtype == np.int32 and idx.dtype == np.int32 and ptr.shape == (nqb + 1,)
    assert ptr[0] == 0 and ptr[-1] == idx.size and np.all(np.diff(ptr) >= 0)
    for qb in range(nqb):
        lst = idx[ptr[qb]:ptr[qb + 1]]
        last_row = min(N, 256 * (qb + 1)) - 1
        assert np.all(np.diff(lst) > 0) and lst.min() >= 0 and lst.max() < nkb
        assert 0 in lst and last_row // 128 in lst
        if causal:
            assert np.all(lst * 128 <= last_row)
    assert np.array_equal(ptr, workloads.block_sparse_pattern(N, seed=3, p_random=p, causal=causal)[0])


@pytest.mark.parametrize("N,causal", [(300, False), (700, True), (1400, True)])
def test_block_sparse_pairs_counts_the_oracle_key_lists(N, causal):
    """The pair count the benchmark prices equals the sum of the oracle's key-list
    lengths over all queries."""
    import oracle
    ptr, idx = workloads.block_sparse_pattern(N, seed=11, p_random=0.3, causal=causal)
    total = sum(len(oracle.Oracle.block_sparse_keys(N, i, ptr, idx, 256, 128, causal))
                for i in range(N))
    assert workloads.block_sparse_pairs(N, ptr, idx, causal) == total
