"""The fp64 oracle against its pins, plus an independent vectorised numpy cross-check."""
import numpy as np
import pytest

import oracle
import workloads
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def _numpy_attention(q, k, v, scale, causal, rows):
    """Vectorised fp64 softmax(scale Q K^T) V for the given rows (a second implementation)."""
    s = scale * (q[rows] @ k.T)
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= rows[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ v, (m + np.log(l))[:, 0]


@pytest.mark.parametrize("name", ["attn_f32_n256", "attn_f32_n256_last", "attn_bf16_n4096",
                                  "attn_bf16_b8h32n8192_causal", "attn_bf16_n131072_causal"])
def test_numpy_cross_check(orc, name):
    w = workloads.ATTN[name]
    heads = [(0, 0)] if w.B * w.H == 1 else [(0, 0), (w.B - 1, w.H - 1)]
    for b, h in heads:
        q, k, v = workloads.attn_head(w, b, h)
        rows = workloads.attn_sample_rows(w, b, h)
        if w.N > 8192:
            rows = rows[::8]
        o, lse = orc.attention_head(q, k, v, w.sm_scale, w.causal, rows, dtype=w.dtype)
        q64, k64, v64 = (orc.to_f64(t, w.dtype) for t in (q, k, v))
        o2, lse2 = _numpy_attention(q64, k64, v64, w.sm_scale, w.causal, rows)
        assert np.max(np.abs(o - o2)) < 1e-12
        assert np.max(np.abs(lse - lse2)) < 1e-12


def test_softmax_numpy_cross_check(orc):
    w = workloads.SOFTMAX["softmax_4096x32768"]
    x = workloads.softmax_input(w, rows=slice(0, 16))
    y = orc.softmax_rows(x)
    x64 = x.astype(np.float64)
    e = np.exp(x64 - x64.max(axis=1, keepdims=True))
    assert np.max(np.abs(y - e / e.sum(axis=1, keepdims=True))) < 1e-15


def test_bf16_decoder_matches_torch(orc):
    import torch
    bits = np.arange(0, 65536, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]          # finite values only
    mine = orc.to_f64(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, ref)
