"""A CPU restatement of the 16-bit attention kernels' rounding, for the CPU tests
that check the GPU tests' gates (test infrastructure; the product never runs it,
and the oracle is a separate, exact definition).

The 16-bit forward kernels compute, per query row and key tile of BN keys (64
at d = 128, 128 at d = 64), with c = scale * log2(e) rounded to fp32:

  * the scores s_j as an fp32 dot product of the 16-bit operands (modelled as
    the exact product rounded once to fp32);
  * a reference maximum m that moves to the running maximum max(m, c max_j s_j)
    only when that has passed it by more than `slack` (8 in log2 units);
  * alpha = 2^(m_old - m_new), weights p_j = 2^(fp32(c s_j - m_new)) rounded to
    the operand type, l = alpha l + sum_j p_j, O = alpha O + sum_j p_j v_j;
  * after the last tile O / l rounded to the operand type, and
    lse = ln 2 (m + log2 l).

Planted mistakes (for tests that show a gate catches them): drop_l_rescale
leaves l unscaled when the reference moves, drop_o_rescale does the same to O.
"""
from __future__ import annotations

import numpy as np

import workloads

LOG2E = np.float32(1.4426950408889634)


def round16(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round-to-nearest-even to bf16 or fp16, returned as float64 values."""
    x32 = np.asarray(x, np.float32)
    if dtype == "bf16":
        return workloads.bf16_bits_to_f32(workloads.f32_to_bf16_bits(x32)).astype(np.float64)
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float64)
    raise ValueError(dtype)


def tile_keys(d: int) -> int:
    return 128 if d == 64 else 64


def forward16(qv, kv, vv, scale, causal, dtype, slack=8.0, bn=None, drop_l_rescale=False,
              drop_o_rescale=False):
    """O [N, d] (rounded to dtype, as float64) and lse [N] of one head, q/k/v given
    as float64 values of 16-bit numbers."""
    qv, kv, vv = (np.asarray(t, np.float64) for t in (qv, kv, vv))
    n, d = qv.shape
    bn = bn or tile_keys(d)
    c = np.float32(np.float32(scale) * LOG2E)
    s32 = (qv @ kv.T).astype(np.float32)
    m = np.full(n, -np.inf)
    l = np.zeros(n)
    o = np.zeros((n, d))
    rows = np.arange(n)
    for j0 in range(0, n, bn):
        keys = np.arange(j0, min(n, j0 + bn))
        s = s32[:, keys].astype(np.float64)
        if causal:
            s = np.where(keys[None, :] <= rows[:, None], s, -np.inf)
        mx = s.max(axis=1)
        live = np.isfinite(mx)
        m_cand = np.where(live, np.maximum(m, (np.float32(mx) * c).astype(np.float64)), m)
        m_new = np.where(m_cand > m + slack, m_cand, m)
        m_sub = np.where(np.isneginf(m_new), 0.0, m_new)
        alpha = np.exp2(m - m_sub)
        arg = (s * np.float64(c) - m_sub[:, None]).astype(np.float32).astype(np.float64)
        p = round16(np.exp2(arg), dtype)
        ps = p.sum(axis=1)
        l = (l if drop_l_rescale else l * alpha) + ps
        o = (o if drop_o_rescale else o * alpha[:, None]) + p @ vv[keys]
        m = m_new
    with np.errstate(divide="ignore", invalid="ignore"):
        out = round16(o / l[:, None], dtype)
        lse = (m + np.log2(l)) * np.log(2.0)
    return out, lse
