"""The GPU tests' gates, checked on the CPU against a model of the 16-bit kernels'
rounding (kernel_model.forward16): the gates must accept that arithmetic, and
must reject it once a plausible mistake is planted in the model (a missing
rescale of l or of O, a wrong denominator on some rows).

This pins the derived logsumexp bound (gpu_util.lse_tolerance) and the
peaked-row gate of the rescale stress cases at both head dims: at d = 64 the
kernel keeps l in a matrix accumulator with its own rescale, and only scores
that rise tile after tile make that rescale matter."""
import numpy as np
import pytest

import kernel_model as km
import oracle
import workloads
from gpu_util import causal_vis, gate, gate_lse, lse_tolerance
from test_parity_attention import large_score_inputs, peaked_gate, rising_inputs


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def model_head(orc, q, k, v, dtype, scale, causal, **planted):
    qv, kv, vv = (orc.to_f64(t, dtype) for t in (q, k, v))
    return km.forward16(qv, kv, vv, scale, causal, dtype, **planted)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_gates_accept_the_kernel_rounding(orc, dtype, d, causal):
    N = 600
    q, k, v = workloads.random_attn(1, 1, N, d, dtype, seed=31 + d + int(causal))
    scale = d ** -0.5
    o, lse = model_head(orc, q[0, 0], k[0, 0], v[0, 0], dtype, scale, causal)
    ro, rl = orc.attention_head(q[0, 0], k[0, 0], v[0, 0], scale, causal, dtype=dtype)
    gate("model O", o, ro, dtype)
    qv, kv = orc.to_f64(q[0, 0], dtype), orc.to_f64(k[0, 0], dtype)
    bound, sigma = lse_tolerance(qv, kv, rl, scale, dtype,
                                 causal_vis(np.arange(N), N) if causal else None)
    gate_lse("model LSE", lse, rl, bound, sigma)
    # the bound is far below the former max(1, |lse|) 1e-2 gate
    assert np.all(bound < 6e-3)


@pytest.mark.parametrize("d", [64, 128])
def test_lse_gate_rejects_a_wrong_denominator(orc, d):
    N, dtype = 600, "bf16"
    q, k, v = workloads.random_attn(1, 1, N, d, dtype, seed=5 + d)
    scale = d ** -0.5
    _, lse = model_head(orc, q[0, 0], k[0, 0], v[0, 0], dtype, scale, True)
    _, rl = orc.attention_head(q[0, 0], k[0, 0], v[0, 0], scale, True, dtype=dtype)
    bound, sigma = lse_tolerance(orc.to_f64(q[0, 0], dtype), orc.to_f64(k[0, 0], dtype), rl, scale,
                                 dtype, causal_vis(np.arange(N), N))
    gate_lse("model LSE", lse, rl, bound, sigma)
    rows = np.random.default_rng(1).random(N) < 0.1
    with pytest.raises(AssertionError):  # l off by 1% on a tenth of the rows
        gate_lse("l x 1.01", lse + np.where(rows, np.log(1.01), 0.0), rl, bound, sigma)
    with pytest.raises(AssertionError):  # l off by 0.05% on every row
        gate_lse("l x 1.0005", lse + np.log(1.0005), rl, bound, sigma)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("step", [3.0, 8.1, 30.0])
def test_rising_case_catches_missing_rescales(orc, dtype, d, step):
    """The rising-score inputs of the GPU test: the model passes the peaked gate,
    and fails it without the rescale of l or without that of O."""
    q, k, v = rising_inputs(dtype, d, step)
    scale = d ** -0.5
    for h in range(q.shape[1]):
        args = (q[0, h], k[0, h], v[0, h], dtype, scale, True)
        o, lse = model_head(orc, *args)
        peaked_gate(orc, f"model rising d{d} step{step}", q[0, h], k[0, h], v[0, h], o, lse, dtype,
                    scale, True)
    if step < 8.0:
        return  # below the slack the reference never moves: no rescale to drop
    for planted in ("drop_l_rescale", "drop_o_rescale"):
        o, lse = model_head(orc, q[0, 0], k[0, 0], v[0, 0], dtype, scale, True, **{planted: True})
        with pytest.raises(AssertionError):
            peaked_gate(orc, f"model {planted}", q[0, 0], k[0, 0], v[0, 0], o, lse, dtype, scale, True)


@pytest.mark.parametrize("d", [64, 128])
def test_large_scores_case_catches_missing_rescales(orc, d):
    dtype = "bf16"
    q, k, v = large_score_inputs(dtype, d)
    scale = d ** -0.5
    o, lse = model_head(orc, q[0, 0], k[0, 0], v[0, 0], dtype, scale, False)
    peaked_gate(orc, f"model large d{d}", q[0, 0], k[0, 0], v[0, 0], o, lse, dtype, scale, False)
    for planted in ("drop_l_rescale", "drop_o_rescale"):
        o, lse = model_head(orc, q[0, 0], k[0, 0], v[0, 0], dtype, scale, False, **{planted: True})
        with pytest.raises(AssertionError):
            peaked_gate(orc, f"model {planted}", q[0, 0], k[0, 0], v[0, 0], o, lse, dtype, scale, False)
