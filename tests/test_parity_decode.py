"""Split-KV decode-shaped attention (fa_decode / fa_decode_f16) on the GPU, through
the C ABI, against the fp64 oracle.

The queries are the last Nq positions of the Nk-key sequence; the oracle is the
definition (each query over its visible keys, three passes in fp64).  Gate: the
stated 16-bit tolerance, max-abs 1e-2 and relative L2 5e-3 on O; the logsumexp
within the bound derived from its arithmetic (gpu_util.lse_tolerance; the merge
of the chunks' partial sums adds a few fp32 roundings, fewer than the n/16 the
bound allows for the sum).

Cases: Nq of 1 (decode), a few (speculative tokens) and more than one 32-query
group (a prefill chunk), Nk across the 32-key tile and the chunk boundaries
(chunks of 4 to 32 tiles), Nq > Nk without the causal mask, both head sizes,
both 16-bit types; the B8 H32 Nq1 Nk32768 d128 workload in full (every head
checked); a workspace shared by two calls; determinism.
"""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import oracle
import workloads
from gpu_util import gate, gate_lse, lse_tolerance, say, to_device, to_f64

pytestmark = pytest.mark.gpu

ENTRY = {"bf16": fa.fa_decode, "f16": fa.fa_decode_f16}


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def run(q, k, v, dtype, scale, causal, ws=None):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    qd, kd, vd = (to_device(t, dtype) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    nbytes = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    assert nbytes > 0
    if ws is None:
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    ENTRY[dtype](qd, kd, vd, o, lse, ws, ws.numel() * 4, B, H, Nq, Nk, d, scale, int(causal))
    torch.cuda.synchronize()
    return o, lse


def check(orc, name, q, k, v, dtype, scale, causal, o, lse, heads=None):
    B, H = q.shape[:2]
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    got_o, ref_o, got_l, ref_l, lb, ls = [], [], [], [], [], []
    for b, h in heads:
        ro, rl = orc.attention_decode(q[b, h], k[b, h], v[b, h], scale, causal, dtype=dtype)
        ref_o.append(ro)
        ref_l.append(rl)
        got_o.append(to_f64(o[b, h]))
        got_l.append(to_f64(lse[b, h]))
        nq, nk = q.shape[2], k.shape[2]
        vis = (np.arange(nk)[None, :] <= (nk - nq + np.arange(nq))[:, None]) if causal else None
        bd, sg = lse_tolerance(orc.to_f64(q[b, h], dtype), orc.to_f64(k[b, h], dtype), rl, scale,
                               dtype, vis)
        lb.append(bd)
        ls.append(sg)
    gate(f"{name} O", np.concatenate(got_o), np.concatenate(ref_o), dtype)
    gate_lse(f"{name} LSE", np.concatenate(got_l), np.concatenate(ref_l), np.concatenate(lb),
             np.concatenate(ls))


SHAPES = [(1, 1), (1, 31), (1, 33), (1, 1000), (1, 4097), (3, 100), (4, 5000), (32, 40),
          (33, 500), (70, 70), (5, 300)]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("nq,nk", SHAPES)
def test_decode_shapes(orc, dtype, d, causal, nq, nk):
    B, H = 2, 3
    say(f"[decode] dtype={dtype} d={d} causal={causal} Nq={nq} Nk={nk}")
    q, _, _ = workloads.random_attn(B, H, nq, d, dtype, seed=nq * 7 + d)
    _, k, v = workloads.random_attn(B, H, nk, d, dtype, seed=nk * 13 + d + 1)
    scale = 1.0 / np.sqrt(d)
    o, lse = run(q, k, v, dtype, scale, causal)
    check(orc, f"decode {dtype} d{d} c{int(causal)} {nq}x{nk}", q, k, v, dtype, scale, causal, o, lse)


@pytest.mark.parametrize("nq,nk", [(40, 7), (64, 1)])
def test_more_queries_than_keys(orc, nq, nk):
    """Without the causal mask any Nq is allowed, also more queries than keys."""
    q, _, _ = workloads.random_attn(1, 2, nq, 128, "bf16", seed=nq)
    _, k, v = workloads.random_attn(1, 2, nk, 128, "bf16", seed=nk + 100)
    say(f"[decode] Nq={nq} > Nk={nk}")
    o, lse = run(q, k, v, "bf16", 0.0884, False)
    check(orc, f"decode {nq}x{nk}", q, k, v, "bf16", 0.0884, False, o, lse)


def test_long_single_head(orc):
    """One head, Nk = 131072 at d = 64: 1024 chunks of 4 tiles, merged per query."""
    q, _, _ = workloads.random_attn(1, 1, 2, 64, "bf16", seed=1)
    _, k, v = workloads.random_attn(1, 1, 131072, 64, "bf16", seed=2)
    say("[decode] 1 head, Nq=2, Nk=131072, d=64")
    o, lse = run(q, k, v, "bf16", 0.125, True)
    check(orc, "decode 2x131072", q, k, v, "bf16", 0.125, True, o, lse)


def test_peaked_scores(orc):
    """Q x 10 (scores with a standard deviation near 10): the trailing reference
    maximum moves several times and a few keys per query hold nearly all the weight."""
    q, _, _ = workloads.random_attn(1, 2, 3, 128, "bf16", seed=5, std=10.0)
    _, k, v = workloads.random_attn(1, 2, 3000, 128, "bf16", seed=6)
    say("[decode] peaked scores")
    o, lse = run(q, k, v, "bf16", 0.0884, True)
    check(orc, "decode peaked", q, k, v, "bf16", 0.0884, True, o, lse)


def test_workload(orc):
    w = workloads.DECODE["decode_bf16_b8h32_q1_kv32768_d128"]
    say(f"[decode workload {w.name}] every head checked")
    q, k, v = workloads.decode_full(w, threads=16)
    o, lse = run(q, k, v, w.dtype, w.sm_scale, w.causal)
    assert torch.isfinite(o.float()).all()
    check(orc, w.name, q, k, v, w.dtype, w.sm_scale, w.causal, o, lse)


def test_equals_forward_when_square(orc):
    """Nq = Nk: the same attention as fa_fwd (both against the oracle, and close
    to each other within the 16-bit rounding of O)."""
    q, k, v = workloads.random_attn(1, 2, 300, 128, "bf16", seed=8)
    o, lse = run(q, k, v, "bf16", 0.0884, True)
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    fo, fl = fa.attention(qd, kd, vd, causal=True, scale=0.0884)
    torch.cuda.synchronize()
    # One 16-bit rounding of O apart, plus fp32 differences.  The two kernels use
    # other tile sizes, so their reference maxima move at other keys and P is
    # rounded to 16 bits against other references: l, the sum of the rounded P,
    # differs by up to about 2^-9 relative in each, so ln l (the logsumexp) by up
    # to about 2^-8.
    assert float(((o.float() - fo.float()).abs() / fo.float().abs().clamp(min=1)).max()) <= 2.0 ** -6
    assert float((lse - fl).abs().max()) <= 2.0 ** -7


def test_workspace_reuse_and_determinism(orc):
    """Two calls share one workspace, the second with fewer chunks; a repeat of the
    first call gives identical bits."""
    qa, _, _ = workloads.random_attn(2, 2, 2, 128, "bf16", seed=21)
    _, ka, va = workloads.random_attn(2, 2, 20000, 128, "bf16", seed=22)
    qb, _, _ = workloads.random_attn(1, 1, 1, 128, "bf16", seed=23)
    _, kb, vb = workloads.random_attn(1, 1, 700, 128, "bf16", seed=24)
    nbytes = fa.fa_decode_workspace_bytes(2, 2, 2, 20000, 128)
    assert nbytes > fa.fa_decode_workspace_bytes(1, 1, 1, 700, 128)
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    oa, la = run(qa, ka, va, "bf16", 0.0884, True, ws=ws)
    oa, la = oa.clone(), la.clone()
    ob, lb = run(qb, kb, vb, "bf16", 0.0884, True, ws=ws)
    check(orc, "reuse a", qa, ka, va, "bf16", 0.0884, True, oa, la)
    check(orc, "reuse b", qb, kb, vb, "bf16", 0.0884, True, ob, lb)
    oa2, la2 = run(qa, ka, va, "bf16", 0.0884, True, ws=ws)
    assert torch.equal(oa.view(torch.int16), oa2.view(torch.int16)) and torch.equal(la, la2)


def test_wrapper():
    q = torch.randn(1, 2, 3, 64, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 2, 500, 64, device="cuda").to(torch.bfloat16)
    v = torch.randn(1, 2, 500, 64, device="cuda").to(torch.bfloat16)
    o, lse = fa.attention_decode(q, k, v, causal=True)
    assert o.shape == q.shape and lse.shape == (1, 2, 3) and torch.isfinite(o.float()).all()
    with pytest.raises(ValueError):
        fa.attention_decode(q, k[:, :1], v)
