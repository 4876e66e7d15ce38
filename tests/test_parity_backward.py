"""Attention backward on the GPU (through the C ABI) against the fp64 oracle.

The backward receives the forward output O (it enters through D_i = <dO_i, O_i>)
and the logsumexp.  The parity cases give the GPU and the oracle the same O --
the oracle's forward output rounded to the storage type, as a caller would hold
it -- and the oracle's logsumexp in fp32, so the comparison measures the
backward kernels' own arithmetic.

Gate.  The stated 16-bit tolerance -- max-abs 1e-2 (taken relative to
max(1, |ref|), since gradients reach several units and rounding the output
alone costs up to 2^-8 |ref|) and relative L2 5e-3 per tensor -- extended, per
element, by what the arithmetic allows where terms cancel.  Each gradient
element is a sum of products in which one factor, P (for dV) or dS (for dK,
dQ), is rounded to 16 bits (unit roundoff u = 2^-8 for bf16, 2^-11 for fp16)
before the fp32 product, and the result is rounded once more, so its error
reaches u M + u |ref|, M being the sum of the absolute values of its terms (the
oracle's magnitude sums); a second u M covers the fp32 effects (recomputed
scores, exp2, dP - D).  Where terms cancel, M is many times |ref| -- dV of an
early key sums thousands of P_ij dO_i of both signs -- so an element passes
when |got - ref| <= max(1e-2 max(1, |ref|), 2 u M + u |ref|).

The chain cases run the GPU forward and feed its O and logsumexp to the GPU
backward, the way a training step does, against the oracle's exact gradients.
There the rounding of O enters D and is amplified by the cancellation in
dP - D on rows with few visible keys, so those cases are gated on relative L2
(1e-2) only.
"""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import oracle
import workloads
from gpu_util import say, to_device, to_f64

pytestmark = pytest.mark.gpu

FWD = {"bf16": fa.fa_fwd, "f16": fa.fa_fwd_f16}
BWD = {"bf16": fa.fa_bwd, "f16": fa.fa_bwd_f16}


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def run_bwd(q, k, v, o, g, lse, dtype, scale, causal):
    """GPU backward of storage-type arrays (o, lse device tensors or host arrays)."""
    B, H, N, d = q.shape
    qd, kd, vd, gd = (to_device(t, dtype) for t in (q, k, v, g))
    od = o if isinstance(o, torch.Tensor) else to_device(o, dtype)
    ld = lse if isinstance(lse, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(lse, np.float32)).cuda()
    dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N) // 4, dtype=torch.float32, device="cuda")
    BWD[dtype](qd, kd, vd, od, gd, ld, dq, dk, dv, ws, B, H, N, d, scale, int(causal))
    torch.cuda.synchronize()
    return dq, dk, dv


def run_chain(q, k, v, g, dtype, scale, causal):
    """GPU forward for O and the logsumexp, then the GPU backward."""
    B, H, N, d = q.shape
    qd, kd, vd = (to_device(t, dtype) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    FWD[dtype](qd, kd, vd, o, lse, B, H, N, d, scale, int(causal))
    return run_bwd(q, k, v, o, g, lse, dtype, scale, causal)


def oracle_forward(orc, q, k, v, dtype, scale, causal, heads=None):
    """O rounded to the storage type and lse in fp32, from the oracle, for `heads`
    (the other heads are left zero)."""
    B, H, N, d = q.shape
    o = np.zeros((B, H, N, d), np.float32)
    lse = np.zeros((B, H, N), np.float32)
    for b, h in heads or [(b, h) for b in range(B) for h in range(H)]:
        ob, lb = orc.attention_head(q[b, h], k[b, h], v[b, h], scale, causal, dtype=dtype)
        o[b, h], lse[b, h] = ob, lb
    return workloads.cast(o, dtype), lse


UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}


def check(orc, name, q, k, v, g, dtype, scale, causal, grads, heads=None, o=None, rel_only=False):
    """Oracle gradients (D from `o` when given) against the GPU's for `heads`."""
    B, H, N, d = q.shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    names = ("dQ", "dK", "dV")
    got = {n: [] for n in names}
    ref = {n: [] for n in names}
    mag = {n: [] for n in names}
    for b, h in heads:
        rq, rk, rv, _, _, mq, mk, mv = orc.attention_backward_head(
            q[b, h], k[b, h], v[b, h], g[b, h], scale, causal, dtype=dtype,
            o=None if o is None else o[b, h], magnitudes=True)
        for n, r, m, t in (("dQ", rq, mq, grads[0]), ("dK", rk, mk, grads[1]), ("dV", rv, mv, grads[2])):
            ref[n].append(r)
            mag[n].append(m)
            got[n].append(to_f64(t[b, h]))
    u = UNIT_ROUNDOFF[dtype]
    for n in names:
        gt, rf, m = np.concatenate(got[n]), np.concatenate(ref[n]), np.concatenate(mag[n])
        err = np.abs(gt - rf)
        rel = float(np.linalg.norm(gt - rf) / max(np.linalg.norm(rf), 1e-300))
        bound = np.maximum(1e-2 * np.maximum(1.0, np.abs(rf)), 2 * u * m + u * np.abs(rf))
        worst = float(np.max(err / bound)) if err.size else 0.0
        say(f"  {name} {n}: max_abs={float(err.max()):.3e} rel_l2={rel:.3e} worst err/bound={worst:.3f}")
        assert np.all(np.isfinite(gt)), f"{name} {n}: non-finite output"
        if rel_only:
            assert not np.any(rf != 0) or rel <= 1e-2, f"{name} {n}: rel_l2 {rel:.3e} > 1e-2"
            continue
        if worst > 1.0:
            r, c = np.unravel_index(int(np.argmax(err / bound)), err.shape)
            raise AssertionError(f"{name} {n}: row {r} dim {c}: |err| {err[r, c]:.3e} > bound "
                                 f"{bound[r, c]:.3e} (ref {rf[r, c]:.4f}, magnitude {m[r, c]:.3f})")
        assert not np.any(rf != 0) or rel <= 5e-3, f"{name} {n}: rel_l2 {rel:.3e} > 5e-3"


def upstream(shape, seed):
    """The upstream gradient dO: iid N(0, 1) in float32, stored like the operands."""
    rng = np.random.default_rng([workloads.BASE_SEED + 700, seed, *shape])
    return rng.standard_normal(shape, dtype=np.float32)


EDGE_N = [1, 2, 63, 64, 65, 129, 200, 300]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", EDGE_N)
def test_backward_edge_shapes(orc, dtype, d, causal, N):
    B, H = 1, 3
    say(f"[attention backward edge] dtype={dtype} d={d} causal={causal} N={N}")
    q, k, v = workloads.random_attn(B, H, N, d, dtype, seed=N * 11 + d)
    g = workloads.cast(upstream((B, H, N, d), N + d), dtype)
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle_forward(orc, q, k, v, dtype, scale, causal)
    grads = run_bwd(q, k, v, o, g, lse, dtype, scale, causal)
    check(orc, f"bwd {dtype} d{d} c{int(causal)} N{N}", q, k, v, g, dtype, scale, causal, grads, o=o)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_backward_several_tiles(orc, causal, d):
    """N = 1000: several query blocks, key blocks and tiles with a ragged tail on each side."""
    B, H, N = 2, 2, 1000
    say(f"[attention backward] bf16 d={d} causal={causal} N={N}")
    q, k, v = workloads.random_attn(B, H, N, d, "bf16", seed=77 + d)
    g = workloads.cast(upstream((B, H, N, d), 5 + d), "bf16")
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle_forward(orc, q, k, v, "bf16", scale, causal)
    grads = run_bwd(q, k, v, o, g, lse, "bf16", scale, causal)
    check(orc, f"bwd bf16 d{d} c{int(causal)} N{N}", q, k, v, g, "bf16", scale, causal, grads, o=o)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("B,H", [(2, 4), (1, 3)])
@pytest.mark.parametrize("N", [700, 1025])
def test_backward_causal_block_pairs(orc, dtype, d, B, H, N):
    """Causal dQ workgroups take two 256-query blocks of one head, one from each
    end of the sequence: odd block counts (3 and 5, ragged last block), with the
    XCD-grouped order (B*H = 8) and the plain one (B*H = 3)."""
    say(f"[attention backward causal pairs] dtype={dtype} d={d} B={B} H={H} N={N}")
    q, k, v = workloads.random_attn(B, H, N, d, dtype, seed=N * 5 + d + H)
    g = workloads.cast(upstream((B, H, N, d), N + 3 * d + H), dtype)
    scale = 1.0 / np.sqrt(d)
    o, lse = oracle_forward(orc, q, k, v, dtype, scale, True)
    grads = run_bwd(q, k, v, o, g, lse, dtype, scale, True)
    check(orc, f"bwd pairs {dtype} d{d} B{B}H{H} N{N}", q, k, v, g, dtype, scale, True, grads, o=o)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [2, 65, 1000])
def test_backward_chain(orc, causal, N):
    """GPU forward then GPU backward, against the oracle's exact gradients (relative L2)."""
    B, H, d = 1, 2, 128
    say(f"[attention backward chain] bf16 d={d} causal={causal} N={N}")
    q, k, v = workloads.random_attn(B, H, N, d, "bf16", seed=300 + N)
    g = workloads.cast(upstream((B, H, N, d), 300 + N), "bf16")
    grads = run_chain(q, k, v, g, "bf16", 1.0 / np.sqrt(d), causal)
    check(orc, f"chain c{int(causal)} N{N}", q, k, v, g, "bf16", 1.0 / np.sqrt(d), causal, grads,
          rel_only=True)


def test_backward_headline_shape(orc):
    """The B8 H32 N8192 d128 causal workload (K rows x U(0.5, 2)) in its full launch;
    eight heads, one in each batch row and spread over the head index (so over
    the XCD groups of the launch), get the oracle's O and logsumexp and are
    checked in full; the other heads get the GPU forward's."""
    w = workloads.ATTN["attn_bf16_b8h32n8192_causal"]
    heads = [(b, (9 * b) % w.H) for b in range(w.B)]
    say(f"[attention backward] attn_bf16_b8h32n8192_causal, heads {heads} checked")
    q, k, v = workloads.attn_full(w, threads=16)
    g = workloads.cast(upstream((w.B, w.H, w.N, w.d), 1), "bf16")
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    od = torch.empty_like(qd)
    ld = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device="cuda")
    fa.fa_fwd(qd, kd, vd, od, ld, w.B, w.H, w.N, w.d, w.sm_scale, 1)
    o_or, l_or = oracle_forward(orc, q, k, v, "bf16", w.sm_scale, True, heads)
    for b, h in heads:
        od[b, h] = to_device(o_or[b, h], "bf16")
        ld[b, h] = torch.from_numpy(l_or[b, h]).cuda()
    del qd, kd, vd
    grads = run_bwd(q, k, v, od, g, ld, "bf16", w.sm_scale, True)
    for t in grads:
        assert torch.isfinite(t.float()).all()
    check(orc, "bwd c4", q, k, v, g, "bf16", w.sm_scale, True, grads, heads=heads, o=o_or)


def test_backward_is_deterministic():
    q, k, v = workloads.random_attn(1, 2, 700, 128, "bf16", seed=3)
    g = workloads.cast(upstream((1, 2, 700, 128), 3), "bf16")
    a = run_chain(q, k, v, g, "bf16", 0.0884, True)
    b = run_chain(q, k, v, g, "bf16", 0.0884, True)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def test_backward_wrapper():
    q, k, v = (to_device(t, "bf16") for t in workloads.random_attn(1, 2, 96, 64, "bf16", seed=9))
    o, lse = fa.attention(q, k, v, causal=True)
    g = torch.randn_like(o)
    dq, dk, dv = fa.attention_backward(q, k, v, o, g, lse, causal=True)
    assert dq.shape == q.shape and dk.dtype == q.dtype and torch.isfinite(dv.float()).all()
    with pytest.raises(ValueError):
        fa.attention_backward(q, k, v, o, g, lse[:, :1])
