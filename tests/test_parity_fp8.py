"""fp8 attention forward (fa_fwd_fp8) on the GPU, through the C ABI, against the
fp64 oracle.

The inputs are E4M3 codes with per-tensor descales; the oracle decodes them with
its own decoder, multiplies by the descales and computes attention on those
exact values.  So the only error of the kernel beyond fp32 arithmetic is its
own rounding of P to E4M3 and of O to bf16, and the gates follow from those
(no tolerance is stated for fp8).

Per element (query i, head dim e), with P the exact probabilities, o the exact
output, p_j = exp(s_ij - m_i) <= 1 the unnormalised weights and l_i their sum:
the kernel multiplies V by P~_j, 2^7 p'_j rounded to E4M3, and divides by the sum
of the P~_j, where p'_j = 2^(x_j - m') is the weight against its reference
maximum m' <= m_i (p'_j >= p_j, and the largest is at least 1).  For
2^7 p'_j >= 2^-6 (normal) the rounding error is at most u = 2^-4 relative;
below, at most 2^-10 absolute, i.e. 2^-17 in units of p.  So

    |O - o| <= (u M1 + 2^-17 A) / (1 - u) + 2^-8 |o| + 1e-5,
    M1 = sum_j P_j |v_je - o_e|,  A = sum_j |v_je - o_e| / l_i,

the last two terms for the bf16 rounding of O and fp32 effects.  That bound is
reached only if every rounding errs the same way; the errors of distinct
weights behave like independent uniform variables, so the gate also requires
the root mean square of |O - o| / sigma to stay below 2, sigma^2 =
(u^2/3) sum_j P_j^2 (v_je - o_e)^2 + (2^-34/3) sum_j (v_je - o_e)^2 / l_i^2 +
(2^-16/3) o_e^2 + 1e-10.  A dropped tile or a misplaced key moves the error far
outside sigma.  The logsumexp: |LSE - lse| <= -ln(1 - u) + 2^-17 n_i / l_i +
1e-4, and rms of its error over sqrt((u^2/3) sum_j P_j^2 + 1e-8) below 2.
"""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import oracle
import workloads
from gpu_util import say, to_f64

pytestmark = pytest.mark.gpu

U8 = 2.0 ** -4      # E4M3 unit roundoff (3 mantissa bits)
SUB = 2.0 ** -17    # half the smallest subnormal step of 2^7 p, in units of p
UBF = 2.0 ** -8     # bf16 unit roundoff


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def run(q8, k8, v8, scale, desc, causal, with_lse=True):
    B, H, N, d = q8.shape
    qd, kd, vd = (torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in (q8, k8, v8))
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda") if with_lse else None
    fa.fa_fwd_fp8(qd, kd, vd, o, lse, B, H, N, d, scale, *desc, int(causal))
    torch.cuda.synchronize()
    return o, lse


def values(orc, t8, descale):
    return orc.to_f64(t8, "fp8") * descale


def check(orc, name, q8, k8, v8, scale, desc, causal, o, lse, heads=None, rows_of=None):
    B, H, N, d = q8.shape
    heads = heads or [(b, h) for b in range(B) for h in range(H)]
    worst_o = worst_l = 0.0
    z_o, z_l = [], []
    for b, h in heads:
        qv, kv, vv = (values(orc, t[b, h], s) for t, s in zip((q8, k8, v8), desc))
        rows = np.arange(N) if rows_of is None else rows_of(b, h)
        ro, rl = orc.attention_head(qv, kv, vv, scale, causal, rows)
        go = to_f64(o[b, h])[rows]
        gl = to_f64(lse[b, h])[rows]
        for n_r, i in enumerate(rows):
            P = orc.attention_probs(qv, kv, scale, causal, int(i))
            vis = np.arange(int(i) + 1) if causal else np.arange(N)
            Pv = P[vis]
            l_i = 1.0 / Pv.max()
            dv = np.abs(vv[vis] - ro[n_r][None, :])              # |v_je - o_e|
            M1 = Pv @ dv
            A = dv.sum(axis=0) / l_i
            bound = (U8 * M1 + SUB * A) / (1 - U8) + UBF * np.abs(ro[n_r]) + 1e-5
            sig = np.sqrt(U8 ** 2 / 3 * (Pv ** 2 @ dv ** 2) + SUB ** 2 / 3 * (dv ** 2).sum(axis=0) / l_i ** 2
                          + UBF ** 2 / 3 * ro[n_r] ** 2 + 1e-10)
            err = np.abs(go[n_r] - ro[n_r])
            assert np.all(np.isfinite(go[n_r])), f"{name}: non-finite O in row {i}"
            worst_o = max(worst_o, float(np.max(err / bound)))
            if np.any(err > bound):
                e = int(np.argmax(err / bound))
                raise AssertionError(f"{name} head ({b},{h}) row {i} dim {e}: |err| {err[e]:.3e} > "
                                     f"bound {bound[e]:.3e} (ref {ro[n_r][e]:.4f})")
            z_o.append(err / sig)
            lbound = -np.log1p(-U8) + SUB * len(vis) / l_i + 1e-4
            lerr = abs(gl[n_r] - rl[n_r])
            worst_l = max(worst_l, lerr / lbound)
            assert lerr <= lbound, f"{name} head ({b},{h}) row {i}: LSE err {lerr:.3e} > {lbound:.3e}"
            z_l.append(lerr / np.sqrt(U8 ** 2 / 3 * float(Pv @ Pv) + 1e-8))
    rms_o = float(np.sqrt(np.mean(np.concatenate(z_o) ** 2)))
    rms_l = float(np.sqrt(np.mean(np.square(z_l))))
    say(f"  {name}: worst O err/bound {worst_o:.3f}, rms O err/sigma {rms_o:.3f}; "
        f"worst LSE err/bound {worst_l:.3f}, rms LSE err/sigma {rms_l:.3f}")
    assert rms_o <= 2.0, f"{name}: rms O error {rms_o:.3f} sigma"
    assert rms_l <= 2.0, f"{name}: rms LSE error {rms_l:.3f} sigma"


def random_fp8(B, H, N, d, seed, desc=(1 / 64, 1 / 64, 1 / 64), std=1.0):
    q, k, v = workloads.random_attn(B, H, N, d, "f32", seed=seed, std=std)
    return tuple(workloads.cast(t / s, "fp8") for t, s in zip((q, k, v), desc))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 2, 63, 64, 65, 129, 200, 300, 1000])
def test_fp8_edge_shapes(orc, causal, N, d):
    B, H = 1, 3
    desc = (1 / 64, 1 / 64, 1 / 64)
    say(f"[attention fp8 edge] d={d} causal={causal} N={N}")
    q8, k8, v8 = random_fp8(B, H, N, d, seed=N + 7 + d, desc=desc)
    o, lse = run(q8, k8, v8, 1 / np.sqrt(d), desc, causal)
    check(orc, f"fp8 d{d} c{int(causal)} N{N}", q8, k8, v8, 1 / np.sqrt(d), desc, causal, o, lse)


def test_fp8_workload(orc):
    """The B8 H32 N8192 d128 causal fp8 workload in its full launch; heads (0, 0), (3, 17)
    and (7, 31) checked on 256 sampled rows each (tile and diagonal boundaries included)."""
    w = workloads.ATTN["attn_fp8_b8h32n8192_causal"]
    say(f"[attention fp8 workload {w.name}]")
    q8, k8, v8 = workloads.attn_full(w, threads=16)
    o, lse = run(q8, k8, v8, w.sm_scale, w.descales, True)
    assert torch.isfinite(o.float()).all()
    check(orc, w.name, q8, k8, v8, w.sm_scale, w.descales, True, o, lse,
          heads=[(0, 0), (3, 17), (7, 31)], rows_of=lambda b, h: workloads.attn_sample_rows(w, b, h))


@pytest.mark.parametrize("step", [0.3, 4.0])
def test_fp8_rising_scores(orc, step):
    """Scores that climb by `step` (log2 units) per 64-key tile: the row maximum
    moves on every tile and O is rescaled each time."""
    B, H, N, d = 1, 2, 1024, 128
    scale = 1.0 / np.sqrt(d)
    q, k, v = workloads.random_attn(B, H, N, d, "f32", seed=int(step * 10) + 3)
    rng = np.random.default_rng([19, int(step * 10)])
    rate = np.float32(step / (64 * scale * np.log2(np.e)))
    q[..., 0] = np.float32(1.0) + np.float32(0.5) * rng.random((B, H, N), dtype=np.float32)
    k[..., 0] = rate * np.arange(N, dtype=np.float32)[None, None, :]
    kmax = float(np.abs(k).max())
    desc = (1 / 64, 2.0 ** np.ceil(np.log2(kmax / 400)), 1 / 64)
    q8, k8, v8 = (workloads.cast(t / s, "fp8") for t, s in zip((q, k, v), desc))
    say(f"[attention fp8 rising scores] step={step} k_descale={desc[1]}")
    o, lse = run(q8, k8, v8, scale, desc, True)
    check(orc, f"fp8 rising step{step}", q8, k8, v8, scale, desc, True, o, lse)


def test_fp8_lse_optional(orc):
    q8, k8, v8 = random_fp8(1, 2, 200, 128, seed=5)
    o1, _ = run(q8, k8, v8, 0.09, (1 / 64,) * 3, True, with_lse=True)
    o2, _ = run(q8, k8, v8, 0.09, (1 / 64,) * 3, True, with_lse=False)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def emulate(orc, q8, k8, v8, desc, scale, causal, tile=64):
    """The fp8 kernel's arithmetic restated on the CPU, for one head: per 64-key
    tile, the reference maximum moves to the row maximum when that passes it by
    more than 1.5 (log2 units), each weight 2^7 p is rounded to E4M3 (the input
    encoder's rounding: nearest, ties to even), l and O sum the rounded weights,
    O is scaled by the V descale over l."""
    qv, kv, vv = (orc.to_f64(t, "fp8") for t in (q8, k8, v8))
    n = qv.shape[0]
    c = scale * desc[0] * desc[1] * np.log2(np.e)
    S = (qv @ kv.T) * c
    O = np.zeros_like(qv)
    L = np.zeros(n)
    for i in range(n):
        m, l, acc = -np.inf, 0.0, np.zeros(qv.shape[1])
        last = i if causal else n - 1
        for t0 in range(0, last + 1, tile):
            x = S[i, t0:min(last + 1, t0 + tile)]
            m_new = max(m, x.max())
            if m_new <= m + 1.5:
                m_new = m
            alpha = 0.0 if m == -np.inf else 2.0 ** (m - m_new)
            p = orc.to_f64(workloads.f32_to_e4m3(2.0 ** (x - m_new + 7)), "fp8")
            l = l * alpha + p.sum()
            acc = acc * alpha + p @ vv[t0:t0 + x.size]
            m = m_new
        O[i] = acc / l * desc[2]
        L[i] = (m + np.log2(l) - 7) * np.log(2)
    return O, L


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_matches_its_arithmetic(orc, causal, d):
    """Against the emulation of the kernel's own rounding every output element
    is expected within the bf16 rounding of O (2^-8 |O|) plus a small absolute
    term; every wave group of the workgroup is covered (N = 300 spans 256 + 44
    queries).  This bound is far tighter than the gate against the exact result.
    The exception is a weight whose E4M3 rounding flips between the kernel's fp32
    and the emulation's fp64 arguments: that moves its row by one E4M3 step
    (2^-3 relative) of the weight's share, which exceeds the bound when the weight
    dominates the row.  A flip needs the argument within about 2^-20 of a rounding
    midpoint, so at most one row per head is allowed outside the bound, and that
    row is held to the one-flip bounds below (the gate against the exact result
    holds for every row in the other tests)."""
    B, H, N = 1, 3, 300
    desc = (1 / 64, 1 / 64, 1 / 64)
    q8, k8, v8 = random_fp8(B, H, N, d, seed=N + 7, desc=desc)
    o, lse = run(q8, k8, v8, 1 / np.sqrt(d), desc, causal)
    for h in range(H):
        eo, el = emulate(orc, q8[0, h], k8[0, h], v8[0, h], desc, 1 / np.sqrt(d), causal)
        go, gl = to_f64(o[0, h]), to_f64(lse[0, h])
        err, lerr = np.abs(go - eo), np.abs(gl - el)
        off = np.unique(np.concatenate([np.nonzero(err > 2.0 ** -7 * np.abs(eo) + 0.01)[0],
                                        np.nonzero(lerr > 5e-3)[0]]))
        say(f"  fp8 emulation d{d} c{int(causal)} head {h}: max |O - emul| {err.max():.2e}, "
            f"max |LSE - emul| {lerr.max():.2e}, rows outside the tight bound {off.tolist()}")
        assert off.size <= 1, f"head {h}: rows {off.tolist()} off the kernel's arithmetic"
        vmax = float(np.abs(orc.to_f64(v8[0, h], "fp8")).max() * desc[2])
        for r in off:  # one flipped weight: |dO| <= 2^-3 * 2 max|v|, |dLSE| <= ln(1 + 2^-3)
            assert err[r].max() <= 2.0 ** -3 * 2 * vmax and lerr[r] <= np.log1p(2.0 ** -3)
