"""Helpers of the GPU parity tests: device upload of the seeded inputs, read-back,
and the pass/fail gates.

Gates (the tolerances stated for this path): fp32 inputs, max-abs <= 1e-4;
bf16 / fp16 inputs, max-abs <= 1e-2 and relative L2 <= 5e-3.  Errors are taken
against the unrounded fp64 oracle over every checked element of a case.  A
failure names the first offending query row and head dimension.

The logsumexp, which the stated tolerances do not name, is gated by a bound
derived from its arithmetic (lse_tolerance).  The kernels form
lse = ln 2 (m + log2 l) with l the fp32 sum of the weights 2^(c s_j - m) after
their rounding to the operand type (unit roundoff u: 2^-8 bf16, 2^-11 fp16; the
fp32 path does not round them), so per row, in natural-log units:

  * rounding the weights moves ln l by at most u / (1 - u) (each weight by a
    relative u at most), plus, in fp16, 2^-25 per weight that falls below the
    normal range (l >= 1 since the largest weight is >= 1);
  * the fp32 sum of l: at most (n/16 + 8) dependent additions per lane (16 keys
    per matrix step or per pair of two-term dot products, then the tile chain
    and the merge of the lane halves), n per key on the fp32 path, 2^-24 each;
  * the hardware 2^x: about one ulp per weight, 2^-22 relative on l;
  * the scores: an fp32 dot product of d exact products and the rounding of
    c = scale log2 e and of the FMA, at most 2 d 2^-24 A_i with
    A_i = scale max_j sum_c |q_ic k_jc| over the visible keys (a convex
    combination of score errors moves the lse by at most the largest);
  * the final log2, the addition of m and the product by ln 2:
    2^-21 (|lse| + 1).

Every element must meet that worst-case sum.  Independent roundings rarely
line up, so the root mean square of the error over its expected spread sigma_i
must also stay below 2, with sigma_i^2 = (u^2 / 3) sum_j P_ij^2 (the variance
of sum_j P_ij delta_j for weight roundings delta_j uniform in [-u, u]) plus the
squares of the other terms taken as random walks: 2^-24 sqrt(depth),
2^-24 (sqrt(d) + 2) A_i, 2^-22 and 2^-22 (|lse| + 1).  At the B8 H32 N8192
d128 workload the worst-case bound is about 4e-3 and sigma about 1e-4 on
rows that spread their weight over a thousand keys.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TOL = {
    "f32": dict(max_abs=1e-4, rel_l2=None),
    "bf16": dict(max_abs=1e-2, rel_l2=5e-3),
    "f16": dict(max_abs=1e-2, rel_l2=5e-3),
}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr)).cuda()


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def stats(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    idx = np.unravel_index(int(np.argmax(diff)), diff.shape) if diff.size else ()
    return {
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)),
        "argmax": tuple(int(i) for i in idx),
        "finite": bool(np.all(np.isfinite(got))),
    }


def gate(what: str, got, ref, dtype: str, rows=None, max_abs=None):
    """Assert the tolerance of `dtype`; rows maps the first axis to query rows.
    max_abs overrides the element bound for cases outside the stated workloads."""
    s = stats(got, ref)
    tol = dict(TOL[dtype])
    if max_abs is not None:
        tol["max_abs"] = max_abs
    say(f"  {what}: max_abs={s['max_abs']:.3e} rel_l2={s['rel_l2']:.3e}")
    assert s["finite"], f"{what}: non-finite output"
    ref64 = np.asarray(ref, np.float64)
    bound = tol["max_abs"]
    bad = np.abs(np.asarray(got, np.float64) - ref64) > bound
    if bad.any():
        first = np.argwhere(bad)[0]
        row = int(first[0]) if rows is None else int(np.asarray(rows)[first[0]])
        col = int(first[-1]) if bad.ndim > 1 else -1
        raise AssertionError(f"{what}: max_abs {s['max_abs']:.3e} > {tol['max_abs']:.0e}; first "
                             f"offending element at query row {row}, head dim {col}")
    # relative L2 is undefined for an all-zero reference (e.g. dQ of one-key rows);
    # the element bound above still applies there
    if tol["rel_l2"] is not None and np.any(ref64 != 0):
        assert s["rel_l2"] <= tol["rel_l2"], f"{what}: rel_l2 {s['rel_l2']:.3e} > {tol['rel_l2']:.0e}"
    return s


UNIT_P = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 0.0}
E24 = 2.0 ** -24


def lse_tolerance(qv, kv, ref, scale, dtype, vis=None):
    """Per-row worst-case bound and expected spread of the logsumexp error.

    qv [R, d] and kv [Nk, d] are the float64 values of the checked query rows and
    of the keys, ref [R] the oracle's (finite) logsumexp, vis [R, Nk] the visible
    keys (None: all).  The derivation is in the module docstring."""
    qv = np.asarray(qv, np.float64)
    kv = np.asarray(kv, np.float64)
    ref = np.asarray(ref, np.float64)
    step = max(1, (1 << 22) // max(1, kv.shape[0]))  # rows per chunk: a few 10 MB per array
    if qv.shape[0] > step:
        parts = [lse_tolerance(qv[r:r + step], kv, ref[r:r + step], scale, dtype,
                               None if vis is None else vis[r:r + step])
                 for r in range(0, qv.shape[0], step)]
        return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])
    d = qv.shape[1]
    s = scale * (qv @ kv.T)
    a = scale * (np.abs(qv) @ np.abs(kv).T)
    if vis is not None:
        s = np.where(vis, s, -np.inf)
        a = np.where(vis, a, 0.0)
        n = vis.sum(axis=1).astype(np.float64)
    else:
        n = np.full(qv.shape[0], float(kv.shape[0]))
    amax = a.max(axis=1)
    sp2 = np.exp(2.0 * (s - ref[:, None])).sum(axis=1)
    u = UNIT_P[dtype]
    depth = n + 8 if dtype == "f32" else n / 16 + 8
    sub = n * 2.0 ** -25 if dtype == "f16" else 0.0
    bound = (u / (1 - u) + sub + depth * E24 + 2.0 ** -22 + 2 * d * E24 * amax
             + 2.0 ** -21 * (np.abs(ref) + 1))
    sigma = np.sqrt(u * u / 3 * sp2 + (np.sqrt(depth) * E24) ** 2 + (2.0 ** -22) ** 2
                    + ((np.sqrt(d) + 2) * E24 * amax) ** 2 + (2.0 ** -22 * (np.abs(ref) + 1)) ** 2
                    + (sub / 2) ** 2)
    return bound, sigma


def gate_lse(what, got, ref, bound, sigma, rows=None):
    """The logsumexp gate: every |got - ref| within `bound`, and the root mean
    square of |got - ref| / sigma at most 2 (lse_tolerance gives both)."""
    got = np.ravel(np.asarray(got, np.float64))
    ref = np.ravel(np.asarray(ref, np.float64))
    bound, sigma = np.ravel(bound), np.ravel(sigma)
    assert np.all(np.isfinite(got)), f"{what}: non-finite logsumexp"
    err = np.abs(got - ref)
    if not err.size:
        return
    ratio = err / bound
    rms = float(np.sqrt(np.mean((err / sigma) ** 2)))
    say(f"  {what}: max_abs={float(err.max()):.3e} worst err/bound={float(ratio.max()):.3f} "
        f"(bound {float(bound.min()):.2e}..{float(bound.max()):.2e}) rms err/sigma={rms:.3f}")
    if ratio.max() > 1.0:
        i = int(np.argmax(ratio))
        row = i if rows is None else int(np.ravel(rows)[i])
        raise AssertionError(f"{what}: query row {row}: |err| {err[i]:.3e} > bound {bound[i]:.3e}")
    assert rms <= 2.0, f"{what}: rms error {rms:.3f} sigma > 2"


def causal_vis(rows, nk):
    """Visible keys of `rows` under the square causal rule (key j <= query i)."""
    return np.asarray(rows)[:, None] >= np.arange(nk)[None, :]


def range_vis(rows, lo, hi, nk):
    """Visible keys of `rows` when query i sees keys lo[i] .. hi[i]."""
    rows = np.asarray(rows)
    j = np.arange(nk)[None, :]
    return (j >= np.asarray(lo)[rows][:, None]) & (j <= np.asarray(hi)[rows][:, None])


def set_vis(sets, nk):
    """Visible keys given one key-index array per checked row."""
    vis = np.zeros((len(sets), nk), bool)
    for r, ks in enumerate(sets):
        vis[r, np.asarray(ks, np.int64)] = True
    return vis


def softmax_rel_gate(what, got, ref, x):
    """Relative gate of the row softmax on every element the fp32 output holds as
    a normal number: |y - y*| <= y* (max(1e-5, 4 2^-23 sqrt(n)) + 2^-22 (|x - m| + 2 R)),
    n the row length, m its maximum and R = max - min of the row.  The first
    term is the pages' check for an fp32 sum of n terms ("100 Days of GPU, Day
    97", Check); the second is the rounding of the exponent argument, formed in
    fp32 as (x - m_t) log2 e against a partial maximum m_t of the row and then
    moved to m by a second factor 2^((m_t - m) log2 e): each rounding is 2^-24
    of an argument of at most |x - m| + |m_t - m| <= |x - m| + R (log2 units
    times log2 e, and 2^a moves by ln 2 times a's error)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    x = np.asarray(x, np.float64)
    n = x.shape[1]
    m = x.max(axis=1, keepdims=True)
    r = m - x.min(axis=1, keepdims=True)
    bound = max(1e-5, 4 * 2.0 ** -23 * np.sqrt(n)) + 2.0 ** -22 * (np.abs(x - m) + 2 * r)
    live = ref > 2.0 ** -126
    if not live.any():
        return
    rel = np.abs(got[live] - ref[live]) / ref[live]
    ratio = rel / bound[live]
    say(f"  {what}: worst relative error {float(rel.max()):.3e}, worst rel/bound {float(ratio.max()):.3f}")
    if ratio.max() > 1.0:
        i = int(np.argmax(ratio))
        r_i, c_i = np.argwhere(live)[i]
        raise AssertionError(f"{what}: row {r_i} col {c_i}: relative error {rel[i]:.3e} > "
                             f"{bound[live][i]:.3e}")


def reversed_rows(N: int, causal: bool) -> int:
    """Rows at the start of each head that the dense causal 16-bit forward computes
    with its key tiles in descending order: a causal workgroup takes query blocks
    mt and n - 1 - mt (256 rows each, n = ceil(N / 256)) and walks the second, the
    shorter one (mt < n // 2), from the diagonal down.  Kernels that walk every
    block upwards give these rows the same keys in another order."""
    return 256 * (((N + 255) // 256) // 2) if causal else 0


def same_but_order(what, o1, l1, o2, l2, N, causal, vmax):
    """o1/l1 against the dense causal forward's o2/l2 for the same keys: bit-equal on
    the rows both walk upwards.  On the rows the dense kernel walks downwards
    (reversed_rows) its reference maximum moves at other tiles, so each 16-bit
    weight may round differently (by at most half a unit, u = 2^-9 of bf16 or 2^-12
    of fp16, relative).  O is the weights' convex combination of V rows, so each
    side is within u * 2 max|V| of the exact combination, and after its own
    rounding to 16 bits within another u |O|: the two differ by at most
    4 u max|V| + 2 u max|O|.  l sums the rounded weights, so each logsumexp is
    within ln(1 + u) of the exact one: they differ by at most 2 u (+ 1e-6 for the
    fp32 arithmetic)."""
    r = reversed_rows(N, causal)
    a1, a2 = o1.view(torch.int16), o2.view(torch.int16)
    assert torch.equal(a1[..., r:, :], a2[..., r:, :]) and torch.equal(l1[..., r:], l2[..., r:]), \
        f"{what}: rows walked in the same order differ"
    if r:
        u = 2.0 ** -9 if o1.dtype == torch.bfloat16 else 2.0 ** -12
        x1, x2 = o1[..., :r, :].float(), o2[..., :r, :].float()
        bad = (x1 - x2).abs() > 4 * u * vmax + 2 * u * torch.maximum(x1.abs(), x2.abs())
        assert not bool(bad.any()), f"{what}: {int(bad.sum())} elements beyond the rounding bound"
        dl = float((l1[..., :r] - l2[..., :r]).abs().max())
        assert dl <= 2 * u + 1e-6, f"{what}: logsumexp differs by {dl:.3g}"
