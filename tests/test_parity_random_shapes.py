"""Seeded random shapes for the entry points (dense, window + documents and
block-sparse forward, split-KV decode, fp8 forward, backward, row softmax and
its split form), each against the fp64 oracle with the gates of the entry's own
parity tests: the sizes, element type, causality, window, document lengths,
pattern and value scales are drawn from seeded generators, so a failure names
a reproducible case."""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import oracle
import workloads
from gpu_util import (causal_vis, gate, gate_lse, lse_tolerance, range_vis, say, softmax_rel_gate,
                      to_device, to_f64)

pytestmark = pytest.mark.gpu

CASES = 24


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def draw(case):
    rng = np.random.default_rng([4242, case])
    return dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), N=int(rng.integers(1, 2500)),
                d=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f16"])),
                causal=bool(rng.integers(0, 2)), window=int(rng.choice([0, 1, 17, 300, 1024])),
                seed=int(rng.integers(0, 1 << 30)), p=float(rng.uniform(0.0, 0.6)))


def compare(orc, name, outs, refs, dtype, tols):
    """tols: per head, the (bound, sigma) of gpu_util.lse_tolerance for its rows."""
    go, gl = np.concatenate([o for o, _ in outs]), np.concatenate([l for _, l in outs])
    ro, rl = np.concatenate([o for o, _ in refs]), np.concatenate([l for _, l in refs])
    lb, ls = np.concatenate([t[0] for t in tols]), np.concatenate([t[1] for t in tols])
    empty = np.isneginf(rl)
    assert np.all(np.isneginf(gl[empty])) and np.all(go[empty] == 0.0), f"{name}: empty rows"
    if (~empty).any():
        gate(f"{name} O", go[~empty], ro[~empty], dtype)
        gate_lse(f"{name} LSE", gl[~empty], rl[~empty], lb[~empty], ls[~empty])


@pytest.mark.parametrize("case", range(CASES))
def test_random_dense(orc, case):
    c = draw(case)
    B, H, N, d, dt = c["B"], c["H"], c["N"], c["d"], c["dtype"]
    say(f"[random dense {case}] {c}")
    q, k, v = workloads.random_attn(B, H, N, d, dt, seed=c["seed"])
    qd, kd, vd = (to_device(t, dt) for t in (q, k, v))
    o, lse = torch.empty_like(qd), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    (fa.fa_fwd if dt == "bf16" else fa.fa_fwd_f16)(qd, kd, vd, o, lse, B, H, N, d, d ** -0.5, int(c["causal"]))
    torch.cuda.synchronize()
    outs, refs, tols = [], [], []
    for b in range(B):
        for h in range(H):
            refs.append(orc.attention_head(q[b, h], k[b, h], v[b, h], d ** -0.5, c["causal"], dtype=dt))
            outs.append((to_f64(o[b, h]), to_f64(lse[b, h])))
            tols.append(lse_tolerance(orc.to_f64(q[b, h], dt), orc.to_f64(k[b, h], dt), refs[-1][1],
                                      d ** -0.5, dt, causal_vis(np.arange(N), N) if c["causal"] else None))
    compare(orc, f"random dense {case}", outs, refs, dt, tols)


@pytest.mark.parametrize("case", range(CASES))
def test_random_local(orc, case):
    c = draw(case + 100)
    B, H, N, d, dt = c["B"], c["H"], c["N"], c["d"], c["dtype"]
    say(f"[random local {case}] {c}")
    q, k, v = workloads.random_attn(B, H, N, d, dt, seed=c["seed"])
    doc = workloads.packed_doc_starts(B, N, c["seed"] % 1000, 1, max(2, N // 2))
    qd, kd, vd = (to_device(t, dt) for t in (q, k, v))
    o, lse = torch.empty_like(qd), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    entry = fa.fa_fwd_local if dt == "bf16" else fa.fa_fwd_local_f16
    entry(qd, kd, vd, o, lse, torch.from_numpy(doc).cuda(), c["window"], B, H, N, d, d ** -0.5)
    torch.cuda.synchronize()
    outs, refs, tols = [], [], []
    for b in range(B):
        lo, hi = workloads.local_ranges(doc[b], c["window"])
        for h in range(H):
            refs.append(orc.attention_ranged(q[b, h], k[b, h], v[b, h], d ** -0.5, lo, hi, np.arange(N), dtype=dt))
            outs.append((to_f64(o[b, h]), to_f64(lse[b, h])))
            tols.append(lse_tolerance(orc.to_f64(q[b, h], dt), orc.to_f64(k[b, h], dt), refs[-1][1],
                                      d ** -0.5, dt, range_vis(np.arange(N), lo, hi, N)))
    compare(orc, f"random local {case}", outs, refs, dt, tols)


@pytest.mark.parametrize("case", range(CASES))
def test_random_blocksparse(orc, case):
    c = draw(case + 200)
    B, H, N, d, dt = c["B"], c["H"], c["N"], c["d"], c["dtype"]
    say(f"[random block-sparse {case}] {c}")
    q, k, v = workloads.random_attn(B, H, N, d, dt, seed=c["seed"])
    rng = np.random.default_rng(c["seed"])
    nqb, nkb = (N + 255) // 256, (N + 127) // 128
    lists = [sorted(int(x) for x in np.nonzero(rng.random(nkb) < c["p"])[0]) for _ in range(nqb)]
    ptr = np.zeros(nqb + 1, np.int32)
    ptr[1:] = np.cumsum([len(x) for x in lists])
    idx = np.asarray([x for l in lists for x in l], np.int32)
    qd, kd, vd = (to_device(t, dt) for t in (q, k, v))
    o, lse = torch.empty_like(qd), torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    entry = fa.fa_fwd_blocksparse if dt == "bf16" else fa.fa_fwd_blocksparse_f16
    entry(qd, kd, vd, o, lse, torch.from_numpy(ptr).cuda(),
          torch.from_numpy(idx).cuda() if idx.size else None, idx.size, B, H, N, d, d ** -0.5,
          int(c["causal"]))
    torch.cuda.synchronize()
    import test_parity_blocksparse as bs
    outs, refs, tols = [], [], []
    for b in range(B):
        for h in range(H):
            refs.append(orc.attention_blocksparse(q[b, h], k[b, h], v[b, h], d ** -0.5, c["causal"],
                                                  ptr, idx, 256, 128, dtype=dt))
            outs.append((to_f64(o[b, h]), to_f64(lse[b, h])))
            tols.append(bs.blocksparse_lse_tolerance(orc, q[b, h], k[b, h], np.arange(N), refs[-1][1],
                                                     d ** -0.5, c["causal"], ptr, idx, dt))
    compare(orc, f"random block-sparse {case}", outs, refs, dt, tols)


@pytest.mark.parametrize("case", range(CASES))
def test_random_decode(orc, case):
    """Split-KV attention of Nq queries at the end of Nk keys, Nq <= Nk when causal."""
    import test_parity_decode as dec
    c = draw(case + 300)
    rng = np.random.default_rng([4343, case])
    Nk = int(rng.integers(1, 20000))
    Nq = int(rng.integers(1, min(Nk, 64) + 1)) if c["causal"] else int(rng.integers(1, 64))
    B, H, d, dt = c["B"], c["H"], c["d"], c["dtype"]
    say(f"[random decode {case}] B={B} H={H} Nq={Nq} Nk={Nk} d={d} {dt} causal={c['causal']}")
    q = workloads.random_attn(B, H, Nq, d, dt, seed=c["seed"])[0]
    _, k, v = workloads.random_attn(B, H, Nk, d, dt, seed=c["seed"] + 1)
    o, lse = dec.run(q, k, v, dt, d ** -0.5, c["causal"])
    dec.check(orc, f"random decode {case}", q, k, v, dt, d ** -0.5, c["causal"], o, lse)


@pytest.mark.parametrize("case", range(CASES))
def test_random_fp8(orc, case):
    """fp8 forward with the derived E4M3 bounds of the fp8 parity tests."""
    import test_parity_fp8 as f8
    c = draw(case + 400)
    B, H, N, d = c["B"], c["H"], min(c["N"], 1200), c["d"]
    say(f"[random fp8 {case}] B={B} H={H} N={N} d={d} causal={c['causal']}")
    desc = (1 / 64, 1 / 64, 1 / 64)
    q8, k8, v8 = f8.random_fp8(B, H, N, d, seed=c["seed"] % 100000, desc=desc)
    o, lse = f8.run(q8, k8, v8, d ** -0.5, desc, c["causal"])
    f8.check(orc, f"random fp8 {case}", q8, k8, v8, d ** -0.5, desc, c["causal"], o, lse)


@pytest.mark.parametrize("case", range(CASES))
def test_random_backward(orc, case):
    """dQ, dK, dV from the oracle's O and logsumexp, with the backward tests' gates."""
    import test_parity_backward as bw
    c = draw(case + 500)
    B, H, N, d, dt = c["B"], c["H"], min(c["N"], 900), c["d"], c["dtype"]
    say(f"[random backward {case}] B={B} H={H} N={N} d={d} {dt} causal={c['causal']}")
    q, k, v = workloads.random_attn(B, H, N, d, dt, seed=c["seed"])
    g = workloads.cast(bw.upstream((B, H, N, d), c["seed"] % 1000), dt)
    o, lse = bw.oracle_forward(orc, q, k, v, dt, d ** -0.5, c["causal"])
    grads = bw.run_bwd(q, k, v, o, g, lse, dt, d ** -0.5, c["causal"])
    bw.check(orc, f"random backward {case}", q, k, v, g, dt, d ** -0.5, c["causal"], grads, o=o)


@pytest.mark.parametrize("case", range(CASES))
def test_random_softmax(orc, case):
    """Row softmax, one workgroup per row and split over workgroups, on random
    row counts, lengths, offsets (aligned or not) and spike densities."""
    import test_parity_softmax as sm
    import test_parity_softmax_split as sp
    rng = np.random.default_rng([4444, case])
    rows = int(rng.integers(1, 40))
    cols = int(rng.choice([int(rng.integers(1, 5000)), int(rng.integers(30000, 70000)),
                           int(rng.integers(100000, 400000))]))
    offset = int(rng.choice([0, 0, 1, 3]))
    x = workloads.random_rows(rows, cols, seed=int(rng.integers(0, 1 << 30)),
                              std=float(rng.uniform(0.5, 4.0)), spike_prob=float(rng.choice([0.0, 1e-3, 0.02])))
    say(f"[random softmax {case}] rows={rows} cols={cols} offset={offset}")
    ref = orc.softmax_rows(x)
    for name, got in (("rows", sm.run_gpu(x, offset)), ("split", sp.run_split(x, offset))):
        g = got.cpu().numpy().astype(np.float64)
        gate(f"random softmax {case} {name}", g, ref, "f32")
        softmax_rel_gate(f"random softmax {case} {name}", g, ref, x)
