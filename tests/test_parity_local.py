"""Causal attention with a sliding window and packed-document starts
(fa_fwd_local) on the GPU, through the C ABI, against the fp64 oracle's
explicit key ranges: query i sees keys max(doc start, i - window + 1) .. i.
Gates are the stated ones (bf16 / fp16: max-abs 1e-2, relative L2 5e-3); the
logsumexp takes the bound derived from its arithmetic (gpu_util.lse_tolerance)
over each row's visible keys."""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import oracle
import workloads
from gpu_util import TORCH_DTYPE, gate, gate_lse, lse_tolerance, range_vis, same_but_order, say, to_device, to_f64

pytestmark = pytest.mark.gpu

ENTRY = {"bf16": fa.fa_fwd_local, "f16": fa.fa_fwd_local_f16}


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def run_local(q, k, v, doc, window, dtype, scale):
    B, H, N, d = q.shape
    qd, kd, vd = (to_device(t, dtype) for t in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    docd = None if doc is None else torch.from_numpy(np.ascontiguousarray(doc, np.int32)).cuda()
    ENTRY[dtype](qd, kd, vd, o, lse, docd, window, B, H, N, d, scale)
    torch.cuda.synchronize()
    return o, lse


def check(orc, name, q, k, v, doc, window, dtype, scale, o, lse, rows_of=None, heads=None):
    B, H, N, d = q.shape
    go, ro, gl, rl, lb, ls = [], [], [], [], [], []
    for b, h in heads or [(b, h) for b in range(B) for h in range(H)]:
        lo, hi = workloads.local_ranges(np.zeros(N, np.int64) if doc is None else doc[b], window)
        rows = np.arange(N) if rows_of is None else rows_of(b, h)
        oo, ll = orc.attention_ranged(q[b, h], k[b, h], v[b, h], scale, lo, hi, rows, dtype=dtype)
        rt = torch.from_numpy(rows).cuda()
        go.append(to_f64(o[b, h].index_select(0, rt)))
        gl.append(to_f64(lse[b, h].index_select(0, rt)))
        ro.append(oo)
        rl.append(ll)
        bd, sg = lse_tolerance(orc.to_f64(q[b, h], dtype)[rows], orc.to_f64(k[b, h], dtype), ll, scale,
                               dtype, range_vis(rows, lo, hi, N))
        lb.append(bd)
        ls.append(sg)
    gate(f"{name} O", np.concatenate(go), np.concatenate(ro), dtype)
    gate_lse(f"{name} LSE", np.concatenate(gl), np.concatenate(rl), np.concatenate(lb), np.concatenate(ls))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,window,docs", [
    (1, 1, False), (65, 1, False), (300, 7, False), (300, 64, False), (1000, 100, False),
    (1000, 0, True), (1000, 129, True), (777, 256, True), (2000, 300, True),
])
def test_local_shapes(orc, dtype, d, N, window, docs):
    B, H = 2, 2
    say(f"[attention local] dtype={dtype} d={d} N={N} window={window} docs={docs}")
    q, k, v = workloads.random_attn(B, H, N, d, dtype, seed=N + window + d)
    doc = workloads.packed_doc_starts(B, N, seed=N + window, min_len=1, max_len=max(2, N // 3)) if docs else None
    scale = 1.0 / np.sqrt(d)
    o, lse = run_local(q, k, v, doc, window, dtype, scale)
    check(orc, f"local {dtype} d{d} N{N} w{window} docs{int(docs)}", q, k, v, doc, window, dtype,
          scale, o, lse)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [0, 100])
def test_local_unordered_document_starts(orc, d, window):
    """doc_start holds any int per position, not only the starts of packed
    documents: seeded values from -50 to N + 50, in no order (so a wave's
    smallest and largest lo_i sit at arbitrary lanes), clamped to 0 .. i as the
    contract states."""
    B, H, N = 2, 2, 1000
    say(f"[attention local] unordered doc starts d={d} window={window}")
    q, k, v = workloads.random_attn(B, H, N, d, "bf16", seed=911 + d + window)
    rng = np.random.default_rng([workloads.BASE_SEED + 950, d, window])
    doc = rng.integers(-50, N + 50, size=(B, N)).astype(np.int32)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_local(q, k, v, doc, window, "bf16", scale)
    check(orc, f"local unordered d{d} w{window}", q, k, v, doc, window, "bf16", scale, o, lse)


def test_local_without_masks_is_causal():
    """window 0 and no documents: the same keys as fa_fwd with causal = 1, in its
    order (the same bits) except on the rows fa_fwd walks downwards."""
    q, k, v = workloads.random_attn(1, 3, 700, 128, "bf16", seed=41)
    o1, l1 = run_local(q, k, v, None, 0, "bf16", 0.0884)
    qd, kd, vd = (to_device(t, "bf16") for t in (q, k, v))
    o2 = torch.empty_like(qd)
    l2 = torch.empty((1, 3, 700), dtype=torch.float32, device="cuda")
    fa.fa_fwd(qd, kd, vd, o2, l2, 1, 3, 700, 128, 0.0884, 1)
    torch.cuda.synchronize()
    same_but_order("window 0", o1, l1, o2, l2, 700, True, float(np.abs(workloads.bf16_bits_to_f32(v)).max()))


def test_local_headline_shape(orc):
    """B8 H32 N8192 d128 with a 1024-key window over packed documents of 512-4096
    tokens, in its full launch; 256 seeded rows per head of four heads checked."""
    lw = workloads.LOCAL_WORKLOAD
    w = workloads.ATTN[lw["base"]]
    say(f"[attention local] {lw['name']}")
    q, k, v = workloads.attn_full(w, threads=16)
    doc = workloads.packed_doc_starts(w.B, w.N, lw["doc_seed"], lw["doc_min"], lw["doc_max"])
    o, lse = run_local(q, k, v, doc, lw["window"], "bf16", w.sm_scale)
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    check(orc, lw["name"], q, k, v, doc, lw["window"], "bf16", w.sm_scale, o, lse,
          rows_of=lambda b, h: workloads.attn_sample_rows(w, b, h),
          heads=[(0, 0), (3, 17), (5, 2), (7, 31)])
