"""fa_decode_static -- split-KV decode with its partials in the library's static
device array, for callers that cannot allocate -- through the C ABI, against
fa_decode with a caller workspace on the same inputs.  Both run the same
kernels with the same split, so the outputs must be bit-identical.  Two calls
in a row, the second smaller than the first (the array keeps the first call's
partials), then the first shape again; and the size limit."""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import workloads
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def inputs(B, H, Nq, Nk, d, seed):
    q = workloads.random_attn(B, H, Nq, d, "bf16", seed=seed)[0]
    _, k, v = workloads.random_attn(B, H, Nk, d, "bf16", seed=seed + 1)
    return tuple(to_device(t, "bf16") for t in (q, k, v))


def both(q, k, v, causal):
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    scale = d ** -0.5
    o1, o2 = torch.empty_like(q), torch.empty_like(q)
    l1 = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    l2 = torch.empty_like(l1)
    nbytes = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    assert 0 < nbytes <= fa.DECODE_STATIC_SCRATCH_BYTES
    ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.fa_decode(q, k, v, o1, l1, ws, nbytes, B, H, Nq, Nk, d, scale, int(causal))
    fa.fa_decode_static(q, k, v, o2, l2, B, H, Nq, Nk, d, scale, int(causal))
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


def same(name, a, b):
    (o1, l1), (o2, l2) = a, b
    assert torch.isfinite(o2.float()).all() and torch.isfinite(l2).all(), f"{name}: non-finite"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"{name}: O differs"
    assert torch.equal(l1, l2), f"{name}: logsumexp differs"


def test_static_scratch_matches_workspace_entry():
    shapes = [(8, 32, 1, 32768, 128, True, 11),   # the decode workload's shape: the largest call
              (2, 3, 5, 3000, 64, True, 12),      # smaller, other head dim, several queries
              (8, 32, 1, 32768, 128, True, 11)]   # the first again after the smaller one
    for B, H, Nq, Nk, d, causal, seed in shapes:
        say(f"[decode static scratch] B={B} H={H} Nq={Nq} Nk={Nk} d={d} causal={causal} "
            f"workspace {fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d)} bytes")
        q, k, v = inputs(B, H, Nq, Nk, d, seed)
        a, b = both(q, k, v, causal)
        same(f"B{B} H{H} Nq{Nq} Nk{Nk} d{d}", a, b)


def test_static_scratch_limit():
    """Sizes whose partials exceed the array are refused before any launch."""
    B, H, Nq, Nk, d = 8, 32, 64, 65536, 128
    assert fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d) > fa.DECODE_STATIC_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, H, 2, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    lib = fa.lib()
    # k and v are never read: the call returns before any launch
    st = lib.fa_decode_static(q.data_ptr(), kv.data_ptr(), kv.data_ptr(), o.data_ptr(), None, B, H,
                              Nq, Nk, d, 0.088, 1, None)
    assert st == fa.FA_ERR_SCRATCH_LIMIT
    assert "SCRATCH" in fa.fa_status_string(st)
