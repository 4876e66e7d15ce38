"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph): the library
allocates nothing and enqueues only kernels on the caller's stream, so a capture
replays the same work.  Each replay is compared bit for bit with the eager result,
with eager work and synchronisations between the replays."""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import workloads
from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def test_forward_softmax_decode_in_a_graph():
    q, k, v = (to_device(t, "bf16") for t in workloads.random_attn(2, 4, 1000, 128, "bf16", seed=31))
    qd = to_device(workloads.random_attn(2, 4, 2, 128, "bf16", seed=32)[0], "bf16")
    x = torch.from_numpy(workloads.random_rows(64, 5000, seed=33, std=3.0)).cuda()
    xs = torch.from_numpy(workloads.random_rows(2, 300000, seed=34, std=3.0)).cuda()
    o, lse = torch.empty_like(q), torch.empty(2, 4, 1000, device="cuda")
    od, lsed = torch.empty_like(qd), torch.empty(2, 4, 2, device="cuda")
    y, ys = torch.empty_like(x), torch.empty_like(xs)
    ws_d = torch.empty(fa.fa_decode_workspace_bytes(2, 4, 2, 1000, 128) // 4, device="cuda")
    ws_s = torch.empty(fa.online_softmax_split_workspace_bytes(2, 300000) // 4, device="cuda")

    def work(stream):
        fa.fa_fwd(q, k, v, o, lse, 2, 4, 1000, 128, 0.0884, 1, stream)
        fa.online_softmax_rows(x, y, 64, 5000, stream)
        fa.fa_decode(qd, k, v, od, lsed, ws_d, ws_d.numel() * 4, 2, 4, 2, 1000, 128, 0.0884, 1, stream)
        fa.online_softmax_rows_split(xs, ys, 2, 300000, ws_s, ws_s.numel() * 4, stream)

    work(None)
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, y, od, lsed, ys)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        work(s)  # warm up on the side stream before capture
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        work(s)
    for rep in range(4):
        for t in (o, lse, y, od, lsed, ys):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("O", "LSE", "softmax", "decode O", "decode LSE", "split softmax"),
                                  (o, lse, y, od, lsed, ys), eager):
            assert torch.equal(got, ref), f"replay {rep}: {name} differs from the eager result"
        # eager work between replays on the default stream
        _ = (x * 2).sum().item()
    say("[graph] 4 replays equal the eager results")


def test_masked_fp8_and_backward_in_a_graph():
    """The window, block-sparse, fp8 and backward entries replayed from one graph."""
    B, H, N, d = 1, 3, 700, 128
    q, k, v = (to_device(t, "bf16") for t in workloads.random_attn(B, H, N, d, "bf16", seed=41))
    g_out = to_device(workloads.random_attn(B, H, N, d, "bf16", seed=42)[0], "bf16")
    doc = torch.from_numpy(workloads.packed_doc_starts(B, N, 3, 50, 300)).cuda()
    ptr, idx = (torch.from_numpy(a).cuda() for a in workloads.block_sparse_pattern(N, 5, p_random=0.3))
    q8, k8, v8 = (torch.from_numpy(workloads.cast(t / (1 / 64), "fp8")).cuda()
                  for t in workloads.random_attn(B, H, N, d, "f32", seed=43))
    outs = {name: (torch.empty_like(q), torch.empty(B, H, N, device="cuda"))
            for name in ("local", "sparse", "fp8", "dense")}
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, H, N) // 4, device="cuda")

    def work(stream):
        fa.fa_fwd_local(q, k, v, *outs["local"], doc, 128, B, H, N, d, 0.0884, stream)
        fa.fa_fwd_blocksparse(q, k, v, *outs["sparse"], ptr, idx, idx.numel(), B, H, N, d, 0.0884, 1,
                              stream)
        fa.fa_fwd_fp8(q8, k8, v8, *outs["fp8"], B, H, N, d, 0.0884, 1 / 64, 1 / 64, 1 / 64, 1, stream)
        fa.fa_fwd(q, k, v, *outs["dense"], B, H, N, d, 0.0884, 1, stream)
        fa.fa_bwd(q, k, v, outs["dense"][0], g_out, outs["dense"][1], dq, dk, dv, ws, B, H, N, d,
                  0.0884, 1, stream)

    results = [t for pair in outs.values() for t in pair] + [dq, dk, dv]
    work(None)
    torch.cuda.synchronize()
    eager = [t.clone() for t in results]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        work(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        work(s)
    for rep in range(4):
        for t in results:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(results, eager)):
            assert torch.equal(got, ref), f"replay {rep}: output {i} differs from the eager result"
        _ = (q.float() * 2).sum().item()
    say("[graph] masked, fp8 and backward: 4 replays equal the eager results")
