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
