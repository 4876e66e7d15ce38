"""The matrix-unit probe the benchmark times beside the attention forward
(fa_mfma_stream), checked exactly: with small-integer bf16 operands every product
and sum is exact in fp32, so each thread's output (the sum of its four
accumulators) is known from the operand fragments and the 32x32x16 operand and
accumulator layouts that tests/test_layout_probe.py pins on the GPU."""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
from gpu_util import say

pytestmark = pytest.mark.gpu

VARIANTS, FRAGS = 16, 16


def expected(ops: np.ndarray, blocks: int, iters: int) -> np.ndarray:
    """ops [VARIANTS, 64 lanes, FRAGS, 8] float64; out [blocks * 512] float64.

    A wave w uses variant w % 16: fragments 0..7 are its A operands a[k], 8..15 its
    B operands b[k]; each iteration adds a[k] b[(3k + 1) % 8] into accumulator k % 4.
    In the 32x32x16 layout lane l holds A row l % 32 and B column l % 32 at
    k = 8 (l // 32) .. + 7, and accumulator column l % 32, rows
    8 (r // 4) + 4 (l // 32) + r % 4 for r = 0..15."""
    lanes = np.arange(64)
    rows_of_lane = np.array([[8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)] for l in lanes])
    out = np.zeros(blocks * 512)
    per_variant = []
    for v in range(VARIANTS):
        total = np.zeros((32, 32))
        for k in range(8):
            a, b = ops[v, :, k], ops[v, :, 8 + (3 * k + 1) % 8]
            amat = np.zeros((32, 16))
            bmat = np.zeros((16, 32))
            for l in lanes:
                amat[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = a[l]
                bmat[8 * (l // 32):8 * (l // 32) + 8, l % 32] = b[l]
            total += amat @ bmat
        # four accumulators each get two of the products; their element sums add up to
        # the sum over all eight products of each lane's 16 entries
        per_lane = np.array([total[rows_of_lane[l], l % 32].sum() for l in lanes]) * iters
        per_variant.append(per_lane)
    for wave in range(blocks * 8):
        out[wave * 64:(wave + 1) * 64] = per_variant[wave % VARIANTS]
    return out


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 5)])
def test_mfma_stream_is_exact(blocks, iters):
    say(f"[mfma stream] blocks={blocks} iters={iters}")
    rng = np.random.default_rng(blocks * 100 + iters)
    vals = rng.integers(-3, 4, size=(VARIANTS, 64, FRAGS, 8)).astype(np.float32)
    ops = torch.from_numpy(vals.ravel()).to(torch.bfloat16).cuda()   # small integers: exact
    assert ops.numel() * 2 == fa.MFMA_STREAM_OPERAND_BYTES
    out = torch.full((blocks * 512 + 64,), 7.0, dtype=torch.float32, device="cuda")
    fa.fa_mfma_stream(ops, out[: blocks * 512], blocks, iters)
    torch.cuda.synchronize()
    got = out[: blocks * 512].cpu().numpy().astype(np.float64)
    want = expected(vals.astype(np.float64), blocks, iters)
    assert np.array_equal(got, want), f"max diff {np.max(np.abs(got - want))}"
    assert torch.all(out[blocks * 512:] == 7.0)
