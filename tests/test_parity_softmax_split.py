"""Split-row softmax (several workgroups per row) on the GPU, through the C ABI,
against the fp64 oracle.

The oracle is the plain row softmax: the split path must reach the same result
up to rounding order.  Gates: max-abs <= 1e-4 (the fp32 tolerance) and, on
every element the fp32 output can hold as a normal number, relative error
<= 2e-5.  The relative bound follows from the arithmetic: the exponent
(x - m) log2(e) carries an absolute error of a few 2^-24 |x - m| (|x - m| < 100
here, so under 1e-5 relative in exp), the hardware exp2 about one ulp, and the
sum l a few dozen fp32 roundings along its reduction tree (each lane sums a
few dozen vectors, then the lane, wave, workgroup and chunk merges).

Cases: the 4 x 2^24 workload in full; rows of 1, 3 and 8 with lengths across
the chunk boundaries (4096-column chunks and the ~2048-workgroup target),
unaligned pointers and lengths that are not multiples of 4; special rows; two
calls with one workspace.
"""
import numpy as np
import pytest
import torch

import online_softmax_04_amd as fa
import oracle
import workloads
from gpu_util import gate, say, softmax_rel_gate, to_f64

pytestmark = pytest.mark.gpu

TINY = 2.0 ** -126


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


def run_split(x: np.ndarray, offset: int = 0, ws=None):
    rows, cols = x.shape
    n = rows * cols
    xb = torch.empty(n + offset, dtype=torch.float32, device="cuda")
    yb = torch.empty(n + offset, dtype=torch.float32, device="cuda")
    xd, yd = xb[offset:], yb[offset:]
    xd.copy_(torch.from_numpy(np.ascontiguousarray(x).ravel()))
    nbytes = fa.online_softmax_split_workspace_bytes(rows, cols)
    assert nbytes >= 8
    if ws is None:
        ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
    fa.online_softmax_rows_split(xd, yd, rows, cols, ws, ws.numel() * 4)
    torch.cuda.synchronize()
    return yd.view(rows, cols)


def check(name, got, ref):
    gate(name, got, ref, "f32")
    big = ref > TINY
    rel = np.abs(got[big] - ref[big]) / ref[big]
    worst = float(rel.max()) if rel.size else 0.0
    say(f"  {name}: worst relative error {worst:.3e}")
    assert worst <= 2e-5, f"{name}: relative error {worst:.3e} > 2e-5"
    assert np.max(np.abs(got.sum(axis=1) - 1.0)) < 1e-4


def test_workload(orc):
    w = workloads.SOFTMAX["softmax_split_4x16777216"]
    say(f"[softmax split workload {w.name}] rows={w.rows} cols={w.cols}")
    x = workloads.softmax_input(w, threads=4)
    got = to_f64(run_split(x))
    ref = orc.softmax_rows(x)
    check(w.name, got, ref)


@pytest.mark.parametrize("rows", [1, 3, 8])
@pytest.mark.parametrize("cols", [1, 5, 4095, 4096, 4097, 8193, 65537, 300000, (1 << 20) + 3])
@pytest.mark.parametrize("offset", [0, 1])
def test_edge(orc, rows, cols, offset):
    say(f"[softmax split edge] rows={rows} cols={cols} offset={offset}")
    x = workloads.random_rows(rows, cols, seed=cols + rows, std=3.0, spike_prob=1e-4)
    check(f"split {rows}x{cols} off={offset}", to_f64(run_split(x, offset)), orc.softmax_rows(x))


def test_many_chunks_per_row(orc):
    """One row of 2^23 + 4: 2047 chunks, so each lane of the merge runs over
    several pairs (512 lanes)."""
    x = workloads.random_rows(1, (1 << 23) + 4, seed=17, std=2.0)
    assert fa.online_softmax_split_workspace_bytes(1, x.shape[1]) // 8 > 3 * 512
    say("[softmax split] 1 x 8388612")
    check("split 1x8388612", to_f64(run_split(x)), orc.softmax_rows(x))


@pytest.mark.parametrize("cols", [7, 40000, 1 << 20])
def test_special_rows(orc, cols):
    say(f"[softmax split special rows] cols={cols}")
    x = np.zeros((4, cols), np.float32)
    x[0] = 1.5                                   # constant row -> 1/cols
    x[1] = -1e4                                  # one spike holds all the mass
    x[1, cols // 2] = 80.0
    x[2] = np.linspace(-60, 60, cols, dtype=np.float32)
    x[3] = -3e38                                 # extreme but finite
    x[3, cols - 1] = 0.0                         # the maximum in the last chunk
    got = to_f64(run_split(x))
    ref = orc.softmax_rows(x)
    gate(f"split special cols={cols}", got, ref, "f32")
    softmax_rel_gate(f"split special cols={cols}", got, ref, x)
    assert np.allclose(got[0], 1.0 / cols, rtol=1e-5, atol=0)
    assert got[1, cols // 2] == 1.0 and got[3, cols - 1] == 1.0


def test_workspace_reuse_and_determinism(orc):
    """Two calls in a row share one workspace, the second smaller; a repeat of
    the first gives identical bits."""
    a = workloads.random_rows(2, 1 << 21, seed=5, std=3.0)
    b = workloads.random_rows(1, 10001, seed=6, std=3.0)
    ws = torch.empty(fa.online_softmax_split_workspace_bytes(2, 1 << 21) // 4, dtype=torch.float32,
                     device="cuda")
    ya = run_split(a, ws=ws).clone()
    yb = run_split(b, ws=ws)
    check("split reuse a", to_f64(ya), orc.softmax_rows(a))
    check("split reuse b", to_f64(yb), orc.softmax_rows(b))
    assert torch.equal(ya, run_split(a, ws=ws))


def test_wrapper():
    x = torch.randn(2, 50000, device="cuda")
    y = fa.softmax_split(x)
    assert torch.allclose(y.sum(dim=1), torch.ones(2, device="cuda"), atol=1e-5)
    with pytest.raises(ValueError):
        fa.softmax_split(x.t())
