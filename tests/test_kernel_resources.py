"""Resources of every kernel the entry points launch, read through
fa_kernel_attributes on the GPU: the hot kernels keep their working set in
registers (no spill bytes), fit the workgroup shape they are written for, and
stay resident as planned (one 512-thread workgroup per compute unit for the
MFMA kernels).  A change that makes the compiler spill shows up here before it
shows up as a slowdown."""
import pytest

import online_softmax_04_amd as fa

pytestmark = pytest.mark.gpu

MFMA_OPS = [
    (fa.OP_FA_FWD, "fa_fwd"), (fa.OP_FA_FWD_F16, "fa_fwd_f16"), (fa.OP_FA_FWD_FP8, "fa_fwd_fp8"),
    (fa.OP_FA_FWD_BLOCKSPARSE, "fa_fwd_blocksparse"), (fa.OP_FA_FWD_LOCAL, "fa_fwd_local"),
    (fa.OP_FA_BWD_DQ, "fa_bwd dQ"),
]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("op,name", MFMA_OPS)
def test_mfma_kernels_do_not_spill(op, name, d, causal):
    if op == fa.OP_FA_FWD_LOCAL and not causal:
        pytest.skip("the window kernel is causal only")
    a = fa.kernel_attributes(op, d, causal)
    print(f"{name} d={d} causal={causal}: {a}", flush=True)
    assert a["private_bytes"] == 0, f"{name}: {a['private_bytes']} spill bytes per lane"
    assert a["threads_per_block"] == 512 and a["blocks_per_cu"] >= 1
    assert 0 < a["regs_per_lane"] <= 256 and 0 < a["lds_bytes"] <= 160 * 1024


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_dkdv_kernel_fits(d, causal):
    """The dK/dV kernel holds two head-dim accumulator sets in its 256 registers
    without spilling."""
    a = fa.kernel_attributes(fa.OP_FA_BWD_DKDV, d, causal)
    print(f"dK/dV d={d} causal={causal}: {a}", flush=True)
    assert a["private_bytes"] == 0 and a["threads_per_block"] == 512 and a["blocks_per_cu"] >= 1


@pytest.mark.parametrize("d", [64, 128])
def test_decode_and_softmax_kernels(d):
    a = fa.kernel_attributes(fa.OP_FA_DECODE, d, True)
    assert a["private_bytes"] == 0 and a["threads_per_block"] == 64 and a["blocks_per_cu"] >= 2
    s = fa.kernel_attributes(fa.OP_SOFTMAX, 32768)
    assert s["private_bytes"] == 0 and s["blocks_per_cu"] >= 2
