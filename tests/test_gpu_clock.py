"""The "_clk" and "_ph" measurement copies of the production kernels: the
same C as the production kernel bit for bit, and per-workgroup clock counters
and per-wave main-loop phase cycles that make sense (the bench derives the
engine clock and the loop's cycle accounting from them)."""
import numpy as np
import pytest

import helpers
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,layout,dtype,shape", [
    ("tn_f16_256x256x64", "tn", "f16", (520, 776, 200)),
    ("nn_bf16_256x256x64", "nn", "bf16", (300, 512, 136)),
    ("tn_f16_128x128x64_r3", "tn", "f16", (264, 392, 1608)),
    ("tn_f16_64x64x64", "tn", "f16", (136, 200, 72)),
    ("tn_f16_256x256x64_pp", "tn", "f16", (520, 776, 200)),
    ("tn_bf16_256x256x64_pp", "tn", "bf16", (300, 512, 1000)),
])
def test_clock_copy_matches_production(name, layout, dtype, shape):
    import torch
    M, N, K = shape
    A = inputs.draw((M, K), dtype, "uniform", 11)
    B = inputs.draw((N, K) if layout == "tn" else (K, N), dtype, "uniform", 12)
    want = helpers.gpu_gemm(layout, dtype, A, B, kernel=hgemm.kernel_index(name))
    k = hgemm.kernel_index(name + "_clk")
    info = hgemm.kernel_table()[k]
    tiles = -(-M // info["bm"]) * -(-N // info["bn"])
    ts = torch.zeros((tiles, 4), dtype=torch.int64, device="cuda")
    dA, dB = helpers.to_dev(A), helpers.to_dev(B)
    dC = helpers.empty_dev(M, N)
    opB = hgemm.OP_T if layout == "tn" else hgemm.OP_N
    ldb = K if layout == "tn" else N
    args = (hgemm.OP_N, opB, M, N, K, dtype, 1.0, dA.data_ptr(), K, dB.data_ptr(), ldb, 0.0,
            dC.data_ptr(), N)
    # too small a counter buffer is refused before launch
    assert hgemm.hgemm_gemm_ws(*args, ts.data_ptr(), tiles * 32 - 1, helpers.stream_ptr(),
                               kernel=k) == hgemm.ERR_UNSUPPORTED
    st = hgemm.hgemm_gemm_ws(*args, ts.data_ptr(), tiles * 32, helpers.stream_ptr(), kernel=k)
    assert st == hgemm.OK
    assert np.array_equal(helpers.to_host(dC), want)
    t = ts.cpu().numpy()
    cyc, real = t[:, 2] - t[:, 0], t[:, 3] - t[:, 1]
    assert (cyc > 0).all() and (real > 0).all(), "every workgroup wrote increasing counters"
    mhz = cyc.sum() / real.sum() * 100.0
    assert 100.0 < mhz < 3000.0, f"engine clock {mhz:.0f} MHz out of any plausible range"


@pytest.mark.parametrize("name,layout,dtype,shape", [
    ("tn_f16_256x256x64", "tn", "f16", (520, 776, 1000)),
    ("nn_bf16_256x256x64", "nn", "bf16", (300, 512, 136)),
    ("tn_f16_128x128x64_r3", "tn", "f16", (264, 392, 1608)),
])
def test_phase_copy_matches_production(name, layout, dtype, shape):
    """The "_ph" copies: the same C as the production kernel bit for bit, and
    per-wave phase sums that add up (wait + barrier + rest of every step but
    the last stays within the loop's cycles, which also count the last
    step's cycles after its barrier)."""
    import torch
    M, N, K = shape
    A = inputs.draw((M, K), dtype, "uniform", 13)
    B = inputs.draw((N, K) if layout == "tn" else (K, N), dtype, "uniform", 14)
    want = helpers.gpu_gemm(layout, dtype, A, B, kernel=hgemm.kernel_index(name))
    k = hgemm.kernel_index(name + "_ph")
    info = hgemm.kernel_table()[k]
    tiles = -(-M // info["bm"]) * -(-N // info["bn"])
    ph = torch.zeros((tiles, 4, 16), dtype=torch.int32, device="cuda")
    dA, dB = helpers.to_dev(A), helpers.to_dev(B)
    dC = helpers.empty_dev(M, N)
    opB = hgemm.OP_T if layout == "tn" else hgemm.OP_N
    ldb = K if layout == "tn" else N
    args = (hgemm.OP_N, opB, M, N, K, dtype, 1.0, dA.data_ptr(), K, dB.data_ptr(), ldb, 0.0,
            dC.data_ptr(), N)
    assert hgemm.hgemm_gemm_ws(*args, ph.data_ptr(), tiles * 256 - 1, helpers.stream_ptr(),
                               kernel=k) == hgemm.ERR_UNSUPPORTED
    assert hgemm.hgemm_gemm_ws(*args, ph.data_ptr(), tiles * 256, helpers.stream_ptr(),
                               kernel=k) == hgemm.OK
    assert np.array_equal(helpers.to_host(dC), want)
    v = ph.cpu().numpy().astype(np.int64).reshape(-1, 16)
    kt = -(-K // 64)
    assert (v[:, 3] == kt).all()
    assert (v[:, 0:3] >= 0).all() and (v[:, 2] > 0).all()
    assert (v[:, 0] + v[:, 1] + v[:, 2] + v[:, 5] <= v[:, 4] + 64).all(), "phases exceed the loop"
    mfma_step = (info["bm"] // 32) * (info["bn"] // 32) * 2
    assert (v[:, 2] >= (kt - 1) * mfma_step * 16 * 0.9).all(), "fewer cycles than the MFMAs need"
    assert ((v[:, 6] > 0) & (v[:, 6] < 2000)).all(), "clock read round trip"
    assert (v[:, 7] > 0).all() and (v[:, 8] > 0).all(), "prologue and epilogue"
    assert (v[:, 9:] == 0).all()
