"""The "_clk" measurement copies of the production kernels: the same C as the
production kernel bit for bit, and per-workgroup clock counters that make
sense (the bench derives the engine clock from them)."""
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
