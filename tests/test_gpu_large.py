"""Large operands near the addressing limits (GPU).

- A tall GEMM, M = 2^23 + 5 rows (A 2 GiB, C 1 GiB): tile-panel bases far past
  2^31 bytes, 64-bit in the kernels; checked on stratified samples (the last,
  ragged rows included) against the oracle.
- A long K, 2^20 + 40 (a K tail at the far end): FP32 accumulation over a
  million terms through the data-parallel kernel and through the automatic K
  split (one tile, many segments); every output element against the oracle.
"""
import numpy as np
import pytest

import helpers
import oracle
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(0, force=False)


def test_tall_m_64bit_panels():
    dt, M, N, K = "f16", (1 << 23) + 5, 64, 128
    block = inputs.draw((4096, K), dt, "uniform", 71)
    A = np.tile(block, ((M + 4095) // 4096, 1))[:M]  # 2 GiB; rows repeat every 4096
    Bt = inputs.draw((N, K), dt, "uniform", 72)
    C = helpers.gpu_gemm("tn", dt, A, Bt)
    r, c = inputs.stratified_samples(M, N, 73)
    r = np.concatenate([r, np.arange(M - 8, M)])        # the ragged last rows
    c = np.concatenate([c, np.arange(8) * 8])
    ref = oracle.hgemm_sampled("tn", dt, A, Bt, r, c)
    helpers.parity(C[r, c], ref, dt, "M = 2^23 + 5")
    # rows 4096 apart hold the same inputs, so equal outputs (same kernel code path)
    assert np.array_equal(C[M - 8:M], C[M - 8 - 4096 * 1000:M - 4096 * 1000])


@pytest.mark.parametrize("path", ["whole", "split"])
def test_long_k(path):
    dt, M, N, K = "bf16", 64, 64, (1 << 20) + 40
    A = inputs.draw((M, K), dt, "normal", 81)
    Bt = inputs.draw((N, K), dt, "normal", 82)
    if path == "whole":
        got = helpers.gpu_gemm("tn", dt, A, Bt)
    else:
        assert hgemm.gemm_ws_size(0, 1, M, N, K, dt) > 0  # the automatic choice splits
        got = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, A, Bt)[:, :N]
    ref = oracle.hgemm("tn", dt, A, Bt)
    helpers.parity(got, ref, dt, f"K = 2^20 + 40, {path}")
