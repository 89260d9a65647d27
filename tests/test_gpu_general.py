"""Parity of the general entry point (operation flags, leading dimensions,
alpha and beta) with the CPU oracle's general form (GPU).

Operands are stored with padded rows (the leading dimensions); C is padded
too, and its padding must come back untouched.  Every combination of the two
operation flags runs on both dtypes, ragged shapes, every kernel of the
stored-transposed-A layouts, beta == 0 with a NaN-filled C, K == 0, and the
(0, 1) / (0, 0) flags must reproduce hgemm_tn / hgemm_nn bit for bit.
"""
import numpy as np
import pytest

import helpers
import oracle
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu

NAN = {"f16": 0x7E00, "bf16": 0x7FC0}


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(0, force=False)


def _case(dt, M, N, K, seed):
    A = inputs.draw((M, K), dt, "uniform", 700 + seed)
    Bl = inputs.draw((K, N), dt, "uniform", 800 + seed)
    Cin = inputs.draw((M, N), dt, "uniform", 900 + seed)
    return A, Bl, Cin


def _check(dt, opA, opB, M, N, K, A, Bl, Cin, alpha, beta, padA, padB, padC, kernel=None,
           what=""):
    As = helpers.stored(A, opA == 1, padA, NAN[dt])
    Bs = helpers.stored(Bl, opB == 1, padB, NAN[dt])
    Cs = helpers.stored(Cin, False, padC, 0x1234)
    got = helpers.gpu_gemm_general(opA, opB, dt, M, N, K, As, Bs, alpha, beta, Cs, kernel)
    ref = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, alpha, beta, Cs)
    helpers.parity(got[:, :N], ref, dt, what or f"op{opA}{opB} {dt} {M}x{N}x{K} a={alpha} b={beta}")
    assert np.all(got[:, N:] == 0x1234), f"{what}: C padding written"


SHAPES = [(264, 200, 328), (72, 1000, 136), (520, 264, 72), (8, 8, 8)]
SCALES = [(1.0, 0.0), (0.5, 0.0), (1.5, -0.75), (-1.0, 1.0)]


@pytest.mark.parametrize("opA", [0, 1])
@pytest.mark.parametrize("opB", [0, 1])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_general_flags_parity(opA, opB, dt):
    for s, (M, N, K) in enumerate(SHAPES):
        A, Bl, Cin = _case(dt, M, N, K, s)
        for alpha, beta in SCALES:
            _check(dt, opA, opB, M, N, K, A, Bl, Cin, alpha, beta, 8 * (s % 3), 16, 8)


@pytest.mark.parametrize("opA", [0, 1])
@pytest.mark.parametrize("opB", [0, 1])
def test_general_beta_zero_does_not_read_c(opA, opB):
    dt, M, N, K = "f16", 200, 136, 264
    A, Bl, _ = _case(dt, M, N, K, 11)
    As, Bs = helpers.stored(A, opA == 1, 8, 0), helpers.stored(Bl, opB == 1, 8, 0)
    Cs = np.full((M, N + 8), NAN[dt], dtype=np.uint16)
    got = helpers.gpu_gemm_general(opA, opB, dt, M, N, K, As, Bs, 2.0, 0.0, Cs)
    ref = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, 2.0, 0.0)
    helpers.parity(got[:, :N], ref, dt, f"beta=0 op{opA}{opB}")
    assert np.all(got[:, N:] == NAN[dt])


def test_general_k_zero_scales_c():
    dt, M, N = "bf16", 40, 48
    Cin = inputs.draw((M, N), dt, "uniform", 5)
    A = np.zeros((M, 8), dtype=np.uint16)
    B = np.zeros((8, N), dtype=np.uint16)
    got = helpers.gpu_gemm_general(0, 0, dt, M, N, 0, A, B, 1.0, 0.5, helpers.stored(Cin, False, 8))
    ref = oracle.gemm(0, 0, dt, M, N, 0, A, B, 1.0, 0.5, helpers.stored(Cin, False, 8))
    assert np.array_equal(got[:, :N], ref)


def _transposed_a_kernels():
    try:
        return [k["index"] for k in hgemm.kernel_table()
                if k["layout"] in (hgemm.AT_TN, hgemm.AT_NN)]
    except ImportError:  # library not built: collected as no cases
        return []


@pytest.mark.parametrize("kernel", _transposed_a_kernels())
def test_every_transposed_a_kernel_ragged(kernel):
    k = hgemm.kernel_table()[kernel]
    dt = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    opB = 1 if k["layout"] == hgemm.AT_TN else 0
    M, N, K = 2 * k["bm"] + 8, 2 * k["bn"] + 24, 3 * k["bk"] + 40
    A, Bl, Cin = _case(dt, M, N, K, kernel)
    _check(dt, 1, opB, M, N, K, A, Bl, Cin, 1.0, 0.0, 8, 8, 8, kernel, k["name"])
    _check(dt, 1, opB, M, N, K, A, Bl, Cin, 0.75, 0.5, 16, 0, 0, kernel, k["name"] + " a/b")


@pytest.mark.parametrize("name", ["tn_f16_256x256x64", "nn_bf16_256x256x64", "tn_bf16_128x128x64",
                                  "nn_f16_64x64x64", "tn_f16_256x256x64_directepi",
                                  "ws_tn_f16_128x256x64", "ws_tn_bf16_128x256x64",
                                  "tn_f16_128x256x64", "tn_f16_256x256x64_w2x4",
                                  "tn_bf16_256x256x64_w2x4", "tn_f16_256x256x64_pp",
                                  "tn_bf16_256x256x64_pp", "tn_f16_128x128x64_ppk",
                                  "tn_bf16_128x128x64_ppk", "nn_f16_256x192x64",
                                  "nn_bf16_192x192x64"])
def test_general_form_on_tn_nn_kernels(name):
    """Leading dimensions, alpha and beta through the TN/NN kernels."""
    k = hgemm.kernel_table()[hgemm.kernel_index(name)]
    dt = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    opB = 1 if k["layout"] == hgemm.TN else 0
    M, N, K = 2 * k["bm"] + 5, 2 * k["bn"] + 24, 3 * k["bk"] + 40
    A, Bl, Cin = _case(dt, M, N, K, 50)
    _check(dt, 0, opB, M, N, K, A, Bl, Cin, -0.5, 2.0, 24, 8, 16, k["index"], name)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_flags_reproduce_tn_nn_bitwise(dt):
    M, N, K = 520, 264, 200
    A = inputs.draw((M, K), dt, "normal", 61)
    Bt = inputs.draw((N, K), dt, "normal", 62)
    tn = helpers.gpu_gemm("tn", dt, A, Bt)
    g = helpers.gpu_gemm_general(0, 1, dt, M, N, K, A, Bt)
    assert np.array_equal(g[:, :N], tn)
    Bn = np.ascontiguousarray(Bt.T)
    nn = helpers.gpu_gemm("nn", dt, A, Bn)
    g = helpers.gpu_gemm_general(0, 0, dt, M, N, K, A, Bn)
    assert np.array_equal(g[:, :N], nn)
    # a stored-transposed A gives the same sums in the same order
    g = helpers.gpu_gemm_general(1, 1, dt, M, N, K, np.ascontiguousarray(A.T), Bt)
    assert np.array_equal(g[:, :N], tn)


@pytest.mark.parametrize("opA,opB,dt", [(1, 0, "bf16"), (1, 1, "f16")])
def test_general_large_sampled(opA, opB, dt):
    """The 256 x 256 kernels of the transposed-A layouts at 2048 x 2048 x 4096
    with padded operands, on a stratified sample."""
    M, N, K = 2048, 2048, 4096
    A = inputs.draw((M, K), dt, "normal", 91)
    Bl = inputs.draw((K, N), dt, "normal", 92)
    Cin = inputs.draw((M, N), dt, "normal", 93)
    As, Bs = helpers.stored(A, opA == 1, 64, 0), helpers.stored(Bl, opB == 1, 32, 0)
    Cs = helpers.stored(Cin, False, 8, 0)
    got = helpers.gpu_gemm_general(opA, opB, dt, M, N, K, As, Bs, 1.0, -1.0, Cs)
    r, c = inputs.stratified_samples(M, N, 77)
    ref = oracle.gemm_sampled(opA, opB, dt, M, N, K, As, Bs, r, c, 1.0, -1.0, Cs)
    helpers.parity(got[r, c], ref, dt, f"large op{opA}{opB} {dt}")
