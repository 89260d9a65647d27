"""Parity of the K-split tail schedule (hgemm_gemm_ws) with the CPU oracle (GPU).

The tiles of the last, partial round are cut into K segments whose FP32
partial sums go to a workspace; a second kernel adds them in order and writes
C.  The oracle does not split (the split only reorders the FP32 sums), so the
parity rule applies unchanged.  Cases: every operation-flag combination on
both dtypes with a ragged K tail and alpha/beta; one K step per segment; the
data-parallel rounds plus a split tail in one call (whole output checked by a
projection, plus sampled elements); the automatic choice; determinism; a
workspace too small (the call must run unsplit, bit for bit).
The workspace is filled with NaN before each call, so that a partial sum read
before it was written shows in C.
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


def _operands(dt, opA, opB, M, N, K, seed, padA=8, padB=16):
    A = inputs.draw((M, K), dt, "uniform", 300 + seed)
    Bl = inputs.draw((K, N), dt, "uniform", 400 + seed)
    Cin = inputs.draw((M, N), dt, "uniform", 500 + seed)
    As = helpers.stored(A, opA == 1, padA, NAN[dt])
    Bs = helpers.stored(Bl, opB == 1, padB, NAN[dt])
    return As, Bs, helpers.stored(Cin, False, 8, 0x1234)


@pytest.mark.parametrize("opA", [0, 1])
@pytest.mark.parametrize("opB", [0, 1])
@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_split_flags_parity(opA, opB, dt):
    """Tail-only grid (3 x 4 tiles, ragged edges), K with a partial last step
    (K = 1000: 16 steps, the last one 40 deep), split 3 ways (5, 5, 6 steps)."""
    M, N, K = 520, 776, 1000
    As, Bs, Cs = _operands(dt, opA, opB, M, N, K, 4 * opA + 2 * opB)
    ws = 12 * 3 * 262144  # 3 x 4 tiles, 3 segments each
    for alpha, beta in [(1.0, 0.0), (1.5, -0.75)]:
        got = helpers.gpu_gemm_ws(opA, opB, dt, M, N, K, As, Bs, alpha, beta, Cs, ws, split=3)
        ref = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, alpha, beta, Cs)
        helpers.parity(got[:, :N], ref, dt, f"split3 op{opA}{opB} {dt} a={alpha} b={beta}")
        assert np.all(got[:, N:] == 0x1234), "C padding written"


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_split_one_step_per_segment(dt):
    """S equal to the number of K steps: each segment is one step, the last
    one the partial step (K = 200 = 3 * 64 + 8)."""
    M, N, K = 264, 520, 200
    As, Bs, Cs = _operands(dt, 0, 1, M, N, K, 7, 0, 0)
    got = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, As, Bs, 1.0, 0.0, Cs, 6 * 4 * 262144, split=4)
    ref = oracle.gemm(0, 1, dt, M, N, K, As, Bs, 1.0, 0.0, Cs)
    helpers.parity(got[:, :N], ref, dt, f"split=KT {dt}")


@pytest.mark.parametrize("layout,dt,split", [("tn", "f16", 4), ("nn", "bf16", 7)])
def test_split_after_whole_rounds(layout, dt, split):
    """4352 x 4352 (289 tiles: one whole round of 256, then a tail of 33
    split `split` ways) x 1024: the whole output by a projection check, and a
    stratified sample element by element."""
    M = N = 4352
    K = 1024
    opB = 1 if layout == "tn" else 0
    A = inputs.draw((M, K), dt, "normal", 41)
    B = inputs.draw((N, K) if layout == "tn" else (K, N), dt, "normal", 42)
    ws = 33 * split * 262144
    got = helpers.gpu_gemm_ws(0, opB, dt, M, N, K, A, B, 1.0, 0.0, None, ws, split=split)[:, :N]
    helpers.freivalds(got, A, B, layout, dt)
    r, c = inputs.stratified_samples(M, N, 43)
    ref = oracle.gemm_sampled(0, opB, dt, M, N, K, A, B, r, c, 1.0, 0.0)
    helpers.parity(got[r, c], ref, dt, f"dp+split {layout} {dt} S={split}")


def test_split_automatic_choice():
    """4608 x 4608 x 8192 bf16 NN: the automatic choice splits the tail (the
    library reports a workspace size); whole output by projection, sample by
    element; and the same call without a workspace (unsplit) agrees."""
    dt, M, N, K = "bf16", 4608, 4608, 8192
    assert hgemm.gemm_ws_size(0, 0, M, N, K, dt) > 0
    A = inputs.draw((M, K), dt, "normal", 51)
    B = inputs.draw((K, N), dt, "normal", 52)
    got = helpers.gpu_gemm_ws(0, 0, dt, M, N, K, A, B)[:, :N]
    helpers.freivalds(got, A, B, "nn", dt)
    r, c = inputs.stratified_samples(M, N, 53)
    ref = oracle.gemm_sampled(0, 0, dt, M, N, K, A, B, r, c, 1.0, 0.0)
    helpers.parity(got[r, c], ref, dt, "automatic split 4608^2 x 8192")
    plain = helpers.gpu_gemm_general(0, 0, dt, M, N, K, A, B)[:, :N]
    helpers.parity(got[r, c], plain[r, c], dt, "split vs unsplit")


def test_split_deterministic_and_small_workspace():
    """Two split calls give the same bits; with a workspace one byte short of
    what the automatic choice needs, the call runs unsplit and reproduces
    hgemm_gemm bit for bit."""
    dt, M, N, K = "f16", 4352, 4352, 4096
    need = hgemm.gemm_ws_size(0, 1, M, N, K, dt)
    assert need > 0
    A = inputs.draw((M, K), dt, "uniform", 61)
    Bt = inputs.draw((N, K), dt, "uniform", 62)
    g1 = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, A, Bt)
    g2 = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, A, Bt)
    assert np.array_equal(g1, g2)
    short = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, A, Bt, ws_bytes=need - 1)
    plain = helpers.gpu_gemm_general(0, 1, dt, M, N, K, A, Bt)
    assert np.array_equal(short, plain)
    r, c = inputs.stratified_samples(M, N, 63)
    ref = oracle.gemm_sampled(0, 1, dt, M, N, K, A, Bt, r, c, 1.0, 0.0)
    helpers.parity(g1[r, c], ref, dt, "automatic split 4352^2 x 4096")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_split_eight_wave_kernel(dt):
    """The 256 x 256 tile on eight waves (2 x 4 wave blocks of 128 x 64): its
    segments store partial sums in eight wave blocks, which the fixup maps
    back to C.  Forced split, whole rounds plus a tail (4352^2: 289 tiles),
    alpha/beta, K tail; sampled elements against the oracle, and the whole
    output against the four-wave kernel's split call."""
    M = N = 4352
    K = 1000
    name = f"tn_{dt}_256x256x64_w2x4"
    k8 = hgemm.kernel_index(name)
    k4 = hgemm.kernel_index(f"tn_{dt}_256x256x64")
    As, Bs, Cs = _operands(dt, 0, 1, M, N, K, 11, 0, 0)
    ws = 33 * 5 * 262144
    got = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, As, Bs, 0.75, -0.5, Cs, ws, split=5, kernel=k8)
    four = helpers.gpu_gemm_ws(0, 1, dt, M, N, K, As, Bs, 0.75, -0.5, Cs, ws, split=5, kernel=k4)
    r, c = inputs.stratified_samples(M, N, 12)
    ref = oracle.gemm_sampled(0, 1, dt, M, N, K, As, Bs, r, c, 0.75, -0.5, Cs)
    helpers.parity(got[r, c], ref, dt, f"{name} split 5")
    # same tile, same K segments, same order of the FP32 sums: the same bits
    assert np.array_equal(got, four), f"{name}: split result differs from the four-wave kernel's"
