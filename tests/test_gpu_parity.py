"""Parity of the HIP path with the CPU oracle (GPU).

* The five measured workloads at full size, in the launch configuration the
  bench times (automatic kernel choice): full output for the 512^3 and 2048^3
  cases; for the larger ones a stratified seeded sample of 4096 elements (one
  per cell of a 64 x 64 grid over C) plus a whole-output Freivalds projection.
* Ragged and degenerate shapes, every kernel of the table, exact integer
  cases, layout invariants and run-to-run determinism.
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


# ------------------------------------------------------------ full workloads
@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_workload_parity(idx):
    w = inputs.workload(idx)
    print(f"\n[parity] workload {idx}: {w.describe()}", flush=True)
    A, B = inputs.operands(w)
    C = helpers.gpu_gemm(w.layout, w.dtype, A, B)
    if w.M * w.N * w.K <= 2048 ** 3:
        ref = oracle.hgemm(w.layout, w.dtype, A, B)
        stats = helpers.parity(C, ref, w.dtype, w.name)
    else:
        rows, cols = inputs.stratified_samples(w.M, w.N, inputs.SAMPLE_SEED_BASE + idx)
        ref = oracle.hgemm_sampled(w.layout, w.dtype, A, B, rows, cols)
        stats = helpers.parity(C[rows, cols], ref, w.dtype, w.name)
        helpers.freivalds(C, A, B, w.layout, w.dtype)
    print(f"[parity] workload {idx}: {stats}", flush=True)


# ------------------------------------------------------------ ragged / edges
EDGE_SHAPES = [
    (1, 8, 8), (17, 24, 72), (300, 136, 200), (257, 264, 64), (64, 64, 8),
    (255, 248, 520), (129, 1000, 200), (1000, 1000, 72), (513, 520, 136),
]


@pytest.mark.parametrize("layout", ["tn", "nn"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_edge_shapes_auto(layout, dtype):
    w = inputs.Workload(0, layout, dtype, 0, 0, 0, "uniform")
    for s, (M, N, K) in enumerate(EDGE_SHAPES):
        A, B = inputs.operands(w, M, N, K, seed_offset=10 * s)
        C = helpers.gpu_gemm(layout, dtype, A, B)
        helpers.parity(C, oracle.hgemm(layout, dtype, A, B), dtype, f"{layout} {dtype} {M}x{N}x{K}")


def _tn_nn_kernels():
    # the "_clk" and "_ph" measurement copies need a counter buffer and have
    # tests of their own (test_gpu_clock.py)
    try:
        return [k["index"] for k in hgemm.kernel_table()
                if k["layout"] in (hgemm.TN, hgemm.NN)
                and not k["name"].endswith(("_clk", "_ph"))]
    except ImportError:  # library not built: collected as no cases
        return []


@pytest.mark.parametrize("kernel", _tn_nn_kernels())
def test_every_kernel_ragged(kernel):
    """The TN/NN entries of the table (the transposed-A ones are covered by
    the general-form tests), including the wave-specialised kernels."""
    tab = hgemm.kernel_table()
    k = tab[kernel]
    assert k["layout"] in (hgemm.TN, hgemm.NN)
    layout = "tn" if k["layout"] == hgemm.TN else "nn"
    dtype = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    w = inputs.Workload(0, layout, dtype, 0, 0, 0, "normal")
    # two tile rows/cols plus a ragged edge, and a K tail
    M, N, K = 2 * k["bm"] + 5, 2 * k["bn"] + 24, 3 * k["bk"] + 40
    A, B = inputs.operands(w, M, N, K, seed_offset=kernel)
    for gm, xcd in ((0, -1), (1, 0), (3, 1)):
        C = helpers.gpu_gemm(layout, dtype, A, B, kernel=kernel, group_m=gm, xcd_remap=xcd)
        helpers.parity(C, oracle.hgemm(layout, dtype, A, B), dtype, f"{k['name']} gm={gm} xcd={xcd}")


@pytest.mark.parametrize("name", ["tn_f16_128x128x64_r3", "nn_bf16_128x128x64_r3",
                                  "tn_bf16_64x64x64_r4", "nn_f16_64x64x64_r4"])
def test_deep_ring_k_tails(name):
    """The deeper-ring kernels (128 x 128 with four A and three B LDS stages,
    64 x 64 with five and four) load three or four steps ahead: K of one to
    six steps puts the partial last step at each of the prologue's loads and
    at the loop's, with ragged M and N."""
    k = hgemm.kernel_table()[hgemm.kernel_index(name)]
    layout = "tn" if k["layout"] == hgemm.TN else "nn"
    dtype = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    w = inputs.Workload(0, layout, dtype, 0, 0, 0, "uniform")
    for s, K in enumerate((8, 72, 136, 200, 264, 328, 64, 192)):
        M, N = 200 + s, 136 + 8 * s
        A, B = inputs.operands(w, M, N, K, seed_offset=40 + s)
        C = helpers.gpu_gemm(layout, dtype, A, B, kernel=k["index"])
        helpers.parity(C, oracle.hgemm(layout, dtype, A, B), dtype, f"{name} {M}x{N}x{K}")


@pytest.mark.parametrize("name", ["tn_f16_256x256x64_persist", "nn_bf16_256x256x64_persist"])
def test_persistent_many_tiles(name):
    """The persistent launch (one workgroup per CU looping over tiles): 4352 x
    4360 is 18 x 18 = 324 tiles, so 68 workgroups take a second tile, the last
    row and column ragged, with a K tail; whole output by projection, a
    stratified sample element by element, and the same bits as the plain
    launch of the same tile code."""
    k = hgemm.kernel_table()[hgemm.kernel_index(name)]
    layout = "tn" if k["layout"] == hgemm.TN else "nn"
    dtype = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    M, N, K = 4352 + 40, 4360, 712
    w = inputs.Workload(0, layout, dtype, 0, 0, 0, "uniform")
    A, B = inputs.operands(w, M, N, K, seed_offset=77)
    C = helpers.gpu_gemm(layout, dtype, A, B, kernel=k["index"])
    helpers.freivalds(C, A, B, layout, dtype)
    r, c = inputs.stratified_samples(M, N, 78)
    ref = oracle.hgemm_sampled(layout, dtype, A, B, r, c)
    helpers.parity(C[r, c], ref, dtype, name)
    plain = helpers.gpu_gemm(layout, dtype, A, B, kernel=hgemm.kernel_index(name[:-len("_persist")]))
    assert np.array_equal(C, plain), f"{name}: differs from the plain launch"


@pytest.mark.parametrize("name", ["tn_f16_192x256x64", "nn_bf16_192x256x64", "tn_f16_256x128x64",
                                  "nn_bf16_256x128x64", "at_tn_bf16_256x128x64",
                                  "at_nn_f16_256x128x64", "tn_bf16_256x192x64",
                                  "at_tn_f16_256x192x64", "tn_f16_192x192x64",
                                  # 192-wide m/n-contiguous operand tiles (384-byte k-rows)
                                  "nn_f16_256x192x64", "nn_bf16_256x192x64",
                                  "nn_f16_192x192x64", "nn_bf16_192x192x64",
                                  "at_tn_f16_192x256x64", "at_tn_bf16_192x256x64",
                                  "at_tn_f16_192x192x64", "at_tn_bf16_192x192x64",
                                  "at_nn_f16_192x256x64", "at_nn_bf16_192x256x64",
                                  "at_nn_f16_256x192x64", "at_nn_bf16_256x192x64",
                                  "at_nn_f16_192x192x64", "at_nn_bf16_192x192x64"])
def test_rectangular_tiles_at_scale(name):
    """The 192 x 256, 256 x 192, 192 x 192 and 256 x 128 production kernels
    on a few rounds of tiles with ragged last tile rows and columns (3000 =
    15 x 192 + 120 = 11 x 256 + 184; 3080 = 16 x 192 + 8) and a K tail: whole
    output by projection, a stratified sample element by element, and the same
    bits as the 256 x 256 kernel, which sums every element over the same K
    slices in the same order.  With an m- or n-contiguous operand 192 wide,
    a 384-byte k-row straddles the 1 KiB load segments."""
    k = hgemm.kernel_table()[hgemm.kernel_index(name)]
    layout = ("tn", "nn", "at_tn", "at_nn")[k["layout"]]
    dtype = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    M, N, K = 3000, 3080, 3112
    print(f"\n[parity] {name} {M}x{N}x{K}", flush=True)
    opA, opB = int(layout.startswith("at_")), int(layout.endswith("tn"))
    A = inputs.draw((M, K), dtype, "uniform", 91)
    Bl = inputs.draw((K, N), dtype, "uniform", 92)
    As = helpers.stored(A, opA == 1, 0, 0)
    Bs = helpers.stored(Bl, opB == 1, 0, 0)
    Cin = np.zeros((M, N), dtype=np.uint16)
    C = helpers.gpu_gemm_general(opA, opB, dtype, M, N, K, As, Bs, 1.0, 0.0, Cin, k["index"])
    square = hgemm.kernel_index(name.replace(name[-10:], "256x256x64"))
    C256 = helpers.gpu_gemm_general(opA, opB, dtype, M, N, K, As, Bs, 1.0, 0.0, Cin, square)
    assert np.array_equal(C, C256), f"{name}: differs from the 256 x 256 kernel"
    r, c = inputs.stratified_samples(M, N, 93)
    ref = oracle.gemm_sampled(opA, opB, dtype, M, N, K, As, Bs, r, c)
    helpers.parity(C[r, c], ref, dtype, name)
    helpers.freivalds(C, A, np.ascontiguousarray(Bl.T), "tn", dtype)


@pytest.mark.parametrize("name", ["tn_f16_256x256x64_pp", "tn_bf16_256x256x64_pp"])
def test_ping_pong_matches_production_bits(name):
    """The two-group kernel sums the same 32-k slices in the same order as the
    production kernel, so the two give the same bits: 3 x 3 tiles with ragged
    last rows and columns, at K that end on a slice boundary, inside a slice
    and inside a K step (and shorter than the three-slice load lead), and
    the oracle on a stratified sample of the largest."""
    k = hgemm.kernel_table()[hgemm.kernel_index(name)]
    dtype = "f16" if k["dtype"] == hgemm.F16 else "bf16"
    prod = hgemm.kernel_index(name[:-len("_pp")])
    w = inputs.Workload(0, "tn", dtype, 0, 0, 0, "uniform")
    for s, K in enumerate((8, 40, 96, 1000, 1064)):
        M, N = 3 * 256 - 37, 3 * 256 - 88
        A, B = inputs.operands(w, M, N, K, seed_offset=90 + s)
        C = helpers.gpu_gemm("tn", dtype, A, B, kernel=k["index"])
        plain = helpers.gpu_gemm("tn", dtype, A, B, kernel=prod)
        assert np.array_equal(C, plain), f"{name} K={K}: differs from the production kernel"
    r, c = inputs.stratified_samples(M, N, 95)
    helpers.parity(C[r, c], oracle.hgemm_sampled("tn", dtype, A, B, r, c), dtype, name)


@pytest.mark.parametrize("layout", ["tn", "nn"])
def test_k_zero_writes_zeros(layout):
    M, N = 40, 48
    A = np.zeros((M, 0), dtype=np.uint16)
    B = np.zeros((N, 0) if layout == "tn" else (0, N), dtype=np.uint16)
    import torch
    dA = torch.zeros(8, dtype=torch.int16, device="cuda")  # K = 0: never read
    C = helpers.gpu_gemm(layout, "f16", A, B, dA=dA, dB=dA)
    assert np.all(C == 0)


def test_empty_outputs_are_noops():
    out = helpers.empty_dev(4, 8, fill=0x1234)
    st = hgemm.hgemm_tn(0, 8, 16, "f16", 0, 0, out.data_ptr(), helpers.stream_ptr())
    assert st == hgemm.OK
    assert np.all(helpers.to_host(out) == 0x1234)


@pytest.mark.parametrize("layout", ["tn", "nn"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_small_integers_exact(layout, dtype):
    """Products and sums exact in FP32 and in the output type: C must equal
    the int64 matmul bit for bit (f16: |x| <= 2, K <= 512; bf16: |x| <= 1,
    K <= 256)."""
    g = np.random.Generator(np.random.PCG64(21))
    hi, K = (2, 512) if dtype == "f16" else (1, 256)
    for M, N in ((300, 264), (64, 1000)):
        Ai = g.integers(-hi, hi + 1, size=(M, K))
        Bi = g.integers(-hi, hi + 1, size=(K, N))
        to = (lambda v: v.astype(np.float16).view(np.uint16)) if dtype == "f16" else \
            (lambda v: inputs.f32_to_bf16_bits(v.astype(np.float32)))
        Bst = Bi.T.copy() if layout == "tn" else Bi
        C = helpers.gpu_gemm(layout, dtype, to(Ai), to(Bst))
        assert np.array_equal(C, to(Ai @ Bi))


def test_identity_and_permutation_exact():
    g = np.random.Generator(np.random.PCG64(22))
    K, N = 264, 136
    Bop = inputs.draw((K, N), "f16", "normal", 5)
    for layout in ("tn", "nn"):
        Bst = Bop.T.copy() if layout == "tn" else Bop
        eye = np.eye(K).astype(np.float16).view(np.uint16)
        assert np.array_equal(helpers.gpu_gemm(layout, "f16", eye, Bst), Bop)
        perm = g.permutation(K)
        P = np.zeros((K, K))
        P[np.arange(K), perm] = 1.0
        assert np.array_equal(helpers.gpu_gemm(layout, "f16", P.astype(np.float16).view(np.uint16),
                                               Bst), Bop[perm])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_layout_invariants(dtype):
    """TN(A, Bt) == NN(A, Bt^T) and TN(A, Bt)^T == TN(Bt, A) within parity;
    the TN/NN pair shares the inner loop, so it is also bit-identical."""
    M, N, K = 392, 520, 328
    A = inputs.draw((M, K), dtype, "uniform", 61)
    Bt = inputs.draw((N, K), dtype, "uniform", 62)
    tn = helpers.gpu_gemm("tn", dtype, A, Bt)
    nn = helpers.gpu_gemm("nn", dtype, A, Bt.T.copy())
    assert np.array_equal(tn, nn)
    tr = helpers.gpu_gemm("tn", dtype, Bt, A)
    helpers.parity(tn.T, tr, dtype, "transpose")


def test_determinism_and_streams():
    """Same inputs give bit-identical C across repeats, launch orders and
    streams (no atomics, no split-K): a tripwire for races."""
    import torch
    w = inputs.workload(3)
    A, B = inputs.operands(w, 2048, 2048, 1024)
    dA, dB = helpers.to_dev(A), helpers.to_dev(B)
    first = helpers.gpu_gemm("nn", "bf16", A, B, dA=dA, dB=dB)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [helpers.empty_dev(2048, 2048) for _ in range(4)]
    # the NaN fills above run on the current stream: the two side streams wait
    # for them before the GEMMs overwrite the outputs
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for i, o in enumerate(outs):
        s = s1 if i % 2 == 0 else s2
        st = hgemm.hgemm_nn(2048, 2048, 1024, "bf16", dA.data_ptr(), dB.data_ptr(), o.data_ptr(),
                            s.cuda_stream)
        assert st == hgemm.OK
    torch.cuda.synchronize()
    for o in outs:
        assert np.array_equal(helpers.to_host(o), first)
