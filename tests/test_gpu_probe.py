"""GPU unit tests of the building blocks the kernels rest on: the MFMA
operand/accumulator lane map and the LDS store/read addressing."""
import numpy as np
import pytest

import helpers
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu


def _bits(vals, dtype):
    v = np.asarray(vals, dtype=np.float64)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return inputs.f32_to_bf16_bits(v.astype(np.float32))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mfma_lane_map(dtype):
    """Lane l holds X[l%32][8*(l//32)+e] and Y[8*(l//32)+e][l%32]; accumulator
    r of lane l is D[8*(r//4) + 4*(l//32) + r%4][l%32].  Small integers keep
    every product and sum exact, so the comparison is bit-exact."""
    import torch
    g = np.random.Generator(np.random.PCG64(3))
    X = g.integers(-3, 4, size=(32, 16))
    Y = g.integers(-3, 4, size=(16, 32))
    D = X @ Y
    lane = np.arange(64)
    e = np.arange(8)
    xl = X[(lane % 32)[:, None], (8 * (lane // 32))[:, None] + e[None, :]]
    yl = Y[(8 * (lane // 32))[:, None] + e[None, :], (lane % 32)[:, None]]
    dx, dy = helpers.to_dev(_bits(xl, dtype)), helpers.to_dev(_bits(yl, dtype))
    dd = torch.full((64, 16), float("nan"), dtype=torch.float32, device="cuda")
    st = hgemm.probe_mfma(dtype, dx.data_ptr(), dy.data_ptr(), dd.data_ptr(), helpers.stream_ptr())
    assert st == hgemm.OK
    got = dd.cpu().numpy()
    r = np.arange(16)
    want = D[8 * (r[None, :] // 4) + 4 * (lane[:, None] // 32) + r[None, :] % 4, (lane % 32)[:, None]]
    assert np.array_equal(got, want.astype(np.float32))


def test_mfma_k_order_is_shared():
    """Only the pairing of X and Y elements along k matters to a GEMM: a
    one-hot k in X must meet the same k in Y (probe each of the 16 k)."""
    import torch
    for k in range(16):
        X = np.zeros((32, 16))
        Y = np.zeros((16, 32))
        X[:, k] = 1.0
        Y[k, :] = 2.0
        lane = np.arange(64)
        e = np.arange(8)
        xl = X[(lane % 32)[:, None], (8 * (lane // 32))[:, None] + e[None, :]]
        yl = Y[(8 * (lane // 32))[:, None] + e[None, :], (lane % 32)[:, None]]
        dx, dy = helpers.to_dev(_bits(xl, "f16")), helpers.to_dev(_bits(yl, "f16"))
        dd = torch.zeros((64, 16), dtype=torch.float32, device="cuda")
        assert hgemm.probe_mfma("f16", dx.data_ptr(), dy.data_ptr(), dd.data_ptr(),
                                helpers.stream_ptr()) == hgemm.OK
        assert np.all(dd.cpu().numpy() == 2.0), f"k={k}"


@pytest.mark.parametrize("layout", [hgemm.LDS_XOR, hgemm.LDS_PLAIN, hgemm.LDS_PAD, hgemm.LDS_XOR_ROW])
def test_lds_roundtrip(layout):
    import torch
    src = np.random.Generator(np.random.PCG64(4)).integers(0, 65536, size=(256, 64)).astype(np.uint16)
    ds = helpers.to_dev(src)
    dd = torch.zeros((256, 64), dtype=torch.int16, device="cuda")
    assert hgemm.probe_lds_roundtrip(layout, ds.data_ptr(), dd.data_ptr(),
                                     helpers.stream_ptr()) == hgemm.OK
    assert np.array_equal(helpers.to_host(dd), src)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mfma16_lane_map(dtype):
    """16x16x32 (the production shape): lane l holds X[l%16][8*(l//16)+e] and
    Y[8*(l//16)+e][l%16]; accumulator r of lane l is D[4*(l//16) + r][l%16].
    Small integers keep every product and sum exact."""
    import torch
    g = np.random.Generator(np.random.PCG64(5))
    X = g.integers(-3, 4, size=(16, 32))
    Y = g.integers(-3, 4, size=(32, 16))
    D = X @ Y
    lane = np.arange(64)
    e = np.arange(8)
    xl = X[(lane % 16)[:, None], (8 * (lane // 16))[:, None] + e[None, :]]
    yl = Y[(8 * (lane // 16))[:, None] + e[None, :], (lane % 16)[:, None]]
    dx, dy = helpers.to_dev(_bits(xl, dtype)), helpers.to_dev(_bits(yl, dtype))
    dd = torch.full((64, 4), float("nan"), dtype=torch.float32, device="cuda")
    assert hgemm.probe_mfma16(dtype, dx.data_ptr(), dy.data_ptr(), dd.data_ptr(),
                              helpers.stream_ptr()) == hgemm.OK
    r = np.arange(4)
    want = D[4 * (lane[:, None] // 16) + r[None, :], (lane % 16)[:, None]]
    assert np.array_equal(dd.cpu().numpy(), want.astype(np.float32))


@pytest.mark.parametrize("mn_major", [0, 1])
@pytest.mark.parametrize("bx", [64, 128, 192, 256])
def test_operand_fragments(mn_major, bx):
    """One K step through the production path (direct-to-LDS placement, XOR
    layout, 16-byte or transposing fragment reads) delivers exactly the
    matrix-core operand: lane l of fragment f, slice sl holds tile element
    (16f + l%16, 32sl + 8(l//16) + e).  Random bit patterns, padded rows."""
    import torch
    tile = np.random.Generator(np.random.PCG64(6 + bx + mn_major)).integers(
        0, 65536, size=(bx, 64)).astype(np.uint16)
    src = helpers.stored(tile, bool(mn_major), 16, 0xFFFF)
    dsrc = helpers.to_dev(src)
    dd = torch.zeros((bx // 16, 2, 64, 8), dtype=torch.int16, device="cuda")
    assert hgemm.probe_fragments(mn_major, bx, dsrc.data_ptr(), src.shape[1], dd.data_ptr(),
                                 helpers.stream_ptr()) == hgemm.OK
    got = helpers.to_host(dd)
    lane, e = np.arange(64), np.arange(8)
    for f in range(bx // 16):
        for sl in range(2):
            want = tile[(16 * f + lane % 16)[:, None], (32 * sl + 8 * (lane // 16))[:, None] + e]
            assert np.array_equal(got[f, sl], want), (f, sl)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("random", [0, 1])
def test_mfma_rate_probe_runs(shape, random):
    """The issue-rate probe launches and its sums and clocks are sane (the
    throughput itself is measured by the bench's microbenchmark mode)."""
    import torch
    waves = 8
    out = torch.full((waves * 64,), float("nan"), device="cuda")
    clk = torch.zeros(2 * waves, dtype=torch.int64, device="cuda")
    assert hgemm.lib().hgemm_probe_mfma_rate(shape, random, waves, 8, out.data_ptr(),
                                             clk.data_ptr(), helpers.stream_ptr()) == hgemm.OK
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    c = clk.cpu().numpy().reshape(-1, 2)
    assert (c[:, 0] > 0).all() and (c[:, 1] > 0).all()


@pytest.mark.parametrize("pattern", range(9))
def test_lds_read_probe_runs(pattern):
    import torch
    out = torch.full((2 * 256,), float("nan"), device="cuda")
    assert hgemm.lib().hgemm_probe_lds_read(2, 3, pattern, out.data_ptr(),
                                            helpers.stream_ptr()) == hgemm.OK
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("mode", range(6))
def test_l2_read_probe_runs(mode):
    import torch
    window = 1 << 20
    buf = torch.zeros(window, dtype=torch.uint8, device="cuda")
    out = torch.full((2 * 256,), float("nan"), device="cuda")
    assert hgemm.lib().hgemm_probe_l2_read(2, 3, mode, buf.data_ptr(), window, 16384,
                                           out.data_ptr(), helpers.stream_ptr()) == hgemm.OK
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


def test_lds_lanes_probe_runs():
    import torch
    offs = torch.tensor([16 * ((7 * l) % 64) for l in range(64)], dtype=torch.int32, device="cuda")
    out = torch.full((2 * 256,), float("nan"), device="cuda")
    assert hgemm.lib().hgemm_probe_lds_lanes(2, 3, offs.data_ptr(), out.data_ptr(),
                                             helpers.stream_ptr()) == hgemm.OK
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
