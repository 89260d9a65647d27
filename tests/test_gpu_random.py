"""Seeded random cases of the general entry points against the CPU oracle (GPU).

Each case draws the operation flags, dtype, a shape (ragged M; N and K
multiples of 8; M too when A is stored transposed), padded leading
dimensions, alpha/beta (including 1/0, 0/x and negative values), and the
path: the automatic choice, a table kernel of the case's layout, or a forced
K split through hgemm_gemm_ws.  Small enough that the oracle computes every
element; the C padding must come back untouched.
"""
import os

import numpy as np
import pytest

import helpers
import oracle
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu

NAN = {"f16": 0x7E00, "bf16": 0x7FC0}
# 96 cases in the suite; HGEMM_RANDOM_CASES=n runs the first n of the same
# seeded sequence (a longer campaign), HGEMM_RANDOM_START=s from case s on
N_CASES = int(os.environ.get("HGEMM_RANDOM_CASES", "96"))
FIRST_CASE = int(os.environ.get("HGEMM_RANDOM_START", "0"))


@pytest.fixture(scope="module", autouse=True)
def _oracle_built():
    oracle.build(0, force=False)


def _case(i):
    g = np.random.Generator(np.random.PCG64(0xC0FFEE + i))
    opA, opB = int(g.integers(0, 2)), int(g.integers(0, 2))
    dt = ("f16", "bf16")[int(g.integers(0, 2))]
    M = int(g.integers(1, 600))
    if opA == 1:
        M = max(8, M // 8 * 8)
    N = 8 * int(g.integers(1, 80))
    K = 8 * int(g.integers(1, 90))
    alpha, beta = [(1.0, 0.0), (0.5, 0.0), (1.0, 1.0), (-1.25, 0.5), (0.0, 2.0)][int(g.integers(0, 5))]
    pads = [8 * int(g.integers(0, 3)) for _ in range(3)]
    path = ("auto", "kernel", "split")[int(g.integers(0, 3))]
    return dict(opA=opA, opB=opB, dt=dt, M=M, N=N, K=K, alpha=alpha, beta=beta, pads=pads,
                path=path, seed=int(g.integers(0, 1 << 30)))


def _kernels_for(opA, opB, dt):
    layout = {(0, 1): hgemm.TN, (0, 0): hgemm.NN, (1, 1): hgemm.AT_TN, (1, 0): hgemm.AT_NN}[(opA, opB)]
    code = hgemm.F16 if dt == "f16" else hgemm.BF16
    # every entry but the register-staged baselines, which take packed operands,
    # alpha 1 and beta 0 only, and the "_clk" and "_ph" measurement copies,
    # which need a counter buffer (tested in test_gpu_clock.py)
    return [k for k in hgemm.kernel_table() if k["layout"] == layout and k["dtype"] == code
            and not k["name"].startswith("rs_") and not k["name"].endswith(("_clk", "_ph"))]


@pytest.mark.parametrize("i", range(FIRST_CASE, FIRST_CASE + N_CASES))
def test_random_case(i):
    c = _case(i)
    opA, opB, dt, M, N, K = c["opA"], c["opB"], c["dt"], c["M"], c["N"], c["K"]
    A = inputs.draw((M, K), dt, "uniform", c["seed"])
    Bl = inputs.draw((K, N), dt, "uniform", c["seed"] + 1)
    Cin = inputs.draw((M, N), dt, "uniform", c["seed"] + 2)
    As = helpers.stored(A, opA == 1, c["pads"][0], NAN[dt])
    Bs = helpers.stored(Bl, opB == 1, c["pads"][1], NAN[dt])
    Cs = helpers.stored(Cin, False, c["pads"][2] + 8, 0x1234)
    what = f"case {i}: {c}"
    S = min(-(-K // 64), 2 + i % 5)  # K segments of a forced split
    if c["path"] == "split" and S >= 2:
        tiles = -(-M // 256) * -(-N // 256)  # all of them the tail (fewer than 256)
        got = helpers.gpu_gemm_ws(opA, opB, dt, M, N, K, As, Bs, c["alpha"], c["beta"], Cs,
                                  tiles * S * 262144, split=S)
    elif c["path"] == "kernel":
        ks = _kernels_for(opA, opB, dt)
        k = ks[i % len(ks)]["index"]
        got = helpers.gpu_gemm_general(opA, opB, dt, M, N, K, As, Bs, c["alpha"], c["beta"], Cs, k)
    else:
        got = helpers.gpu_gemm_general(opA, opB, dt, M, N, K, As, Bs, c["alpha"], c["beta"], Cs)
    ref = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, c["alpha"], c["beta"], Cs)
    helpers.parity(got[:, :N], ref, dt, what)
    assert np.all(got[:, N:] == 0x1234), f"{what}: C padding written"
