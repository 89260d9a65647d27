"""hgemm_gemm_noalloc (the K split through the library's static scratch)
against hgemm_gemm_ws with a caller workspace, through the C ABI: two calls in
a row, the second with smaller operands, each bit-identical to the workspace
call and within the parity rule of the oracle on stratified samples."""
import numpy as np
import pytest

import helpers
import oracle
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu

# (opA, opB, dtype, M, N, K, alpha, beta, pad): the first needs the whole
# scratch (64 MiB of partial sums: a tail of 32 tiles in 8 segments), the
# second less, with alpha/beta and padded leading dimensions
CALLS = [
    (hgemm.OP_N, hgemm.OP_T, "f16", 4096, 4608, 6144, 1.0, 0.0, 0),
    (hgemm.OP_N, hgemm.OP_N, "bf16", 4352, 4352, 4096, 0.75, -0.5, 8),
]


def _operands(opA, opB, dt, M, N, K, pad, seed):
    A = inputs.draw((M, K), dt, "uniform", seed)
    Bl = inputs.draw((K, N), dt, "uniform", seed + 1)
    As = helpers.stored(A, opA == hgemm.OP_T, pad)
    Bs = helpers.stored(Bl, opB == hgemm.OP_T, pad)
    Cs = helpers.stored(inputs.draw((M, N), dt, "uniform", seed + 2), False, pad)
    return As, Bs, Cs


def test_noalloc_matches_workspace_call_twice():
    import torch
    oracle.build(0, force=False)
    sp = helpers.stream_ptr()
    for i, (opA, opB, dt, M, N, K, al, be, pad) in enumerate(CALLS):
        need = hgemm.gemm_ws_size(opA, opB, M, N, K, dt)
        assert 0 < need <= hgemm.NOALLOC_SCRATCH_BYTES, (M, N, K, need)
        print(f"[noalloc] call {i}: op{opA}{opB} {dt} {M}x{N}x{K} alpha {al} beta {be} "
              f"pad {pad}, split workspace {need} bytes", flush=True)
        As, Bs, Cs = _operands(opA, opB, dt, M, N, K, pad, 5000 + 10 * i)
        # reference: the existing entry point with a NaN-filled caller workspace
        want = helpers.gpu_gemm_ws(opA, opB, dt, M, N, K, As, Bs, al, be, Cs.copy())
        dA, dB, dC = helpers.to_dev(As), helpers.to_dev(Bs), helpers.to_dev(Cs)
        st = hgemm.hgemm_gemm_noalloc(opA, opB, M, N, K, dt, al, dA.data_ptr(), As.shape[1],
                                      dB.data_ptr(), Bs.shape[1], be, dC.data_ptr(),
                                      Cs.shape[1], sp)
        assert st == hgemm.OK, (st, hgemm.lib().hgemm_last_hip_error())
        got = helpers.to_host(dC)
        assert np.array_equal(got, want), f"call {i}: differs from hgemm_gemm_ws"
        assert np.array_equal(got[:, N:], Cs[:, N:]), f"call {i}: wrote into C's padding"
        rows, cols = inputs.stratified_samples(M, N, 77 + i)
        ref = oracle.gemm_sampled(opA, opB, dt, M, N, K, As, Bs, rows, cols, al, be, Cs)
        helpers.parity(got[rows, cols], ref, dt, f"noalloc call {i}")
        del dA, dB, dC
        torch.cuda.synchronize()


def test_noalloc_unsplit_shape_matches_gemm():
    """A shape with no tail to split runs the plain kernels: bit-identical to
    hgemm_gemm, and the scratch is not touched."""
    opA, opB, dt, M, N, K = hgemm.OP_N, hgemm.OP_T, "f16", 1000, 1024, 520
    assert hgemm.gemm_ws_size(opA, opB, M, N, K, dt) == 0
    As, Bs, Cs = _operands(opA, opB, dt, M, N, K, 0, 6100)
    want = helpers.gpu_gemm_general(opA, opB, dt, M, N, K, As, Bs, C_st=Cs.copy())
    dA, dB, dC = helpers.to_dev(As), helpers.to_dev(Bs), helpers.to_dev(Cs)
    st = hgemm.hgemm_gemm_noalloc(opA, opB, M, N, K, dt, 1.0, dA.data_ptr(), K, dB.data_ptr(), K,
                                  0.0, dC.data_ptr(), N, helpers.stream_ptr())
    assert st == hgemm.OK
    assert np.array_equal(helpers.to_host(dC), want)
