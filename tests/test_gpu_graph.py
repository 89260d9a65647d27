"""The entry points under HIP graph capture (GPU).

Serving loops capture their launches once and replay them.  The library's
calls enqueue kernels only (no allocation, no memset, no synchronisation), so
a capture on PyTorch's graph stream records them.  A data-parallel call and a
K-split call (two launches and a workspace) are captured, then replayed three
times with new operand values copied into the captured buffers between the
replays, with eager work and synchronisation in between; every replay must
equal the eager result bit for bit.
"""
import numpy as np
import pytest

import helpers
from dense_half_precision_amd import hgemm, inputs

pytestmark = pytest.mark.gpu


def _replays(call, dA, dB, dC, new_operands, eager):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up outside the capture
        call(torch.cuda.current_stream().cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream().cuda_stream)
    for r, (A, B) in enumerate(new_operands):
        dA.copy_(helpers.to_dev(A))
        dB.copy_(helpers.to_dev(B))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dC.cpu().numpy().view(np.uint16).copy()
        want = eager(A, B)
        assert np.array_equal(got, want), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_graph_replay_whole_k(dt):
    import torch
    M, N, K = 1000, 776, 520
    dA = helpers.to_dev(inputs.draw((M, K), dt, "uniform", 1))
    dB = helpers.to_dev(inputs.draw((N, K), dt, "uniform", 2))
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")

    def call(stream):
        st = hgemm.hgemm_tn(M, N, K, dt, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), stream)
        assert st == hgemm.OK

    ops = [(inputs.draw((M, K), dt, "uniform", 10 + r), inputs.draw((N, K), dt, "uniform", 20 + r))
           for r in range(3)]
    _replays(call, dA, dB, dC, ops, lambda A, B: helpers.gpu_gemm("tn", dt, A, B))


def test_graph_replay_k_split():
    import torch
    dt, M, N, K = "bf16", 520, 776, 2048  # 3 x 4 tail tiles, split 4 ways
    S = 4
    ws_bytes = 12 * S * 262144
    ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
    dA = helpers.to_dev(inputs.draw((M, K), dt, "normal", 3))
    dB = helpers.to_dev(inputs.draw((K, N), dt, "normal", 4))
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")

    def call(stream):
        st = hgemm.hgemm_gemm_ws(0, 0, M, N, K, dt, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                                 dC.data_ptr(), N, ws.data_ptr(), ws_bytes, stream, split=S)
        assert st == hgemm.OK

    ops = [(inputs.draw((M, K), dt, "normal", 30 + r), inputs.draw((K, N), dt, "normal", 40 + r))
           for r in range(3)]
    _replays(call, dA, dB, dC, ops,
             lambda A, B: helpers.gpu_gemm_ws(0, 0, dt, M, N, K, A, B, 1.0, 0.0,
                                              np.zeros((M, N), np.uint16), ws_bytes, split=S))
