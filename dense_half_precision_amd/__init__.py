"""MI355X-native dense half-precision GEMM (HGEMM).

``C[M,N] = A[M,K] @ Bop[K,N]`` with FP16 or BF16 inputs, FP32 accumulation
and FP16/BF16 output, in the TN (B stored N x K) and NN (B stored K x N)
layouts.  The arithmetic runs in hand-written HIP kernels for gfx950 behind
the C ABI of ``libhgemm.so`` (declared in ``include/hgemm.h``); this package
only marshals arguments to it.
"""
