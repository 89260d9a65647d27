"""Shared test helpers: device transfer of raw 16-bit operands, calls through
the C ABI, and the parity rule.

Parity rule (for every floating-point comparison with the oracle):
    |C - ref| <= 1e-2 * (1 + |ref|)   element-wise, and
    ||C - ref||_F / ||ref||_F <= 2e-3 over the compared elements,
with C and ref decoded exactly to float64.  The GPU accumulates in FP32 and
rounds once to the output type; the oracle accumulates in FP64 and rounds
once.  The difference is one FP32 accumulation error (about K * 2^-24 *
sum|a*b| in the worst case) plus at most one output ulp from the double
rounding; for the workloads here that is well under both bounds, which still
flag any wrong, missing or misplaced tile.
"""
from __future__ import annotations

import numpy as np

ATOL_REL = 1e-2
FRO_REL = 2e-3


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def parity(got_bits: np.ndarray, ref_bits: np.ndarray, dtype: str, what: str = "") -> dict:
    """Check the parity rule; returns the error statistics."""
    c = decode(got_bits, dtype)
    r = decode(ref_bits, dtype)
    assert c.shape == r.shape, f"{what}: shapes {c.shape} vs {r.shape}"
    assert np.all(np.isfinite(c)), f"{what}: non-finite output at {np.argwhere(~np.isfinite(c))[:4]}"
    err = np.abs(c - r)
    bound = ATOL_REL * (1.0 + np.abs(r))
    bad = np.argwhere(err > bound)
    stats = dict(max_abs=float(err.max()) if err.size else 0.0,
                 max_rel=float((err / bound).max() * ATOL_REL) if err.size else 0.0)
    assert bad.size == 0, (f"{what}: {len(bad)} elements outside 1e-2*(1+|ref|); first "
                           f"{tuple(bad[0])}: got {c[tuple(bad[0])]}, ref {r[tuple(bad[0])]}")
    nr = np.linalg.norm(r)
    fro = float(np.linalg.norm(c - r) / nr) if nr > 0 else float(np.linalg.norm(c - r))
    stats["fro_rel"] = fro
    assert fro <= FRO_REL, f"{what}: relative Frobenius error {fro:.3e} > {FRO_REL}"
    return stats


def freivalds(C_bits: np.ndarray, A_bits: np.ndarray, B_bits: np.ndarray, layout: str,
              dtype: str, seed: int = 99) -> None:
    """Whole-output projection check: C x == A (Bop x) for a random +-1 x,
    in float64, with a per-row bound of 6 sqrt(N) half-ulps of max|C| plus the
    parity rule's own slack.  Flags any wrong or missing tile anywhere."""
    g = np.random.Generator(np.random.PCG64(seed))
    M, N = C_bits.shape
    x = g.choice(np.array([-1.0, 1.0]), size=N)
    C = decode(C_bits, dtype)
    # An unwritten element keeps the NaN fill of the output buffer; a NaN
    # would also make the tolerance below NaN and every comparison pass, so
    # non-finite output fails here first.
    nonfinite = np.argwhere(~np.isfinite(C))
    assert nonfinite.size == 0, (f"Freivalds check: {len(nonfinite)} non-finite output "
                                 f"elements, first at {tuple(nonfinite[0])}")
    Bv = decode(B_bits, dtype)
    y = Bv.T @ x if layout == "tn" else Bv @ x  # Bop x, length K
    del Bv
    A = decode(A_bits, dtype)
    want = A @ y
    del A
    got = C @ x
    cmax = np.abs(C).max()
    ulp_bits = 11 if dtype == "f16" else 8
    half_ulp = 2.0 ** (np.floor(np.log2(max(cmax, 1e-30))) - ulp_bits)
    tol = 6.0 * np.sqrt(N) * half_ulp + 1e-3 * np.sqrt(N) * (1.0 + cmax)
    bad = np.argwhere(np.abs(got - want) > tol)
    assert bad.size == 0, (f"Freivalds check failed on {len(bad)} rows, first row {bad[0][0]}: "
                           f"{got[bad[0][0]]} vs {want[bad[0][0]]} (tol {tol})")


# ---------------------------------------------------------------- device side
def to_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


def empty_dev(M: int, N: int, fill: int = 0x7E00):
    """Output buffer pre-filled with a NaN pattern so unwritten elements show."""
    import torch
    t = torch.empty((M, N), dtype=torch.int16, device="cuda")
    t.fill_(np.int16(np.uint16(fill).view(np.int16)))
    return t


def to_host(t) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy().view(np.uint16)


def stream_ptr() -> int:
    import torch
    return torch.cuda.current_stream().cuda_stream


def gpu_gemm(layout: str, dtype: str, A_bits: np.ndarray, B_bits: np.ndarray, kernel: int = -1,
             group_m: int = 0, xcd_remap: int = -1, dA=None, dB=None, out=None) -> np.ndarray:
    """Run the HIP path through the C ABI; returns C bits (uint16)."""
    from dense_half_precision_amd import hgemm
    M, K = A_bits.shape
    N = B_bits.shape[0] if layout == "tn" else B_bits.shape[1]
    dA = to_dev(A_bits) if dA is None else dA
    dB = to_dev(B_bits) if dB is None else dB
    dC = empty_dev(M, N) if out is None else out
    fn = hgemm.hgemm_tn_ex if layout == "tn" else hgemm.hgemm_nn_ex
    st = fn(M, N, K, dtype, dA.data_ptr(), dB.data_ptr(), dC.data_ptr(), stream_ptr(),
            kernel=kernel, group_m=group_m, xcd_remap=xcd_remap)
    assert st == hgemm.OK, (f"{layout} {dtype} {M}x{N}x{K}: status {st}, hipError_t "
                            f"{hgemm.lib().hgemm_last_hip_error()}")
    return to_host(dC)


def stored(logical: np.ndarray, transposed: bool, pad: int, fill: int = 0) -> np.ndarray:
    """A logical matrix (or its transpose) in a buffer whose rows are `pad`
    elements longer than needed; the row length is the leading dimension."""
    src = logical.T if transposed else logical
    out = np.full((src.shape[0], src.shape[1] + pad), fill, dtype=np.uint16)
    out[:, :src.shape[1]] = src
    return out


def gpu_gemm_general(opA: int, opB: int, dtype: str, M: int, N: int, K: int, A_st: np.ndarray,
                     B_st: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
                     C_st: np.ndarray | None = None, kernel: int | None = None) -> np.ndarray:
    """hgemm_gemm through the C ABI on stored operands (leading dimension =
    stored row length); returns the whole stored C.  Without C_st, C is an
    M x (N + 8) buffer of NaN patterns, so that both unwritten elements and
    writes into the padding show."""
    from dense_half_precision_amd import hgemm
    if C_st is None:
        C_st = np.full((M, N + 8), 0x7E00 if dtype == "f16" else 0x7FC0, dtype=np.uint16)
    dA, dB, dC = to_dev(A_st), to_dev(B_st), to_dev(C_st)
    st = hgemm.hgemm_gemm(opA, opB, M, N, K, dtype, alpha, dA.data_ptr(), A_st.shape[1],
                          dB.data_ptr(), B_st.shape[1], beta, dC.data_ptr(), C_st.shape[1],
                          stream_ptr(), kernel=kernel)
    assert st == hgemm.OK, (f"gemm op{opA}{opB} {dtype} {M}x{N}x{K}: status {st}, hipError_t "
                            f"{hgemm.lib().hgemm_last_hip_error()}")
    return to_host(dC)


def gpu_gemm_ws(opA: int, opB: int, dtype: str, M: int, N: int, K: int, A_st: np.ndarray,
                B_st: np.ndarray, alpha: float = 1.0, beta: float = 0.0,
                C_st: np.ndarray | None = None, ws_bytes: int | None = None, split: int = 0,
                kernel: int | None = None) -> np.ndarray:
    """hgemm_gemm_ws through the C ABI (a K split of the tail with a workspace
    of ws_bytes, by default the size hgemm_gemm_ws_size reports, at least
    16 bytes); the workspace is filled with NaN first, so that a partial sum
    read before it was written shows.  Returns the whole stored C."""
    import torch
    from dense_half_precision_amd import hgemm
    if C_st is None:
        C_st = np.full((M, N + 8), 0x7E00 if dtype == "f16" else 0x7FC0, dtype=np.uint16)
    if ws_bytes is None:
        ws_bytes = hgemm.gemm_ws_size(opA, opB, M, N, K, dtype)
    ws = torch.full((max(ws_bytes + 3, 16) // 4,), float("nan"), dtype=torch.float32,
                    device="cuda")
    dA, dB, dC = to_dev(A_st), to_dev(B_st), to_dev(C_st)
    st = hgemm.hgemm_gemm_ws(opA, opB, M, N, K, dtype, alpha, dA.data_ptr(), A_st.shape[1],
                             dB.data_ptr(), B_st.shape[1], beta, dC.data_ptr(), C_st.shape[1],
                             ws.data_ptr(), ws_bytes, stream_ptr(), kernel=kernel, split=split)
    assert st == hgemm.OK, (f"gemm_ws op{opA}{opB} {dtype} {M}x{N}x{K} split {split}: status "
                            f"{st}, hipError_t {hgemm.lib().hgemm_last_hip_error()}")
    return to_host(dC)
