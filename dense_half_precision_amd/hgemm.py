"""Thin Python binding of libhgemm.so (the C ABI in include/hgemm.h).

Only argument marshalling happens here; every step of the GEMM runs in the
library's HIP kernels.  Importing this module does not need a GPU, but the
library must be built (``__graft_entry__.build()``); there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libhgemm.so")
HEADERS = [os.path.join(ROOT, "include", h) for h in ("hgemm.h", "hgemm_probe.h")]

F16, BF16 = 0, 1
TN, NN, AT_TN, AT_NN = 0, 1, 2, 3  # kernel layouts (hgemm_kernel_info)
OP_N, OP_T = 0, 1                  # operation flags of hgemm_gemm
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_SCRATCH = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20  # HGEMM_NOALLOC_SCRATCH_BYTES
DTYPE_CODES = {"f16": F16, "fp16": F16, "float16": F16, "bf16": BF16, "bfloat16": BF16}
LDS_XOR, LDS_PLAIN, LDS_PAD, LDS_XOR_ROW = 0, 1, 2, 3


class HgemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().hgemm_status_string(status).decode()
        if status == ERR_HIP:
            msg += f" (hipError_t {_lib().hgemm_last_hip_error()})"
        super().__init__(f"{where}: {msg}")


class Config(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("xcd_remap", ctypes.c_int32), ("split", ctypes.c_int32)]


_LIB = None


def _lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    # PyTorch ships its own copy of the HIP runtime under the same soname.  Load
    # it first, so that this library binds to the runtime that owns torch's
    # device memory and streams; loaded the other way round the process ends
    # up with two runtimes and the second one finds no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    gemm = [i64, i64, i64, i32, vp, vp, vp, vp]
    for name in ("hgemm_tn", "hgemm_nn"):
        getattr(lib, name).argtypes = gemm
        getattr(lib, name).restype = i32
    for name in ("hgemm_tn_ex", "hgemm_nn_ex"):
        getattr(lib, name).argtypes = gemm + [ctypes.POINTER(Config)]
        getattr(lib, name).restype = i32
    f32 = ctypes.c_float
    general = [i32, i32, i64, i64, i64, i32, f32, vp, i64, vp, i64, f32, vp, i64, vp]
    lib.hgemm_gemm.argtypes = general
    lib.hgemm_gemm.restype = i32
    lib.hgemm_gemm_ex.argtypes = general + [ctypes.POINTER(Config)]
    lib.hgemm_gemm_ex.restype = i32
    ws = general[:-1] + [vp, ctypes.c_size_t, vp]
    lib.hgemm_gemm_ws.argtypes = ws
    lib.hgemm_gemm_ws.restype = i32
    lib.hgemm_gemm_ws_ex.argtypes = ws + [ctypes.POINTER(Config)]
    lib.hgemm_gemm_ws_ex.restype = i32
    lib.hgemm_gemm_noalloc.argtypes = general
    lib.hgemm_gemm_noalloc.restype = i32
    lib.hgemm_gemm_ws_size.argtypes = [i32, i32, i64, i64, i64, i32]
    lib.hgemm_gemm_ws_size.restype = ctypes.c_size_t
    lib.hgemm_status_string.argtypes = [i32]
    lib.hgemm_status_string.restype = ctypes.c_char_p
    lib.hgemm_last_hip_error.restype = i32
    lib.hgemm_version.restype = ctypes.c_char_p
    lib.hgemm_kernel_count.restype = i32
    lib.hgemm_kernel_info.argtypes = [i32, ip, ip, ip, ip, ip]
    lib.hgemm_kernel_info.restype = ctypes.c_char_p
    lib.hgemm_auto_kernel.argtypes = [i32, i32, i64, i64, i64]
    lib.hgemm_auto_kernel.restype = i32
    lib.hgemm_probe_mfma.argtypes = [i32, vp, vp, vp, vp]
    lib.hgemm_probe_mfma.restype = i32
    lib.hgemm_probe_mfma16.argtypes = [i32, vp, vp, vp, vp]
    lib.hgemm_probe_mfma16.restype = i32
    lib.hgemm_probe_fragments.argtypes = [i32, i32, vp, i64, vp, vp]
    lib.hgemm_probe_fragments.restype = i32
    lib.hgemm_probe_operand_offsets.argtypes = [i32, i32, ip, ip, ip]
    lib.hgemm_probe_operand_offsets.restype = i32
    lib.hgemm_probe_lds_roundtrip.argtypes = [i32, vp, vp, vp]
    lib.hgemm_probe_lds_roundtrip.restype = i32
    lib.hgemm_probe_mfma_peak.argtypes = [i32, i32, vp, vp, vp]
    lib.hgemm_probe_mfma_peak.restype = i32
    lib.hgemm_probe_mfma_rate.argtypes = [i32, i32, i32, i32, vp, vp, vp]
    lib.hgemm_probe_mfma_rate.restype = i32
    lib.hgemm_probe_lds_read.argtypes = [i32, i32, i32, vp, vp]
    lib.hgemm_probe_lds_read.restype = i32
    lib.hgemm_probe_lds_lanes.argtypes = [i32, i32, vp, vp, vp]
    lib.hgemm_probe_lds_lanes.restype = i32
    lib.hgemm_probe_l2_read.argtypes = [i32, i32, i32, vp, ctypes.c_uint32, ctypes.c_uint32, vp, vp]
    lib.hgemm_probe_l2_read.restype = i32
    lib.hgemm_probe_mix.argtypes = [i32, i32, i32, i32, i32, vp, ctypes.c_uint32, vp, vp, vp]
    lib.hgemm_probe_mix.restype = i32
    lib.hgemm_probe_lds_offsets.argtypes = [i32, i32, ip]
    lib.hgemm_probe_lds_offsets.restype = i32
    lib.hgemm_probe_tile_order.argtypes = [i32, i32, i32, i32, ip, ip]
    lib.hgemm_probe_tile_order.restype = i32
    _LIB = lib
    return lib


def lib() -> ctypes.CDLL:
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _lib()


def declared_functions() -> list[str]:
    """Names of the functions declared in include/*.h."""
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"\b(hgemm_\w+)\s*\(", text)
    return sorted(set(names))


def _dt(dtype) -> int:
    return dtype if isinstance(dtype, int) else DTYPE_CODES[str(dtype).lower()]


def _check(status: int, where: str) -> None:
    if status != OK:
        raise HgemmError(status, where)


# --- raw C-ABI calls (pointers as ints) --------------------------------------
def hgemm_tn(M, N, K, dtype, A, Bt, C, stream=0) -> int:
    return _lib().hgemm_tn(M, N, K, _dt(dtype), A, Bt, C, stream)


def hgemm_nn(M, N, K, dtype, A, B, C, stream=0) -> int:
    return _lib().hgemm_nn(M, N, K, _dt(dtype), A, B, C, stream)


def hgemm_tn_ex(M, N, K, dtype, A, Bt, C, stream=0, kernel=-1, group_m=0, xcd_remap=-1) -> int:
    cfg = Config(kernel, group_m, xcd_remap, 0)
    return _lib().hgemm_tn_ex(M, N, K, _dt(dtype), A, Bt, C, stream, ctypes.byref(cfg))


def hgemm_nn_ex(M, N, K, dtype, A, B, C, stream=0, kernel=-1, group_m=0, xcd_remap=-1) -> int:
    cfg = Config(kernel, group_m, xcd_remap, 0)
    return _lib().hgemm_nn_ex(M, N, K, _dt(dtype), A, B, C, stream, ctypes.byref(cfg))


def hgemm_gemm(opA, opB, M, N, K, dtype, alpha, A, lda, B, ldb, beta, C, ldc, stream=0,
               kernel=None, group_m=0, xcd_remap=-1) -> int:
    """General form (see include/hgemm.h); with `kernel` set, hgemm_gemm_ex."""
    args = (opA, opB, M, N, K, _dt(dtype), float(alpha), A, lda, B, ldb, float(beta), C, ldc,
            stream)
    if kernel is None and group_m == 0 and xcd_remap == -1:
        return _lib().hgemm_gemm(*args)
    cfg = Config(-1 if kernel is None else kernel, group_m, xcd_remap, 0)
    return _lib().hgemm_gemm_ex(*args, ctypes.byref(cfg))


def hgemm_gemm_ws(opA, opB, M, N, K, dtype, alpha, A, lda, B, ldb, beta, C, ldc, workspace,
                  ws_bytes, stream=0, kernel=None, group_m=0, xcd_remap=-1, split=0) -> int:
    """General form with a workspace for the K split of the tail (see
    include/hgemm.h); with any option set, hgemm_gemm_ws_ex."""
    args = (opA, opB, M, N, K, _dt(dtype), float(alpha), A, lda, B, ldb, float(beta), C, ldc,
            workspace, ws_bytes, stream)
    if kernel is None and group_m == 0 and xcd_remap == -1 and split == 0:
        return _lib().hgemm_gemm_ws(*args)
    cfg = Config(-1 if kernel is None else kernel, group_m, xcd_remap, split)
    return _lib().hgemm_gemm_ws_ex(*args, ctypes.byref(cfg))


def hgemm_gemm_noalloc(opA, opB, M, N, K, dtype, alpha, A, lda, B, ldb, beta, C, ldc,
                       stream=0) -> int:
    """General form with the K split's partial sums in the library's static
    scratch: no allocation, no workspace (see include/hgemm.h)."""
    return _lib().hgemm_gemm_noalloc(opA, opB, M, N, K, _dt(dtype), float(alpha), A, lda, B, ldb,
                                     float(beta), C, ldc, stream)


def gemm_ws_size(opA, opB, M, N, K, dtype) -> int:
    return _lib().hgemm_gemm_ws_size(opA, opB, M, N, K, _dt(dtype))


def kernel_table() -> list[dict]:
    out = []
    for i in range(_lib().hgemm_kernel_count()):
        v = [ctypes.c_int() for _ in range(5)]
        name = _lib().hgemm_kernel_info(i, *[ctypes.byref(x) for x in v])
        out.append(dict(index=i, name=name.decode(), layout=v[0].value, dtype=v[1].value,
                        bm=v[2].value, bn=v[3].value, bk=v[4].value))
    return out


def kernel_index(name: str) -> int:
    for k in kernel_table():
        if k["name"] == name:
            return k["index"]
    raise KeyError(name)


def auto_kernel(layout, dtype, M, N, K) -> int:
    return _lib().hgemm_auto_kernel(layout, _dt(dtype), M, N, K)


# --- torch convenience (device memory and streams only) ----------------------
def _torch_dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}; use float16 or bfloat16")


def _stream_ptr(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def matmul_tn(A, Bt, out=None, stream=None, **cfg):
    """C = A @ Bt.T for CUDA tensors A[M,K], Bt[N,K] (row-major, same dtype)."""
    import torch
    if A.dim() != 2 or Bt.dim() != 2 or A.shape[1] != Bt.shape[1]:
        raise ValueError(f"bad shapes {tuple(A.shape)} x {tuple(Bt.shape)}^T")
    if A.dtype != Bt.dtype or not (A.is_cuda and Bt.is_cuda):
        raise TypeError("A and Bt must be CUDA tensors of one dtype")
    if not (A.is_contiguous() and Bt.is_contiguous()):
        raise ValueError("A and Bt must be contiguous (row-major)")
    M, K = A.shape
    N = Bt.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != A.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of the input dtype")
    dt = _torch_dtype_code(A)
    sp = _stream_ptr(stream)
    if cfg:
        st = hgemm_tn_ex(M, N, K, dt, A.data_ptr(), Bt.data_ptr(), out.data_ptr(), sp, **cfg)
    else:
        st = hgemm_tn(M, N, K, dt, A.data_ptr(), Bt.data_ptr(), out.data_ptr(), sp)
    _check(st, "hgemm_tn")
    return out


def matmul_nn(A, B, out=None, stream=None, **cfg):
    """C = A @ B for CUDA tensors A[M,K], B[K,N] (row-major, same dtype)."""
    import torch
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"bad shapes {tuple(A.shape)} x {tuple(B.shape)}")
    if A.dtype != B.dtype or not (A.is_cuda and B.is_cuda):
        raise TypeError("A and B must be CUDA tensors of one dtype")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    M, K = A.shape
    N = B.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif out.shape != (M, N) or out.dtype != A.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous [M, N] tensor of the input dtype")
    dt = _torch_dtype_code(A)
    sp = _stream_ptr(stream)
    if cfg:
        st = hgemm_nn_ex(M, N, K, dt, A.data_ptr(), B.data_ptr(), out.data_ptr(), sp, **cfg)
    else:
        st = hgemm_nn(M, N, K, dt, A.data_ptr(), B.data_ptr(), out.data_ptr(), sp)
    _check(st, "hgemm_nn")
    return out


def gemm(A, B, C=None, alpha=1.0, beta=0.0, transA=False, transB=False, stream=None,
         workspace=None, **cfg):
    """C = alpha * op(A) @ op(B) + beta * C for 2-D CUDA tensors of one dtype.

    op(X) is X, or X.T when the trans flag is set (the tensor then holds the
    operand stored transposed).  Rows may be strided (leading dimension =
    stride(0)); columns must be contiguous.  With beta == 0, C (if given) is
    only written.  `workspace` (a contiguous CUDA tensor, gemm_ws_size bytes
    or more) allows the K split of the tail tiles.
    """
    import torch
    for name, t in (("A", A), ("B", B)):
        if t.dim() != 2 or not t.is_cuda or t.stride(1) != 1:
            raise ValueError(f"{name} must be a 2-D CUDA tensor with contiguous rows")
    M, K = (A.shape[1], A.shape[0]) if transA else (A.shape[0], A.shape[1])
    K2, N = (B.shape[1], B.shape[0]) if transB else (B.shape[0], B.shape[1])
    if K2 != K:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have one dtype")
    if C is None:
        if beta != 0:
            raise ValueError("beta != 0 needs C")
        C = torch.empty((M, N), dtype=A.dtype, device=A.device)
    elif C.shape != (M, N) or C.dtype != A.dtype or C.stride(1) != 1:
        raise ValueError("C must be [M, N] of the input dtype with contiguous rows")
    opA, opB = OP_T if transA else OP_N, OP_T if transB else OP_N
    args = (opA, opB, M, N, K, _torch_dtype_code(A), alpha, A.data_ptr(), A.stride(0),
            B.data_ptr(), B.stride(0), beta, C.data_ptr(), C.stride(0))
    if workspace is None:
        st = hgemm_gemm(*args, _stream_ptr(stream), **cfg)
        _check(st, "hgemm_gemm")
    else:
        if not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous CUDA tensor")
        nbytes = workspace.numel() * workspace.element_size()
        st = hgemm_gemm_ws(*args, workspace.data_ptr(), nbytes, _stream_ptr(stream), **cfg)
        _check(st, "hgemm_gemm_ws")
    return C


def probe_mfma(dtype, x_ptr, y_ptr, d_ptr, stream=0) -> int:
    return _lib().hgemm_probe_mfma(_dt(dtype), x_ptr, y_ptr, d_ptr, stream)


def probe_mfma16(dtype, x_ptr, y_ptr, d_ptr, stream=0) -> int:
    return _lib().hgemm_probe_mfma16(_dt(dtype), x_ptr, y_ptr, d_ptr, stream)


def probe_fragments(mn_major, bx, src_ptr, ld, dst_ptr, stream=0) -> int:
    return _lib().hgemm_probe_fragments(mn_major, bx, src_ptr, ld, dst_ptr, stream)


def probe_lds_roundtrip(lds_layout, src_ptr, dst_ptr, stream=0) -> int:
    return _lib().hgemm_probe_lds_roundtrip(lds_layout, src_ptr, dst_ptr, stream)


def tile_order(tiles_m, tiles_n, group_m, xcd_remap):
    """(tm, tn) lists: the tile each workgroup id computes (host-side code)."""
    total = tiles_m * tiles_n
    tm = (ctypes.c_int * total)()
    tn = (ctypes.c_int * total)()
    _check(_lib().hgemm_probe_tile_order(tiles_m, tiles_n, group_m, xcd_remap, tm, tn),
           "hgemm_probe_tile_order")
    return list(tm), list(tn)


def operand_offsets(mn_major: int, bx: int):
    """The production kernels' LDS placement of one operand K step (host-side
    code): (load_row, load_chunk) per [segment][lane], read_off per
    [fragment][slice][read][lane]."""
    import numpy as np
    reads = 2 if mn_major else 1
    lr = (ctypes.c_int * (bx // 8 * 64))()
    lc = (ctypes.c_int * (bx // 8 * 64))()
    ro = (ctypes.c_int * (bx // 16 * 2 * reads * 64))()
    _check(_lib().hgemm_probe_operand_offsets(mn_major, bx, lr, lc, ro),
           "hgemm_probe_operand_offsets")
    return (np.array(lr).reshape(bx // 8, 64), np.array(lc).reshape(bx // 8, 64),
            np.array(ro).reshape(bx // 16, 2, reads, 64))


def lds_offsets(lds_layout, rows=256):
    """offsets[r][c]: byte offset of chunk c of tile row r in an LDS stage."""
    buf = (ctypes.c_int * (rows * 8))()
    _check(_lib().hgemm_probe_lds_offsets(lds_layout, rows, buf), "hgemm_probe_lds_offsets")
    return [list(buf[r * 8:(r + 1) * 8]) for r in range(rows)]
