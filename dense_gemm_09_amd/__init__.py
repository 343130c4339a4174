"""Python binding of the gemm355 C ABI (libgemm355.so).

Argument marshalling only: every step of the GEMM runs in the library's HIP
kernels. torch tensors supply device memory and the current stream. The
functions keep the C names and argument order; tensors stand in for device
pointers, and each tensor is checked to cover every byte the call will touch
(so a wrong size raises here instead of faulting on the GPU).

If the shared library is missing, every entry point raises RuntimeError: there
is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm355.so")

ROW, COL = 0, 1
OUT_F32, OUT_BF16 = 0, 1
QOUT_INT8, QOUT_E4M3 = 0, 1
ACT_NONE, ACT_RELU, ACT_GELU_ERF, ACT_GELU_TANH = 0, 1, 2, 3

STATUS = ["GEMM_OK", "GEMM_ERR_NULL_POINTER", "GEMM_ERR_BAD_DIM", "GEMM_ERR_BAD_LD",
          "GEMM_ERR_BAD_ENUM", "GEMM_ERR_UNSUPPORTED", "GEMM_ERR_WORKSPACE_TOO_SMALL",
          "GEMM_ERR_HIP"]
EXPORTS = ["gemm_bf16", "gemm_bf16_noalloc", "gemm_fp8_scaled", "gemm_mxfp8", "gemm_bf16_quant", "gemm_fp8_scaled_quant",
           "gemm_quantize_fp8_rows", "gemm_pack_b", "gemm_workspace_size", "gemm_plan",
           "gemm_status_string"]


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("workspace_bytes", ctypes.c_size_t)]


_lib = None

_I64, _F32, _P, _SZ, _I32 = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int


def lib() -> ctypes.CDLL:
    """Load libgemm355.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"gemm355 HIP library not built: {LIB_PATH} is missing "
                               "(run `python -m dense_gemm_09_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        L.gemm_bf16.restype = _I32
        L.gemm_bf16.argtypes = [_I64, _I64, _I64, _F32, _P, _I64, _I32, _P, _I64, _I32, _F32,
                                _P, _I64, _I32, _P, _I32, _P, _SZ, _P]
        L.gemm_bf16_noalloc.restype = _I32
        L.gemm_bf16_noalloc.argtypes = [_I64, _I64, _I64, _F32, _P, _I64, _I32, _P, _I64, _I32,
                                        _F32, _P, _I64, _I32, _P, _I32, _P]
        L.gemm_fp8_scaled.restype = _I32
        L.gemm_fp8_scaled.argtypes = [_I64, _I64, _I64, _F32, _P, _I64, _I32, _P, _I64, _I32,
                                      _P, _P, _F32, _P, _I64, _I32, _P, _I32, _P, _SZ, _P]
        L.gemm_mxfp8.restype = _I32
        L.gemm_mxfp8.argtypes = [_I64, _I64, _I64, _F32, _P, _I64, _I32, _P, _I64, _I32, _P, _I64,
                                 _P, _I64, _F32, _P, _I64, _I32, _P, _I32, _P, _SZ, _P]
        L.gemm_bf16_quant.restype = _I32
        L.gemm_bf16_quant.argtypes = [_I64, _I64, _I64, _F32, _P, _I64, _I32, _P, _I64, _I32,
                                      _P, _I32, _P, _P, _P, _I64, _I32, _P, _SZ, _P]
        L.gemm_fp8_scaled_quant.restype = _I32
        L.gemm_fp8_scaled_quant.argtypes = [_I64, _I64, _I64, _F32, _P, _I64, _I32, _P, _I64,
                                            _I32, _P, _P, _P, _I32, _P, _P, _P, _I64, _I32, _P,
                                            _SZ, _P]
        L.gemm_pack_b.restype = _I32
        L.gemm_pack_b.argtypes = [_I64, _I64, _P, _I64, _I32, _I32, _P, _I64, _P]
        L.gemm_quantize_fp8_rows.restype = _I32
        L.gemm_quantize_fp8_rows.argtypes = [_I64, _I64, _P, _I64, _P, _I64, _P, _P]
        L.gemm_workspace_size.restype = _SZ
        L.gemm_workspace_size.argtypes = [_I64, _I64, _I64, _I32]
        L.gemm_plan.restype = _I32
        L.gemm_plan.argtypes = [_I64, _I64, _I64, _I32, ctypes.POINTER(PlanInfo)]
        L.gemm_status_string.restype = ctypes.c_char_p
        L.gemm_status_string.argtypes = [_I32]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gemm_status_string(status).decode()


def workspace_size(M: int, N: int, K: int, is_fp8: bool) -> int:
    return int(lib().gemm_workspace_size(M, N, K, 1 if is_fp8 else 0))


def plan(M: int, N: int, K: int, is_fp8: bool) -> PlanInfo:
    info = PlanInfo()
    st = lib().gemm_plan(M, N, K, 1 if is_fp8 else 0, ctypes.byref(info))
    if st != 0:
        raise GemmError(st, "gemm_plan")
    return info


# ------------------------------------------------------------------ marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.untyped_storage().nbytes() - t.storage_offset() * t.element_size()


def _need(t, nbytes: int, what: str):
    if t is None or isinstance(t, int) or nbytes <= 0:
        return
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous (pass the leading dimension instead)")
    if _nbytes(t) < nbytes:
        raise ValueError(f"{what} holds {_nbytes(t)} bytes, the call reads/writes {nbytes}")


def _extent(rows: int, cols: int, ld: int) -> int:
    """Elements spanned by a rows x cols block stored with leading dimension ld."""
    return 0 if rows == 0 or cols == 0 else (rows - 1) * ld + cols


def _check_operands(M, N, K, A, lda, la, B, ldb, lb, C, ldc, c_dtype, esize, bias):
    if M > 0 and N > 0:
        if K > 0:
            _need(A, esize * (_extent(M, K, lda) if la == ROW else _extent(K, M, lda)), "A")
            _need(B, esize * (_extent(K, N, ldb) if lb == ROW else _extent(N, K, ldb)), "B")
        _need(C, (4 if c_dtype == OUT_F32 else 2) * _extent(M, N, ldc), "C")
        _need(bias, 2 * N, "bias")


def _stream(stream) -> int:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def gemm_bf16(M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, beta, C, ldc, c_dtype,
              bias=None, act=ACT_NONE, workspace=None, workspace_bytes=None, stream=None):
    """C = act(alpha * A B + beta * C + bias), BF16 inputs, FP32 accumulation.

    A, B, C, bias, workspace: device tensors (or raw device addresses as int).
    With workspace=None a workspace of the required size is allocated here, on
    the stream the call runs on.
    """
    L = lib()
    _check_operands(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, c_dtype, 2, bias)
    workspace, workspace_bytes = _workspace(M, N, K, False, workspace, workspace_bytes, stream)
    st = L.gemm_bf16(M, N, K, alpha, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b, beta,
                     _ptr(C), ldc, c_dtype, _ptr(bias), act, _ptr(workspace), workspace_bytes,
                     _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_bf16")


def gemm_bf16_noalloc(M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, beta, C, ldc, c_dtype,
                      bias=None, act=ACT_NONE, stream=None):
    """gemm_bf16 without a workspace: split-K partials go to the library's
    per-GPU scratch array (nothing is allocated; calls overlapping on one GPU race)."""
    L = lib()
    _check_operands(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, c_dtype, 2, bias)
    st = L.gemm_bf16_noalloc(M, N, K, alpha, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b,
                             beta, _ptr(C), ldc, c_dtype, _ptr(bias), act, _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_bf16_noalloc")


def gemm_fp8_scaled(M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, scale_a, scale_b,
                    beta, C, ldc, c_dtype, bias=None, act=ACT_NONE, workspace=None,
                    workspace_bytes=None, stream=None):
    """C = act(alpha * scale_a[m] scale_b[n] * A B + beta * C + bias), E4M3 inputs."""
    L = lib()
    _check_operands(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, c_dtype, 1, bias)
    if M > 0 and N > 0:
        _need(scale_a, 4 * M, "scale_a")
        _need(scale_b, 4 * N, "scale_b")
    workspace, workspace_bytes = _workspace(M, N, K, True, workspace, workspace_bytes, stream)
    st = L.gemm_fp8_scaled(M, N, K, alpha, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b,
                           _ptr(scale_a), _ptr(scale_b), beta, _ptr(C), ldc, c_dtype,
                           _ptr(bias), act, _ptr(workspace), workspace_bytes, _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_fp8_scaled")


def gemm_mxfp8(M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, scale_a, ldsa, scale_b, ldsb,
               beta, C, ldc, c_dtype, bias=None, act=ACT_NONE, workspace=None,
               workspace_bytes=None, stream=None):
    """C = act(alpha * sum_k a 2^(SA-127) b 2^(SB-127) + beta * C + bias): E4M3 with E8M0
    scales per 32 K elements (scale_a: M rows of ldsa bytes, scale_b: N rows of ldsb)."""
    L = lib()
    _check_operands(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, c_dtype, 1, bias)
    if M > 0 and N > 0 and K > 0:
        _need(scale_a, M * ldsa, "scale_a")
        _need(scale_b, N * ldsb, "scale_b")
    workspace, workspace_bytes = _workspace(M, N, K, True, workspace, workspace_bytes, stream)
    st = L.gemm_mxfp8(M, N, K, alpha, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b,
                      _ptr(scale_a), ldsa, _ptr(scale_b), ldsb, beta, _ptr(C), ldc, c_dtype,
                      _ptr(bias), act, _ptr(workspace), workspace_bytes, _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_mxfp8")


def _check_quant_out(M, N, Q, ldq, out_scale, out_zero):
    if M > 0 and N > 0:
        _need(Q, _extent(M, N, ldq), "Q")
        _need(out_scale, 4 * M, "out_scale")
        _need(out_zero, 4 * M, "out_zero")


def gemm_bf16_quant(M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, bias, act, out_scale,
                    out_zero, Q, ldq, q_dtype, workspace=None, workspace_bytes=None,
                    stream=None):
    """Q = quant(act(alpha * A B + bias)) per row: INT8 (scale, zero point) or E4M3 (scale)."""
    L = lib()
    _check_operands(M, N, K, A, lda, layout_a, B, ldb, layout_b, None, ldq, OUT_BF16, 2, bias)
    _check_quant_out(M, N, Q, ldq, out_scale, out_zero)
    workspace, workspace_bytes = _workspace(M, N, K, False, workspace, workspace_bytes, stream)
    st = L.gemm_bf16_quant(M, N, K, alpha, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b,
                           _ptr(bias), act, _ptr(out_scale), _ptr(out_zero), _ptr(Q), ldq,
                           q_dtype, _ptr(workspace), workspace_bytes, _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_bf16_quant")


def gemm_fp8_scaled_quant(M, N, K, alpha, A, lda, layout_a, B, ldb, layout_b, scale_a, scale_b,
                          bias, act, out_scale, out_zero, Q, ldq, q_dtype, workspace=None,
                          workspace_bytes=None, stream=None):
    """Q = quant(act(alpha * scale_a[m] scale_b[n] * A B + bias)) per row, E4M3 inputs."""
    L = lib()
    _check_operands(M, N, K, A, lda, layout_a, B, ldb, layout_b, None, ldq, OUT_BF16, 1, bias)
    _check_quant_out(M, N, Q, ldq, out_scale, out_zero)
    if M > 0 and N > 0:
        _need(scale_a, 4 * M, "scale_a")
        _need(scale_b, 4 * N, "scale_b")
    workspace, workspace_bytes = _workspace(M, N, K, True, workspace, workspace_bytes, stream)
    st = L.gemm_fp8_scaled_quant(M, N, K, alpha, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b,
                                 _ptr(scale_a), _ptr(scale_b), _ptr(bias), act, _ptr(out_scale),
                                 _ptr(out_zero), _ptr(Q), ldq, q_dtype, _ptr(workspace),
                                 workspace_bytes, _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_fp8_scaled_quant")


def pack_b(K, N, B, ldb, layout_b, elem_bytes, Bp, ldbp, stream=None):
    """One-time reorder of B (K x N) into K-major rows: Bp[n*ldbp + k] = b(k, n)."""
    L = lib()
    if K > 0 and N > 0:
        _need(B, elem_bytes * (_extent(K, N, ldb) if layout_b == ROW else _extent(N, K, ldb)), "B")
        _need(Bp, elem_bytes * _extent(N, K, ldbp), "Bp")
    st = L.gemm_pack_b(K, N, _ptr(B), ldb, layout_b, elem_bytes, _ptr(Bp), ldbp, _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_pack_b")


def quantize_fp8_rows(M, K, X, ldx, Q, ldq, scale, stream=None):
    """Per-token E4M3 quantisation of BF16 rows: scale[m] = amax/448, Q = e4m3(x / scale)."""
    L = lib()
    if M > 0 and K > 0:
        _need(X, 2 * _extent(M, K, ldx), "X")
        _need(Q, _extent(M, K, ldq), "Q")
    if M > 0:
        _need(scale, 4 * M, "scale")
    st = L.gemm_quantize_fp8_rows(M, K, _ptr(X), ldx, _ptr(Q), ldq, _ptr(scale), _stream(stream))
    if st != 0:
        raise GemmError(st, "gemm_quantize_fp8_rows")


def _torch_stream(stream):
    """The torch stream object of a call's `stream` argument (None: current)."""
    import torch
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, int):
        return torch.cuda.default_stream() if stream == 0 else torch.cuda.ExternalStream(stream)
    return stream


def _workspace(M, N, K, fp8, workspace, workspace_bytes, stream):
    if workspace is None:
        need = workspace_size(M, N, K, fp8) if M >= 0 and N >= 0 and K >= 0 else 0
        if need == 0:
            return None, 0
        import torch
        # Allocated on the stream the kernels run on: torch's caching allocator
        # then gives the block to a later allocation only in that stream's
        # order, i.e. after this call's kernels have finished with it.
        s = _torch_stream(stream)
        with torch.cuda.stream(s):
            workspace = torch.empty(need, dtype=torch.uint8, device=s.device)
        return workspace, need
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace) if not isinstance(workspace, int) else 0
    return workspace, workspace_bytes
