"""Python binding of libblockgemm (MI355X / gfx950 GEMM library).

Argument marshalling only: every function here forwards device pointers,
sizes and the current HIP stream to the C ABI declared in include/blockgemm.h
and raises BlockGemmError on a non-OK status. All arithmetic runs in the HIP
kernels of the shared library; there is no fallback path. PyTorch provides
device memory and streams.

Importing this module fails if the library has not been built, or was built
from older sources (`python block_scaled_fp4_gemm_amd/build.py`, or
__graft_entry__.build()).
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libblockgemm.so")

_REBUILD = "python block_scaled_fp4_gemm_amd/build.py"

if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `{_REBUILD}`")

lib = ctypes.CDLL(_LIB_PATH)

_p, _u32, _f32, _sz = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "gemm_bf16": [_p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_bf16_strided": [_p, _u32, _p, _u32, _p, _u32, _u32, _u32, _u32, _p],
    "gemm_bf16_dual": [_p, _p, _p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_bf16_scaled_acc": [_p, _p, _p, _u32, _u32, _u32, _f32, _p],
    "gemm_bf16_splitk": [_p, _p, _p, _p, _sz, _u32, _u32, _u32, _u32, _p],
    "gemm_bf16_ordered": [_p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_bf16_ordered_f32": [_p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_fp4_blockscaled": [_p, _p, _p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_w4a16": [_p, _p, _p, _f32, _p, _u32, _u32, _u32, _p],
    "gemm_fp4_blockscaled_batched": [_p, _p, _p, _p, _p, _u32, _u32, _u32, _u32, _p],
    "gemm_fp4_blockscaled_splitk": [_p, _p, _p, _p, _p, _p, _sz, _u32, _u32, _u32, _u32, _p],
    "fp4_scales_from_blocked": [_p, _p, _u32, _u32, _u32, _p],
    "bf16_scaled_add": [_p, _p, _sz, _f32, _p],
}
for _name, _args in _SIGS.items():
    try:
        _fn = getattr(lib, _name)
    except AttributeError as _e:
        raise ImportError(f"{_LIB_PATH} lacks {_name} (built from older sources): rebuild it with "
                          f"`{_REBUILD}`") from _e
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
lib.gemm_bf16_splitk_workspace_bytes.argtypes = [_u32, _u32, _u32]
lib.gemm_bf16_splitk_workspace_bytes.restype = ctypes.c_size_t
lib.bg_status_string.argtypes = [ctypes.c_int]
lib.bg_status_string.restype = ctypes.c_char_p

EXPORTS = tuple(_SIGS) + ("gemm_bf16_splitk_workspace_bytes", "bg_status_string")

BG_OK, BG_ERR_NULL, BG_ERR_SHAPE, BG_ERR_ALIGN, BG_ERR_WORKSPACE, BG_ERR_ALIAS, BG_ERR_DEVICE, \
    BG_ERR_LAUNCH = range(8)


class BlockGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {bg_status_string(status)} (status {status})")


def bg_status_string(status: int) -> str:
    return lib.bg_status_string(int(status)).decode()


def gemm_bf16_splitk_workspace_bytes(m: int, n: int, k_splits: int) -> int:
    return int(lib.gemm_bf16_splitk_workspace_bytes(m, n, k_splits))


def _check(status: int, where: str) -> None:
    if status != BG_OK:
        raise BlockGemmError(status, where)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (row-major)")
    return t.data_ptr()


def _bits16(t: torch.Tensor) -> torch.Tensor:
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"expected bfloat16 (or its 16-bit pattern), got {t.dtype}")
    return t


def gemm_bf16(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """C[M,N] = bf16(A[M,K] @ B[N,K]^T), FP32 accumulation."""
    m, k = _bits16(a).shape
    n = _bits16(b).shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _check(lib.gemm_bf16(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream(stream)), "gemm_bf16")
    return out


def gemm_bf16_dual(a: torch.Tensor, b0: torch.Tensor, b1: torch.Tensor, out0: torch.Tensor | None = None,
                   out1: torch.Tensor | None = None, stream=None):
    """C0 = bf16(A @ B0^T) and C1 = bf16(A @ B1^T) (same shapes) in one launch."""
    m, k = _bits16(a).shape
    n = _bits16(b0).shape[0]
    if tuple(_bits16(b1).shape) != tuple(b0.shape):
        raise ValueError("B0 and B1 must have the same shape")
    if out0 is None:
        out0 = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if out1 is None:
        out1 = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _check(lib.gemm_bf16_dual(_ptr(a), _ptr(b0), _ptr(b1), _ptr(out0), _ptr(out1), m, n, k, _stream(stream)),
           "gemm_bf16_dual")
    return out0, out1


def _rows(t: torch.Tensor, what: str):
    """(rows, cols, row stride) of a 2-D tensor whose rows are contiguous."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{what} must be 2-D with contiguous rows")
    return t.shape[0], t.shape[1], t.stride(0) if t.shape[0] > 1 else max(t.shape[1], 1)


def gemm_bf16_strided(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor, stream=None):
    """C = bf16(A @ B^T) on row-strided views (each row contiguous, any row stride)."""
    m, k, lda = _rows(a, "A")
    n, kb, ldb = _rows(b, "B")
    mc, nc, ldc = _rows(out, "C")
    if kb != k or (mc, nc) != (m, n):
        raise ValueError("shapes must be A [M,K], B [N,K], C [M,N]")
    for t in (a, b, out):
        _bits16(t)
    _check(lib.gemm_bf16_strided(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, m, n, k,
                                 _stream(stream)), "gemm_bf16_strided")
    return out


def gemm_bf16_scaled_acc(x: torch.Tensor, b: torch.Tensor, out: torch.Tensor, scale: float,
                         stream=None):
    """out[M,N] = bf16(out + scale * bf16(X[M,K] @ B[N,K]^T)), in place."""
    m, k = _bits16(x).shape
    n = _bits16(b).shape[0]
    _check(lib.gemm_bf16_scaled_acc(_ptr(x), _ptr(b), _ptr(_bits16(out)), m, n, k, float(scale),
                                    _stream(stream)), "gemm_bf16_scaled_acc")
    return out


def gemm_bf16_splitk(a: torch.Tensor, b: torch.Tensor, k_splits: int,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     stream=None):
    """Split-K GEMM with an FP32 workspace of k_splits*M*N floats (allocated if None)."""
    m, k = _bits16(a).shape
    n = _bits16(b).shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if workspace is None and k_splits > 1:
        workspace = torch.empty((k_splits, m, n), dtype=torch.float32, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gemm_bf16_splitk(_ptr(a), _ptr(b), _ptr(out), _ptr(workspace), ws_bytes, m, n, k,
                                k_splits, _stream(stream)), "gemm_bf16_splitk")
    return out


def gemm_bf16_ordered(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                      stream=None):
    """Strict k = 0..K-1 FP32 recurrence per output (no FMA), BF16 out."""
    m, k = _bits16(a).shape
    n = _bits16(b).shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _check(lib.gemm_bf16_ordered(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream(stream)),
           "gemm_bf16_ordered")
    return out


def gemm_bf16_ordered_f32(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                          stream=None):
    """As gemm_bf16_ordered, storing the FP32 sums."""
    m, k = _bits16(a).shape
    n = _bits16(b).shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _check(lib.gemm_bf16_ordered_f32(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream(stream)),
           "gemm_bf16_ordered_f32")
    return out


def gemm_fp4_blockscaled(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                         out: torch.Tensor | None = None, stream=None):
    """C = bf16(deq(A) @ deq(B)^T): A [M,K/2] packed e2m1, SFA [M,K/16] e4m3fn, same for B."""
    for t in (a, sfa, b, sfb):
        if t.element_size() != 1:
            raise TypeError("packed FP4 operands and scales are byte tensors")
    m, kh = a.shape
    n = b.shape[0]
    k = 2 * kh
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _check(lib.gemm_fp4_blockscaled(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(out), m, n, k,
                                    _stream(stream)), "gemm_fp4_blockscaled")
    return out


def gemm_fp4_blockscaled_batched(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                 out: torch.Tensor | None = None, stream=None):
    """C[l] = bf16(deq(A[l]) @ deq(B[l])^T) for A [L,M,K/2], SFA [L,M,K/16], B [L,N,K/2], SFB [L,N,K/16]."""
    for t in (a, sfa, b, sfb):
        if t.element_size() != 1 or t.dim() != 3:
            raise TypeError("batched FP4 operands and scales are 3-D byte tensors")
    l, m, kh = a.shape
    n = b.shape[1]
    if out is None:
        out = torch.empty((l, m, n), dtype=torch.bfloat16, device=a.device)
    _check(lib.gemm_fp4_blockscaled_batched(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(out), m, n, 2 * kh, l,
                                            _stream(stream)), "gemm_fp4_blockscaled_batched")
    return out


def gemm_fp4_blockscaled_splitk(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                k_splits: int, workspace: torch.Tensor | None = None,
                                out: torch.Tensor | None = None, stream=None):
    """FP4 GEMM through k_splits FP32 planes (workspace of k_splits*M*N floats, allocated if None)."""
    m, kh = a.shape
    n = b.shape[0]
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    if workspace is None and k_splits > 1:
        workspace = torch.empty((k_splits, m, n), dtype=torch.float32, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * 4
    _check(lib.gemm_fp4_blockscaled_splitk(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(out), _ptr(workspace),
                                           ws_bytes, m, n, 2 * kh, k_splits, _stream(stream)),
           "gemm_fp4_blockscaled_splitk")
    return out


def fp4_scales_from_blocked(blocked: torch.Tensor, rows: int, k_groups: int, batch: int = 1,
                            out: torch.Tensor | None = None, stream=None):
    """Plain [batch, rows, k_groups] scale bytes from the blocked (l, tile_m, tile_k, 32, 4, 4) layout."""
    if blocked.element_size() != 1:
        raise TypeError("scales are byte tensors")
    if out is None:
        out = torch.empty((batch, rows, k_groups), dtype=torch.uint8, device=blocked.device)
    _check(lib.fp4_scales_from_blocked(_ptr(blocked), _ptr(out), rows, k_groups, batch, _stream(stream)),
           "fp4_scales_from_blocked")
    return out


def gemm_w4a16(a: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor, scale_2: float,
               out: torch.Tensor | None = None, stream=None):
    """C = bf16(scale_2 * (A @ deq(B)^T)): A [M,K] bf16, B [N,K/2] packed e2m1, SFB [N,K/16] e4m3fn."""
    for t in (b, sfb):
        if t.element_size() != 1:
            raise TypeError("packed FP4 weights and scales are byte tensors")
    m, k = _bits16(a).shape
    n = b.shape[0]
    if b.shape[1] * 2 != k:
        raise ValueError("B must be [N, K/2] bytes for A [M, K]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=a.device)
    _check(lib.gemm_w4a16(_ptr(a), _ptr(b), _ptr(sfb), float(scale_2), _ptr(out), m, n, k, _stream(stream)),
           "gemm_w4a16")
    return out


def bf16_scaled_add(out: torch.Tensor, delta: torch.Tensor, scale: float, stream=None):
    """out = bf16(out + fl32(scale * delta)) elementwise, in place."""
    if out.numel() != delta.numel():
        raise ValueError("out and delta must have the same number of elements")
    _check(lib.bf16_scaled_add(_ptr(_bits16(out)), _ptr(_bits16(delta)), out.numel(), float(scale),
                               _stream(stream)), "bf16_scaled_add")
    return out
