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
    "gemm_bf16_splitk_noalloc": [_p, _p, _p, _u32, _u32, _u32, _u32, _p],
    "gemm_bf16_streamk": [_p, _p, _p, _p, _sz, _u32, _u32, _u32, _p],
    "gemm_bf16_streamk_workspace": [_u32, _u32, _u32, _p],
    "bg_streamk_plan": [_u32, _u32, _u32, _p, _sz, _p],
    "gemm_bf16_ordered": [_p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_bf16_ordered_f32": [_p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_fp4_blockscaled": [_p, _p, _p, _p, _p, _u32, _u32, _u32, _p],
    "gemm_w4a16": [_p, _p, _p, _f32, _p, _u32, _u32, _u32, _p],
    "gemm_w4a16_t": [_p, _p, _p, _u32, _f32, _p, _u32, _u32, _u32, _p],
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
lib.bg_tune_set.argtypes = [ctypes.c_int, ctypes.c_int]
lib.bg_tune_set.restype = ctypes.c_int
lib.bg_tune_get.argtypes = [ctypes.c_int]
lib.bg_tune_get.restype = ctypes.c_int
lib.bg_tile_map.argtypes = [ctypes.c_int, _u32, _u32, _p, _p]
lib.bg_tile_map.restype = ctypes.c_int

EXPORTS = tuple(_SIGS) + ("gemm_bf16_splitk_workspace_bytes", "bg_status_string", "bg_tune_set", "bg_tune_get",
                          "bg_tile_map")

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


# ---------------------------------------------------------------------------
# Argument checks. The C ABI sees only pointers and sizes, so everything it
# cannot see is checked here, before the library is called: tensor kind,
# element size, shape (including outputs the caller supplies), contiguity and
# that every tensor lives on the current HIP device. A failed check raises and
# launches nothing.
# ---------------------------------------------------------------------------

def _tensor(t, what: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor, got {type(t).__name__}")
    return t


def _bits16(t: torch.Tensor, what: str = "tensor") -> torch.Tensor:
    _tensor(t, what)
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{what}: expected bfloat16 (or its 16-bit pattern), got {t.dtype}")
    return t


def _bytes(t: torch.Tensor, what: str) -> torch.Tensor:
    _tensor(t, what)
    if t.element_size() != 1 or t.dtype == torch.bool:
        raise TypeError(f"{what}: expected a byte tensor (uint8, int8 or an FP8 dtype), got {t.dtype}")
    return t


def _f32(t: torch.Tensor, what: str) -> torch.Tensor:
    _tensor(t, what)
    if t.dtype != torch.float32:
        raise TypeError(f"{what}: expected float32, got {t.dtype}")
    return t


def _shape(t: torch.Tensor, shape, what: str) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _dims(t: torch.Tensor, n: int, what: str):
    if t.dim() != n:
        raise ValueError(f"{what} must be {n}-D, got shape {tuple(t.shape)}")
    return tuple(t.shape)


# torch's raw accessors for the current device and stream (the public
# torch.cuda.current_stream() builds a Stream object per call: about 3 us of a
# 10 us call on MI355X), with the public API as the fallback
_raw_device = getattr(torch._C, "_cuda_getDevice", None)
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _current_device() -> int:
    return _raw_device() if _raw_device is not None else torch.cuda.current_device()


def _on_device(*ts) -> None:
    """Every tensor (None skipped) is on the current HIP device (contiguity is
    checked where its pointer is taken, in _ptr)."""
    ts = [t for t in ts if t is not None]
    for t in ts:
        if not t.is_cuda:
            raise ValueError(f"tensors must be on a HIP device, got one on {t.device}")
    cur = _current_device()
    for t in ts:
        if t.get_device() != cur:
            raise ValueError(f"tensors must be on the current device cuda:{cur}, got one on {t.device}")


def _stream(stream) -> int | None:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(_current_device())
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (row-major)")
    return t.data_ptr()


def _out16(out, shape, like: torch.Tensor, what: str = "out") -> torch.Tensor:
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=like.device)
    _shape(_bits16(out, what), shape, what)
    return out


def _workspace(ws, k_splits: int, m: int, n: int):
    if ws is None:
        return None
    _f32(ws, "workspace")
    if ws.numel() < k_splits * m * n:
        raise ValueError(f"workspace holds {ws.numel()} floats, {k_splits * m * n} needed")
    return ws


def _fp4_operands(a, sfa, b, sfb, batched: bool = False):
    """Shapes of packed FP4 operands: A [(L,) M, K/2], SFA [(L,) M, K/16], B and SFB likewise."""
    nd = 3 if batched else 2
    for t, w in ((a, "A"), (sfa, "SFA"), (b, "B"), (sfb, "SFB")):
        _dims(_bytes(t, w), nd, w)
    lead = a.shape[:-2]
    m, kh = a.shape[-2:]
    n = b.shape[-2]
    k = 2 * kh
    if k % 16 != 0:
        raise ValueError(f"K = {k} must be a multiple of 16 (one scale per 16 elements)")
    _shape(b, (*lead, n, kh), "B")
    _shape(sfa, (*lead, m, k // 16), "SFA")
    _shape(sfb, (*lead, n, k // 16), "SFB")
    return lead, m, n, k


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------

def gemm_bf16(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    """C[M,N] = bf16(A[M,K] @ B[N,K]^T), FP32 accumulation."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    out = _out16(out, (m, n), a)
    _on_device(a, b, out)
    _check(lib.gemm_bf16(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream(stream)), "gemm_bf16")
    return out


def gemm_bf16_dual(a: torch.Tensor, b0: torch.Tensor, b1: torch.Tensor, out0: torch.Tensor | None = None,
                   out1: torch.Tensor | None = None, stream=None):
    """C0 = bf16(A @ B0^T) and C1 = bf16(A @ B1^T) (same shapes) in one launch."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b0, "B0"), 2, "B0")
    _shape(b0, (n, k), "B0")
    _shape(_bits16(b1, "B1"), (n, k), "B1")
    out0 = _out16(out0, (m, n), a, "out0")
    out1 = _out16(out1, (m, n), a, "out1")
    _on_device(a, b0, b1, out0, out1)
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
    for t, w in ((a, "A"), (b, "B"), (out, "C")):
        _bits16(t, w)
    m, k, lda = _rows(a, "A")
    n, kb, ldb = _rows(b, "B")
    mc, nc, ldc = _rows(out, "C")
    if kb != k or (mc, nc) != (m, n):
        raise ValueError("shapes must be A [M,K], B [N,K], C [M,N]")
    _on_device(a, b, out)
    _check(lib.gemm_bf16_strided(a.data_ptr(), lda, b.data_ptr(), ldb, out.data_ptr(), ldc, m, n, k,
                                 _stream(stream)), "gemm_bf16_strided")
    return out


def gemm_bf16_scaled_acc(x: torch.Tensor, b: torch.Tensor, out: torch.Tensor, scale: float,
                         stream=None):
    """out[M,N] = bf16(out + scale * bf16(X[M,K] @ B[N,K]^T)), in place."""
    m, k = _dims(_bits16(x, "X"), 2, "X")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    _shape(_bits16(out, "out"), (m, n), "out")
    _on_device(x, b, out)
    _check(lib.gemm_bf16_scaled_acc(_ptr(x), _ptr(b), _ptr(out), m, n, k, float(scale),
                                    _stream(stream)), "gemm_bf16_scaled_acc")
    return out


def gemm_bf16_splitk(a: torch.Tensor, b: torch.Tensor, k_splits: int,
                     workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     stream=None):
    """Split-K GEMM with an FP32 workspace of k_splits*M*N floats (allocated if None)."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    out = _out16(out, (m, n), a)
    workspace = _workspace(workspace, k_splits, m, n)
    _on_device(a, b, out, workspace)
    if workspace is None and k_splits > 1:
        workspace = torch.empty((k_splits, m, n), dtype=torch.float32, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * 4
    _check(lib.gemm_bf16_splitk(_ptr(a), _ptr(b), _ptr(out), _ptr(workspace), ws_bytes, m, n, k,
                                k_splits, _stream(stream)), "gemm_bf16_splitk")
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # BG_NOALLOC_SCRATCH_BYTES


def gemm_bf16_splitk_noalloc(a: torch.Tensor, b: torch.Tensor, k_splits: int, out: torch.Tensor,
                             stream=None):
    """Split-K GEMM whose FP32 planes live in the library's static per-device
    scratch (k_splits*M*N*4 <= NOALLOC_SCRATCH_BYTES); allocates nothing, so
    `out` must be supplied. Calls that may overlap on one device race."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    if out is None:
        raise ValueError("gemm_bf16_splitk_noalloc allocates nothing: pass `out`")
    _shape(_bits16(out, "out"), (m, n), "out")
    _on_device(a, b, out)
    _check(lib.gemm_bf16_splitk_noalloc(_ptr(a), _ptr(b), _ptr(out), m, n, k, k_splits, _stream(stream)),
           "gemm_bf16_splitk_noalloc")
    return out


def gemm_bf16_streamk_workspace(m: int, n: int, k: int) -> int:
    """Bytes of workspace gemm_bf16_streamk needs for (M, N, K) on the current device."""
    nbytes = ctypes.c_size_t(0)
    _check(lib.gemm_bf16_streamk_workspace(m, n, k, ctypes.byref(nbytes)), "gemm_bf16_streamk_workspace")
    return int(nbytes.value)


def gemm_bf16_streamk(a: torch.Tensor, b: torch.Tensor, workspace: torch.Tensor | None = None,
                      out: torch.Tensor | None = None, stream=None):
    """C = bf16(A @ B^T) with the stream-K schedule. `workspace` is a byte
    tensor of at least gemm_bf16_streamk_workspace(M, N, K) bytes (allocated
    if None); it needs no initialization."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    out = _out16(out, (m, n), a)
    _on_device(a, b, out, workspace)
    if workspace is None:
        need = gemm_bf16_streamk_workspace(m, n, k) if m and n else 0
        workspace = torch.empty(need, dtype=torch.uint8, device=a.device) if need else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.gemm_bf16_streamk(_ptr(a), _ptr(b), _ptr(out), _ptr(workspace), ws_bytes, m, n, k,
                                 _stream(stream)), "gemm_bf16_streamk")
    return out


def streamk_plan(tiles: int, steps: int, wgs_per_xcd: int):
    """The stream-K plan (host only): an int32 array of rows (workgroup, grid
    tile, first step, end step, partial, lowest source or -1), one per piece
    of work, in the order the kernel runs them."""
    import numpy as np
    count = ctypes.c_size_t(0)
    _check(lib.bg_streamk_plan(tiles, steps, wgs_per_xcd, None, 0, ctypes.byref(count)), "bg_streamk_plan")
    rows = np.zeros((count.value, 6), np.int32)
    _check(lib.bg_streamk_plan(tiles, steps, wgs_per_xcd, rows.ctypes.data if count.value else None,
                               count.value, ctypes.byref(count)), "bg_streamk_plan")
    return rows


def gemm_bf16_ordered(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                      stream=None):
    """Strict k = 0..K-1 FP32 recurrence per output (no FMA), BF16 out."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    out = _out16(out, (m, n), a)
    _on_device(a, b, out)
    _check(lib.gemm_bf16_ordered(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream(stream)),
           "gemm_bf16_ordered")
    return out


def gemm_bf16_ordered_f32(a: torch.Tensor, b: torch.Tensor, out: torch.Tensor | None = None,
                          stream=None):
    """As gemm_bf16_ordered, storing the FP32 sums."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bits16(b, "B"), 2, "B")
    _shape(b, (n, k), "B")
    if out is None:
        out = torch.empty((m, n), dtype=torch.float32, device=a.device)
    _shape(_f32(out, "out"), (m, n), "out")
    _on_device(a, b, out)
    _check(lib.gemm_bf16_ordered_f32(_ptr(a), _ptr(b), _ptr(out), m, n, k, _stream(stream)),
           "gemm_bf16_ordered_f32")
    return out


def gemm_fp4_blockscaled(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                         out: torch.Tensor | None = None, stream=None):
    """C = bf16(deq(A) @ deq(B)^T): A [M,K/2] packed e2m1, SFA [M,K/16] e4m3fn, same for B."""
    _, m, n, k = _fp4_operands(a, sfa, b, sfb)
    out = _out16(out, (m, n), a)
    _on_device(a, sfa, b, sfb, out)
    _check(lib.gemm_fp4_blockscaled(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(out), m, n, k,
                                    _stream(stream)), "gemm_fp4_blockscaled")
    return out


def gemm_fp4_blockscaled_batched(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                 out: torch.Tensor | None = None, stream=None):
    """C[l] = bf16(deq(A[l]) @ deq(B[l])^T) for A [L,M,K/2], SFA [L,M,K/16], B [L,N,K/2], SFB [L,N,K/16]."""
    (l,), m, n, k = _fp4_operands(a, sfa, b, sfb, batched=True)
    out = _out16(out, (l, m, n), a)
    _on_device(a, sfa, b, sfb, out)
    _check(lib.gemm_fp4_blockscaled_batched(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(out), m, n, k, l,
                                            _stream(stream)), "gemm_fp4_blockscaled_batched")
    return out


def gemm_fp4_blockscaled_splitk(a: torch.Tensor, sfa: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor,
                                k_splits: int, workspace: torch.Tensor | None = None,
                                out: torch.Tensor | None = None, stream=None):
    """FP4 GEMM through k_splits FP32 planes (workspace of k_splits*M*N floats, allocated if None)."""
    _, m, n, k = _fp4_operands(a, sfa, b, sfb)
    out = _out16(out, (m, n), a)
    workspace = _workspace(workspace, k_splits, m, n)
    _on_device(a, sfa, b, sfb, out, workspace)
    if workspace is None and k_splits > 1:
        workspace = torch.empty((k_splits, m, n), dtype=torch.float32, device=a.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * 4
    _check(lib.gemm_fp4_blockscaled_splitk(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(out), _ptr(workspace),
                                           ws_bytes, m, n, k, k_splits, _stream(stream)),
           "gemm_fp4_blockscaled_splitk")
    return out


def fp4_scales_from_blocked(blocked: torch.Tensor, rows: int, k_groups: int, batch: int = 1,
                            out: torch.Tensor | None = None, stream=None):
    """Plain [batch, rows, k_groups] scale bytes from the blocked (l, tile_m, tile_k, 32, 4, 4) layout."""
    _bytes(blocked, "blocked")
    if blocked.numel() != batch * rows * k_groups:
        raise ValueError(f"blocked holds {blocked.numel()} bytes, {batch * rows * k_groups} expected")
    if out is None:
        out = torch.empty((batch, rows, k_groups), dtype=torch.uint8, device=blocked.device)
    _shape(_bytes(out, "out"), (batch, rows, k_groups), "out")
    _on_device(blocked, out)
    _check(lib.fp4_scales_from_blocked(_ptr(blocked), _ptr(out), rows, k_groups, batch, _stream(stream)),
           "fp4_scales_from_blocked")
    return out


def gemm_w4a16(a: torch.Tensor, b: torch.Tensor, sfb: torch.Tensor, scale_2: float,
               out: torch.Tensor | None = None, stream=None):
    """C = bf16(scale_2 * (A @ deq(B)^T)): A [M,K] bf16, B [N,K/2] packed e2m1, SFB [N,K/16] e4m3fn."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    n, _ = _dims(_bytes(b, "B"), 2, "B")
    if k % 16 != 0:
        raise ValueError(f"K = {k} must be a multiple of 16 (one scale per 16 elements)")
    _shape(b, (n, k // 2), "B")
    _shape(_bytes(sfb, "SFB"), (n, k // 16), "SFB")
    out = _out16(out, (m, n), a)
    _on_device(a, b, sfb, out)
    _check(lib.gemm_w4a16(_ptr(a), _ptr(b), _ptr(sfb), float(scale_2), _ptr(out), m, n, k, _stream(stream)),
           "gemm_w4a16")
    return out


def gemm_w4a16_t(a: torch.Tensor, bt: torch.Tensor, sfbt: torch.Tensor, n: int, scale_2: float,
                 out: torch.Tensor | None = None, stream=None):
    """gemm_w4a16 with transposed weights: Bt [K/2, ldb] bytes (k pairs as rows), SFBt [K/16, ldb],
    ldb >= n taken from Bt's row length (pad columns n..ldb-1 unused)."""
    m, k = _dims(_bits16(a, "A"), 2, "A")
    if k % 16 != 0:
        raise ValueError(f"K = {k} must be a multiple of 16 (one scale per 16 elements)")
    rows, ldb = _dims(_bytes(bt, "Bt"), 2, "Bt")
    if rows != k // 2 or ldb < n or n < 0:
        raise ValueError(f"Bt must be [K/2, ldb] = [{k // 2}, >= {n}], got {tuple(bt.shape)}")
    _shape(_bytes(sfbt, "SFBt"), (k // 16, ldb), "SFBt")
    out = _out16(out, (m, n), a)
    _on_device(a, bt, sfbt, out)
    _check(lib.gemm_w4a16_t(_ptr(a), _ptr(bt), _ptr(sfbt), ldb, float(scale_2), _ptr(out), m, n, k,
                            _stream(stream)), "gemm_w4a16_t")
    return out


def bf16_scaled_add(out: torch.Tensor, delta: torch.Tensor, scale: float, stream=None):
    """out = bf16(out + fl32(scale * delta)) elementwise, in place."""
    _bits16(out, "out")
    _bits16(delta, "delta")
    if out.numel() != delta.numel():
        raise ValueError("out and delta must have the same number of elements")
    _on_device(out, delta)
    _check(lib.bf16_scaled_add(_ptr(out), _ptr(delta), out.numel(), float(scale), _stream(stream)),
           "bf16_scaled_add")
    return out


# ---------------------------------------------------------------------------
# Tuning overrides and the tile-order helper (host only)
# ---------------------------------------------------------------------------

TUNE_TILE, TUNE_COLSPLIT, TUNE_ORDERED, TUNE_FP4_TILE, TUNE_FP4_SPLITK_TILE, TUNE_W4A16_TILE, \
    TUNE_STREAMK_TILE = range(7)


def tune_set(key: int, value: int) -> None:
    """Force one automatic choice of the library (value -1 restores it)."""
    _check(lib.bg_tune_set(int(key), int(value)), "bg_tune_set")


def tune_get(key: int) -> int:
    return int(lib.bg_tune_get(int(key)))


class tuned:
    """Context manager: `with tuned(TUNE_TILE, 3): ...` forces a choice and restores the previous one."""

    def __init__(self, key: int, value: int):
        self.key, self.value, self.prev = key, value, None

    def __enter__(self):
        self.prev = tune_get(self.key)
        tune_set(self.key, self.value)
        return self

    def __exit__(self, *exc):
        tune_set(self.key, self.prev)
        return False


def tile_map(order: int, tiles_m: int, tiles_n: int):
    """(tm, tn) int32 arrays: the tile each workgroup of a tiles_m x tiles_n grid computes."""
    import numpy as np
    n = tiles_m * tiles_n
    tm = np.zeros(n, np.int32)
    tn = np.zeros(n, np.int32)
    _check(lib.bg_tile_map(int(order), tiles_m, tiles_n, tm.ctypes.data, tn.ctypes.data), "bg_tile_map")
    return tm, tn
