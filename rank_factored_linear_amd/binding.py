"""Thin Python binding of libtb.so (ctypes).

Argument marshalling only: every step of the projection runs in the HIP
kernels behind the C ABI declared in ``include/tb.h``.  PyTorch supplies
device memory and the current HIP stream.  There is no fallback: if the
library is missing or fails to load, the import raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtb.so")

TB_OK, TB_ERR_INVALID_ARGUMENT, TB_ERR_UNSUPPORTED, TB_ERR_HIP = 0, 1, 2, 3
TB_F32, TB_BF16 = 0, 1
MAX_GROUP = 8
WORKSPACE_CONTROL_BYTES = MAX_GROUP * 65536
FROBENIUS_WORKSPACE_BYTES = 65536

EXPORTED = (
    "tb_band_index", "tb_linear_forward_workspace_size", "tb_linear_forward", "tb_dense_forward",
    "tb_linear_forward_group_workspace_size", "tb_linear_forward_group",
    "tb_reconstruct_weight", "tb_rel_frobenius_error", "tb_reconstruction_error",
    "tb_shared_block", "tb_row_scale", "tb_lowrank_factors_workspace_size", "tb_lowrank_factors",
    "tb_lowrank_factors_batch", "tb_refine_shared_block_workspace_size", "tb_refine_shared_block",
    "tb_debug_set_wait_polls", "tb_status_string", "tb_last_error", "tb_linear_forward_no_alloc",
)
NO_ALLOC_SCRATCH_BYTES = 96 << 20
DEFAULT_WAIT_POLLS = 1 << 20
MAX_BAND_LAYERS = 128
MAX_PROBE = 512


class Projection(ctypes.Structure):
    """tb_projection: one member of a grouped forward call."""
    _fields_ = [("x", ctypes.c_void_p), ("s", ctypes.c_void_p), ("w0", ctypes.c_void_p), ("u", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("y", ctypes.c_void_p), ("out_dim", ctypes.c_int64),
                ("in_dim", ctypes.c_int64), ("rank", ctypes.c_int64)]


class TBError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libtb status {status}: {message}")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m rank_factored_linear_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    c_i32, c_i64, c_p, c_sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    lib.tb_band_index.argtypes = [c_i32, c_i32, c_i32, ctypes.POINTER(c_i32)]
    lib.tb_linear_forward_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i64, ctypes.c_int, ctypes.POINTER(c_sz)]
    lib.tb_linear_forward.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_i64, ctypes.c_int, c_p, c_sz, c_p]
    lib.tb_dense_forward.argtypes = [c_p, c_p, c_p, c_i64, c_i64, c_i64, ctypes.c_int, c_p, c_sz, c_p]
    lib.tb_linear_forward_group_workspace_size.argtypes = [c_i32, ctypes.POINTER(Projection), c_i64, ctypes.c_int,
                                                           ctypes.POINTER(c_sz)]
    lib.tb_linear_forward_group.argtypes = [c_i32, ctypes.POINTER(Projection), c_i64, ctypes.c_int, c_p, c_sz, c_p]
    lib.tb_reconstruct_weight.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_int, c_p]
    lib.tb_rel_frobenius_error.argtypes = [c_p, c_p, c_i64, c_i64, ctypes.c_int, c_p, c_p, c_sz, c_p]
    lib.tb_reconstruction_error.argtypes = [c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, ctypes.c_int, ctypes.c_int,
                                            c_p, c_p, c_sz, c_p]
    lib.tb_shared_block.argtypes = [ctypes.POINTER(c_p), c_i32, c_i64, c_i64, ctypes.c_int, c_p, c_p]
    lib.tb_row_scale.argtypes = [c_p, c_p, c_i64, c_i64, ctypes.c_int, c_p, c_p]
    lib.tb_lowrank_factors_workspace_size.argtypes = [c_i64, c_i64, c_i64, c_i64, ctypes.POINTER(c_sz)]
    lib.tb_lowrank_factors.argtypes = [c_p, c_p, c_p, c_i64, c_i64, c_i64, ctypes.c_int, c_p, c_i64, c_i32, c_p, c_p,
                                       c_p, c_sz, c_p]
    lib.tb_lowrank_factors_batch.argtypes = [ctypes.POINTER(c_p), c_i32, ctypes.POINTER(c_p), c_p, c_i64, c_i64, c_i64,
                                             ctypes.c_int, c_p,
                                             c_i64, c_i32, c_p, c_p, c_p, c_sz, c_p]
    lib.tb_refine_shared_block_workspace_size.argtypes = [c_i64, c_i64, c_i32, c_i64, ctypes.POINTER(c_sz)]
    lib.tb_refine_shared_block.argtypes = [ctypes.POINTER(c_p), ctypes.POINTER(c_p), ctypes.POINTER(c_p),
                                           ctypes.POINTER(c_p), c_i32, c_i64, c_i64, c_i64, ctypes.c_int, c_p, c_p,
                                           c_p, c_sz, c_p]
    lib.tb_debug_set_wait_polls.argtypes = [c_i32]
    lib.tb_linear_forward_no_alloc.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p, c_i64, c_i64, c_i64, c_i64, ctypes.c_int,
                                               c_p]
    lib.tb_status_string.argtypes = [ctypes.c_int]
    lib.tb_status_string.restype = ctypes.c_char_p
    lib.tb_last_error.argtypes = []
    lib.tb_last_error.restype = ctypes.c_char_p
    for name in ("tb_band_index", "tb_linear_forward_workspace_size", "tb_linear_forward",
                 "tb_linear_forward_group_workspace_size", "tb_linear_forward_group",
                 "tb_reconstruct_weight", "tb_rel_frobenius_error", "tb_reconstruction_error"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


lib = _load()


def _check(status: int) -> None:
    if status != TB_OK:
        raise TBError(status, lib.tb_last_error().decode())


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return TB_BF16
    if dt == torch.float32:
        return TB_F32
    raise TBError(TB_ERR_UNSUPPORTED, f"dtype {dt} is not supported (bfloat16 or float32)")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need_cuda(*ts):
    """Every tensor is contiguous and lives on the current GPU (the device the library launches on)."""
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise TBError(TB_ERR_INVALID_ARGUMENT, "tensors must live on the GPU")
            if t.device.index != torch.cuda.current_device():
                raise TBError(TB_ERR_INVALID_ARGUMENT,
                              f"tensor on {t.device}, but the current device is cuda:{torch.cuda.current_device()}")
            if not t.is_contiguous():
                raise TBError(TB_ERR_UNSUPPORTED, "tensors must be contiguous")


# Shape and dtype checks run before the device checks and before anything
# crosses the C ABI: the library sees raw pointers only, so a mis-sized
# tensor would otherwise become out-of-bounds device reads or writes.


def _expect(name: str, t: torch.Tensor, shape, dtype: torch.dtype | None = None) -> None:
    if tuple(t.shape) != tuple(shape):
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"{name} must be {list(shape)}, got {list(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"{name} must be {dtype}, got {t.dtype}")


def _expect_out(out: torch.Tensor | None, shape, dtype: torch.dtype | None = None) -> None:
    if out is not None:
        _expect("out", out, shape, dtype)


def _output(out: torch.Tensor | None, shape, dtype: torch.dtype, like: torch.Tensor) -> torch.Tensor:
    """A new output of this shape and dtype on like's device, or the caller's `out` after checking it."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _expect("out", out, shape, dtype)
    if out.device != like.device:
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"out is on {out.device}, the inputs on {like.device}")
    return out


def _projection_dims(x, s, W0, U, V):
    """(m, out_dim, in_dim, rank, U, V) of one projection after checking every operand against x and W0:
    x [m, in], W0 [out, in], s [out] or None, U [out, rank] and V [in, rank] or both None; one dtype.
    A rank-0 U/V pair becomes None."""
    if x.dim() != 2 or W0.dim() != 2:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "x must be [m, in] and W0 [out, in]")
    _dtype_code(x.dtype)
    m, in_dim = x.shape
    out_dim = W0.shape[0]
    _expect("W0", W0, (out_dim, in_dim), x.dtype)
    if s is not None:
        _expect("s", s, (out_dim,), x.dtype)
    if (U is None) != (V is None):
        raise TBError(TB_ERR_INVALID_ARGUMENT, "U and V are given together or not at all")
    rank = 0
    if U is not None:
        if U.dim() != 2:
            raise TBError(TB_ERR_INVALID_ARGUMENT, "U must be [out, rank]")
        rank = U.shape[1]
        _expect("U", U, (out_dim, rank), x.dtype)
        _expect("V", V, (in_dim, rank), x.dtype)
        if rank == 0:
            U = V = None
    return m, out_dim, in_dim, rank, U, V


def _workspace_bytes(ws: torch.Tensor) -> int:
    _need_cuda(ws)
    return ws.numel() * ws.element_size()


# ---------------------------------------------------------------------------
# Workspace: one zero-initialised buffer per (device, stream), grown on
# demand.  Its control words are zero when created and the library keeps
# them consistent from call to call.
# ---------------------------------------------------------------------------
_ws_lock = threading.Lock()
_ws: dict = {}


def workspace_for(nbytes: int) -> torch.Tensor:
    dev = torch.cuda.current_device()
    key = (dev, torch.cuda.current_stream().cuda_stream)
    with _ws_lock:
        buf = _ws.get(key)
        if buf is None or buf.numel() < nbytes:
            size = max(nbytes, WORKSPACE_CONTROL_BYTES)
            size = (size + (1 << 20) - 1) >> 20 << 20
            buf = torch.zeros(size, dtype=torch.uint8, device=f"cuda:{dev}")
            _ws[key] = buf
        return buf


def set_wait_polls(polls: int = DEFAULT_WAIT_POLLS) -> None:
    """Bound of the decode kernels' wait for x . V (tb_debug_set_wait_polls); 0 forces the timeout path."""
    _check(lib.tb_debug_set_wait_polls(polls))


def workspace_error_word() -> int:
    """Sticky error word of the current stream's workspace (nonzero if a bounded wait timed out)."""
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    buf = _ws.get(key)
    if buf is None:
        return 0
    return int(buf[:32].view(torch.int32)[2].item())


# ---------------------------------------------------------------------------
# Entry points
# ---------------------------------------------------------------------------


def band_index(num_layers: int, num_bands: int, layer: int) -> int:
    out = ctypes.c_int32(-1)
    _check(lib.tb_band_index(num_layers, num_bands, layer, ctypes.byref(out)))
    return out.value


def linear_forward_workspace_size(m: int, out_dim: int, in_dim: int, rank: int, dtype: torch.dtype) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.tb_linear_forward_workspace_size(m, out_dim, in_dim, rank, _dtype_code(dtype), ctypes.byref(out)))
    return out.value


def linear_forward(x: torch.Tensor, s: torch.Tensor | None, W0: torch.Tensor, U: torch.Tensor | None,
                   V: torch.Tensor | None, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = s * (x @ W0.T) + (x @ V) @ U.T on the GPU, via tb_linear_forward (s None: unit scale)."""
    m, out_dim, in_dim, rank, U, V = _projection_dims(x, s, W0, U, V)
    _expect_out(out, (m, out_dim), x.dtype)
    _need_cuda(x, s, W0, U, V, out)
    out = _output(out, (m, out_dim), x.dtype, x)
    need = linear_forward_workspace_size(m, out_dim, in_dim, rank, x.dtype)
    ws = workspace if workspace is not None else workspace_for(need)
    _check(lib.tb_linear_forward(_ptr(x), _ptr(s), _ptr(W0), _ptr(U), _ptr(V), _ptr(out), m, out_dim, in_dim, rank,
                                 _dtype_code(x.dtype), _ptr(ws), _workspace_bytes(ws), _stream()))
    return out


def linear_forward_no_alloc(x: torch.Tensor, s: torch.Tensor | None, W0: torch.Tensor, U: torch.Tensor | None,
                            V: torch.Tensor | None, out: torch.Tensor | None = None) -> torch.Tensor:
    """linear_forward with the library's static device scratch as its workspace (tb_linear_forward_no_alloc):
    with `out` given, nothing is allocated."""
    m, out_dim, in_dim, rank, U, V = _projection_dims(x, s, W0, U, V)
    _expect_out(out, (m, out_dim), x.dtype)
    _need_cuda(x, s, W0, U, V, out)
    out = _output(out, (m, out_dim), x.dtype, x)
    _check(lib.tb_linear_forward_no_alloc(_ptr(x), _ptr(s), _ptr(W0), _ptr(U), _ptr(V), _ptr(out), m, out_dim, in_dim,
                                          rank, _dtype_code(x.dtype), _stream()))
    return out


def dense_forward(x: torch.Tensor, W: torch.Tensor, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = x @ W.T on the GPU, via tb_dense_forward (a weight materialised once, e.g. by reconstruct_weight)."""
    m, out_dim, in_dim, _, _, _ = _projection_dims(x, None, W, None, None)
    _expect_out(out, (m, out_dim), x.dtype)
    _need_cuda(x, W, out)
    out = _output(out, (m, out_dim), x.dtype, x)
    need = linear_forward_workspace_size(m, out_dim, in_dim, 0, x.dtype)
    ws = workspace if workspace is not None else workspace_for(need)
    _check(lib.tb_dense_forward(_ptr(x), _ptr(W), _ptr(out), m, out_dim, in_dim, _dtype_code(x.dtype), _ptr(ws),
                                _workspace_bytes(ws), _stream()))
    return out


def projection_array(members) -> ctypes.Array:
    """tb_projection array for (x, s, W0, U, V, y) tuples (U, V may be None)."""
    arr = (Projection * len(members))()
    for j, (x, s, W0, U, V, y) in enumerate(members):
        rank = 0 if U is None else U.shape[1]
        arr[j] = Projection(_ptr(x), _ptr(s), _ptr(W0), _ptr(U) if rank else None, _ptr(V) if rank else None, _ptr(y),
                            W0.shape[0], W0.shape[1], rank)
    return arr


def linear_forward_group(members, workspace: torch.Tensor | None = None, outs=None) -> list:
    """Several independent projections [(x, s, W0, U, V), ...] of one token count and dtype in one call
    (tb_linear_forward_group); returns their outputs (written into `outs` when given)."""
    if not 1 <= len(members) <= MAX_GROUP:
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"a group holds 1..{MAX_GROUP} projections")
    if outs is not None and len(outs) != len(members):
        raise TBError(TB_ERR_INVALID_ARGUMENT, "one output per member")
    dims = []
    for j, (x, s, W0, U, V) in enumerate(members):
        m, out_dim, in_dim, rank, U, V = _projection_dims(x, s, W0, U, V)
        if m != members[0][0].shape[0] or x.dtype != members[0][0].dtype:
            raise TBError(TB_ERR_INVALID_ARGUMENT, "group members must share the token count and dtype")
        if outs is not None:
            _expect_out(outs[j], (m, out_dim), x.dtype)
        dims.append((x, s, W0, U, V))
    full = []
    for j, (x, s, W0, U, V) in enumerate(dims):
        _need_cuda(x, s, W0, U, V)
        y = _output(None if outs is None else outs[j], (x.shape[0], W0.shape[0]), x.dtype, x)
        _need_cuda(y)
        full.append((x, s, W0, U, V, y))
    m, dtype = members[0][0].shape[0], members[0][0].dtype
    arr = projection_array(full)
    need = ctypes.c_size_t(0)
    _check(lib.tb_linear_forward_group_workspace_size(len(full), arr, m, _dtype_code(dtype), ctypes.byref(need)))
    ws = workspace if workspace is not None else workspace_for(need.value)
    _check(lib.tb_linear_forward_group(len(full), arr, m, _dtype_code(dtype), _ptr(ws), _workspace_bytes(ws),
                                       _stream()))
    return [f[5] for f in full]


def _bundle_dims(s, W0, U, V):
    """(out_dim, in_dim, rank, U, V) of a bundle after checking s [out], U [out, rank], V [in, rank] against W0
    (one dtype); a rank-0 U/V pair becomes None."""
    if W0.dim() != 2:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "W0 must be [out, in]")
    _dtype_code(W0.dtype)
    out_dim, in_dim = W0.shape
    _expect("s", s, (out_dim,), W0.dtype)
    if (U is None) != (V is None):
        raise TBError(TB_ERR_INVALID_ARGUMENT, "U and V are given together or not at all")
    rank = 0
    if U is not None:
        if U.dim() != 2:
            raise TBError(TB_ERR_INVALID_ARGUMENT, "U must be [out, rank]")
        rank = U.shape[1]
        _expect("U", U, (out_dim, rank), W0.dtype)
        _expect("V", V, (in_dim, rank), W0.dtype)
        if rank == 0:
            U = V = None
    return out_dim, in_dim, rank, U, V


def reconstruct_weight(s: torch.Tensor, W0: torch.Tensor, U: torch.Tensor | None, V: torch.Tensor | None,
                       out_dtype: torch.dtype = torch.float32, out: torch.Tensor | None = None) -> torch.Tensor:
    """diag(s) @ W0 + U @ V.T on the GPU, via tb_reconstruct_weight (into `out` when given; its dtype wins)."""
    out_dim, in_dim, rank, U, V = _bundle_dims(s, W0, U, V)
    _expect_out(out, (out_dim, in_dim))
    _need_cuda(s, W0, U, V, out)
    out = _output(out, (out_dim, in_dim), out_dtype if out is None else out.dtype, W0)
    _check(lib.tb_reconstruct_weight(_ptr(s), _ptr(W0), _ptr(U), _ptr(V), _ptr(out), out_dim, in_dim, rank,
                                     _dtype_code(W0.dtype), _dtype_code(out.dtype), _stream()))
    return out


def _expect_error_out(out: torch.Tensor | None) -> None:
    """The error lands in one device double."""
    if out is not None and (out.dtype != torch.float64 or out.numel() != 1):
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"out must hold one float64, got {out.dtype} {list(out.shape)}")


def _error_output(out: torch.Tensor | None, like: torch.Tensor) -> torch.Tensor:
    if out is None:
        return torch.empty((), dtype=torch.float64, device=like.device)
    _need_cuda(out)
    return out


_frob_ws: dict = {}


def _error_workspace() -> torch.Tensor:
    key = (torch.cuda.current_device(), torch.cuda.current_stream().cuda_stream)
    ws = _frob_ws.get(key)
    if ws is None:
        ws = torch.zeros(FROBENIUS_WORKSPACE_BYTES, dtype=torch.uint8, device=f"cuda:{key[0]}")
        _frob_ws[key] = ws
    return ws


def rel_frobenius_error(original: torch.Tensor, reconstructed: torch.Tensor,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """||original - reconstructed||_F / ||original||_F as a 0-d float64 GPU tensor (no sync)."""
    if original.dim() != 2:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "original must be 2-D")
    _dtype_code(original.dtype)
    _expect("reconstructed", reconstructed, original.shape, original.dtype)
    _expect_error_out(out)
    _need_cuda(original, reconstructed)
    rows, cols = original.shape
    out = _error_output(out, original)
    ws = _error_workspace()
    _check(lib.tb_rel_frobenius_error(_ptr(original), _ptr(reconstructed), rows, cols, _dtype_code(original.dtype),
                                      _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def reconstruction_error(original: torch.Tensor, s: torch.Tensor, W0: torch.Tensor, U: torch.Tensor | None,
                         V: torch.Tensor | None, out: torch.Tensor | None = None) -> torch.Tensor:
    """relative_frobenius_error(original, diag(s) @ W0 + U @ V.T) without forming the rebuilt weight, as a 0-d
    float64 GPU tensor (no sync), via tb_reconstruction_error."""
    out_dim, in_dim, rank, U, V = _bundle_dims(s, W0, U, V)
    _expect("original", original, (out_dim, in_dim))
    _dtype_code(original.dtype)
    _expect_error_out(out)
    _need_cuda(original, s, W0, U, V)
    out = _error_output(out, W0)
    ws = _error_workspace()
    _check(lib.tb_reconstruction_error(_ptr(s), _ptr(W0), _ptr(U), _ptr(V), _ptr(original), out_dim, in_dim, rank,
                                       _dtype_code(W0.dtype), _dtype_code(original.dtype), _ptr(out), _ptr(ws),
                                       ws.numel(), _stream()))
    return out


# ---------------------------------------------------------------------------
# Analytic decomposition
# ---------------------------------------------------------------------------


def shared_block(weights, out: torch.Tensor | None = None) -> torch.Tensor:
    """Mean of a band's weight matrices (fp32), via tb_shared_block."""
    n = len(weights)
    if not 1 <= n <= MAX_BAND_LAYERS:
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"a band holds 1..{MAX_BAND_LAYERS} layers")
    if weights[0].dim() != 2:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "weights must be [out, in]")
    out_dim, in_dim = weights[0].shape
    for j, w in enumerate(weights):
        _expect(f"weights[{j}]", w, (out_dim, in_dim), weights[0].dtype)
    _expect_out(out, (out_dim, in_dim), torch.float32)
    _need_cuda(*weights, out)
    out = _output(out, (out_dim, in_dim), torch.float32, weights[0])
    ptrs = (ctypes.c_void_p * n)(*[w.data_ptr() for w in weights])
    _check(lib.tb_shared_block(ptrs, n, out_dim, in_dim, _dtype_code(weights[0].dtype), _ptr(out), _stream()))
    return out


def row_scale(weight: torch.Tensor, W0: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Per-row least-squares scale of weight against W0 (fp32 [out]), via tb_row_scale."""
    if weight.dim() != 2:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "weight must be [out, in]")
    _expect("W0", W0, weight.shape, torch.float32)
    _expect_out(out, (weight.shape[0],), torch.float32)
    _need_cuda(weight, W0, out)
    out = _output(out, (weight.shape[0],), torch.float32, weight)
    _check(lib.tb_row_scale(_ptr(weight), _ptr(W0), weight.shape[0], weight.shape[1], _dtype_code(weight.dtype),
                            _ptr(out), _stream()))
    return out


def lowrank_factors_workspace_size(out_dim: int, in_dim: int, rank: int, k: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.tb_lowrank_factors_workspace_size(out_dim, in_dim, rank, k, ctypes.byref(out)))
    return out.value


def lowrank_factors(weight: torch.Tensor, W0: torch.Tensor, s: torch.Tensor, rank: int, omega: torch.Tensor,
                    power_iters: int, workspace: torch.Tensor | None = None):
    """U [out, rank], V [in, rank] (fp32) of weight - diag(s) W0 by the randomized SVD with probe omega [in, k],
    via tb_lowrank_factors."""
    if weight.dim() != 2 or omega.dim() != 2:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "weight must be [out, in] and omega [in, k]")
    out_dim, in_dim = weight.shape
    k = omega.shape[1]
    _expect("W0", W0, (out_dim, in_dim), torch.float32)
    _expect("s", s, (out_dim,), torch.float32)
    _expect("omega", omega, (in_dim, k), torch.float32)
    _need_cuda(weight, W0, s, omega)
    U = torch.zeros((out_dim, rank), dtype=torch.float32, device=weight.device)
    V = torch.zeros((in_dim, rank), dtype=torch.float32, device=weight.device)
    need = lowrank_factors_workspace_size(out_dim, in_dim, rank, k)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        torch.empty(need, dtype=torch.uint8, device=weight.device)
    _check(lib.tb_lowrank_factors(_ptr(weight), _ptr(W0), _ptr(s), out_dim, in_dim, rank, _dtype_code(weight.dtype),
                                  _ptr(omega), k, power_iters, _ptr(U) if rank else None, _ptr(V) if rank else None,
                                  _ptr(ws), ws.numel(), _stream()))
    return U, V


def lowrank_factors_batch(weights, W0s, S: torch.Tensor, rank: int, omega: torch.Tensor,
                          power_iters: int, workspace: torch.Tensor | None = None):
    """U [n, out, rank], V [n, in, rank] (fp32) for n weights of one shape, each with its shared block (W0s: one
    fp32 tensor for all, or a list of n), S [n, out], omega [n, in, k], via tb_lowrank_factors_batch."""
    n = len(weights)
    if weights[0].dim() != 2 or omega.dim() != 3:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "weights must be [out, in] and omega [n, in, k]")
    out_dim, in_dim = weights[0].shape
    k = omega.shape[2]
    W0s = list(W0s) if isinstance(W0s, (list, tuple)) else [W0s] * n
    if len(W0s) != n:
        raise TBError(TB_ERR_INVALID_ARGUMENT, "one shared block per weight")
    for j in range(n):
        _expect(f"weights[{j}]", weights[j], (out_dim, in_dim), weights[0].dtype)
        _expect(f"W0s[{j}]", W0s[j], (out_dim, in_dim), torch.float32)
    _expect("S", S, (n, out_dim), torch.float32)
    _expect("omega", omega, (n, in_dim, k), torch.float32)
    _need_cuda(S, omega, *weights, *W0s)
    U = torch.zeros((n, out_dim, rank), dtype=torch.float32, device=S.device)
    V = torch.zeros((n, in_dim, rank), dtype=torch.float32, device=S.device)
    need = n * lowrank_factors_workspace_size(out_dim, in_dim, rank, k)
    ws = workspace if workspace is not None and workspace.numel() >= need else \
        torch.empty(need, dtype=torch.uint8, device=S.device)
    ptrs = (ctypes.c_void_p * n)(*[w.data_ptr() for w in weights])
    w0p = (ctypes.c_void_p * n)(*[w.data_ptr() for w in W0s])
    _check(lib.tb_lowrank_factors_batch(ptrs, n, w0p, _ptr(S), out_dim, in_dim, rank,
                                        _dtype_code(weights[0].dtype), _ptr(omega), k, power_iters,
                                        _ptr(U) if rank else None, _ptr(V) if rank else None, _ptr(ws), ws.numel(),
                                        _stream()))
    return U, V


def decompose(weights, num_bands: int, rank: int, oversampling: int = 16, power_iters: int = 2, seed: int = 0,
              batch_bytes: int = 24 << 30) -> dict:
    """One family's theta bundle on the GPU: per band the shared block, per layer the row scale, and the low-rank
    factors of all layers batched (tb_lowrank_factors_batch, at most `batch_bytes` of workspace per call).  The
    randomized SVD uses k = min(rank + oversampling, out, in) and one probe per layer, drawn from a seeded normal
    generator in layer order.  Returns {"W0": [per band], "band": [per layer], "s", "U", "V": [per layer]} of
    fp32 device tensors."""
    L = len(weights)
    bands = [band_index(L, num_bands, l) for l in range(L)]
    out_dim, in_dim = weights[0].shape
    dev = weights[0].device
    W0 = [shared_block([weights[l] for l in range(L) if bands[l] == b]) for b in range(num_bands)]
    res = {"W0": W0, "band": bands, "s": [row_scale(weights[l], W0[bands[l]]) for l in range(L)],
           "U": [None] * L, "V": [None] * L}
    if rank == 0:
        res["U"] = [torch.zeros((out_dim, 0), dtype=torch.float32, device=dev) for _ in range(L)]
        res["V"] = [torch.zeros((in_dim, 0), dtype=torch.float32, device=dev) for _ in range(L)]
        return res
    k = min(rank + oversampling, out_dim, in_dim, MAX_PROBE)
    gen = torch.Generator(device="cpu").manual_seed(seed)
    omegas = [torch.randn((in_dim, k), generator=gen, dtype=torch.float32) for _ in range(L)]
    per = lowrank_factors_workspace_size(out_dim, in_dim, rank, k)
    chunk = max(1, min(MAX_BAND_LAYERS, batch_bytes // per))
    for c0 in range(0, L, chunk):
        part = list(range(c0, min(L, c0 + chunk)))
        S = torch.stack([res["s"][l] for l in part])
        om = torch.stack([omegas[l] for l in part]).to(dev)
        U, V = lowrank_factors_batch([weights[l] for l in part], [W0[bands[l]] for l in part], S, rank, om,
                                     power_iters)
        for j, l in enumerate(part):
            res["U"][l], res["V"][l] = U[j], V[j]
    return res


def refine_shared_block(weights, s_list, U_list, V_list, W0_prev: torch.Tensor,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """Least-squares refit of a band's shared block with every layer's s, U, V fixed (fp32), via
    tb_refine_shared_block; `out` may be W0_prev itself."""
    n = len(weights)
    if W0_prev.dim() != 2 or not (len(s_list) == len(U_list) == len(V_list) == n):
        raise TBError(TB_ERR_INVALID_ARGUMENT, "W0_prev must be [out, in], with s, U, V lists as long as weights")
    out_dim, in_dim = W0_prev.shape
    _expect("W0_prev", W0_prev, (out_dim, in_dim), torch.float32)
    rank = 0 if U_list[0] is None else U_list[0].shape[1]
    for j in range(n):
        _expect(f"weights[{j}]", weights[j], (out_dim, in_dim), weights[0].dtype)
        _expect(f"s[{j}]", s_list[j], (out_dim,), torch.float32)
        if rank:
            _expect(f"U[{j}]", U_list[j], (out_dim, rank), torch.float32)
            _expect(f"V[{j}]", V_list[j], (in_dim, rank), torch.float32)
    _expect_out(out, (out_dim, in_dim), torch.float32)
    _need_cuda(W0_prev, out, *weights, *s_list, *(U_list if rank else []), *(V_list if rank else []))
    out = _output(out, (out_dim, in_dim), torch.float32, W0_prev)
    arr = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])
    need = ctypes.c_size_t(0)
    _check(lib.tb_refine_shared_block_workspace_size(out_dim, in_dim, n, rank, ctypes.byref(need)))
    ws = torch.empty(need.value, dtype=torch.uint8, device=W0_prev.device)
    _check(lib.tb_refine_shared_block(arr(weights), arr(s_list), arr(U_list) if rank else None,
                                      arr(V_list) if rank else None, n, out_dim, in_dim, rank,
                                      _dtype_code(weights[0].dtype), _ptr(W0_prev), _ptr(out), _ptr(ws), ws.numel(),
                                      _stream()))
    return out


def als_decompose(weights, num_bands: int, rank: int, iters: int, oversampling: int = 16, power_iters: int = 2,
                  seed: int = 0) -> dict:
    """decompose() followed by `iters` rounds of alternating least squares: every band's W0 refitted with s, U, V
    fixed (refine_shared_block), then every layer's s and U, V against the new W0 (new probes per round)."""
    bun = decompose(weights, num_bands, rank, oversampling, power_iters, seed)
    L = len(weights)
    bands = bun["band"]
    out_dim, in_dim = weights[0].shape
    dev = weights[0].device
    k = min(rank + oversampling, out_dim, in_dim, MAX_PROBE)
    for it in range(iters):
        for b in range(num_bands):
            mem = [l for l in range(L) if bands[l] == b]
            refine_shared_block([weights[l] for l in mem], [bun["s"][l] for l in mem],
                                [bun["U"][l] if rank else None for l in mem],
                                [bun["V"][l] if rank else None for l in mem], bun["W0"][b], out=bun["W0"][b])
        bun["s"] = [row_scale(weights[l], bun["W0"][bands[l]]) for l in range(L)]
        if rank:
            gen = torch.Generator(device="cpu").manual_seed(seed + 1 + it)
            om = torch.stack([torch.randn((in_dim, k), generator=gen, dtype=torch.float32) for _ in range(L)]).to(dev)
            U, V = lowrank_factors_batch(weights, [bun["W0"][bands[l]] for l in range(L)], torch.stack(bun["s"]), rank,
                                         om, power_iters)
            bun["U"] = [U[l] for l in range(L)]
            bun["V"] = [V[l] for l in range(L)]
    return bun



# The seven projection families of a decoder layer ("The theta bundle", section "Projection families").
ATTENTION_FAMILIES = ("q_proj", "k_proj", "v_proj", "o_proj")
MLP_FAMILIES = ("gate_proj", "up_proj", "down_proj")


def decompose_model(weights_by_family: dict, num_bands: int, rank: int, tie_families: str = "all",
                    oversampling: int = 16, power_iters: int = 2, seed: int = 0) -> dict:
    """Theta bundles for the projection families of a model ("The theta bundle", section "Projection families").

    weights_by_family maps a family name to its per-layer weights.  tie_families="all": every family goes through
    decompose() (family j of the dict order uses seed + j).  tie_families="attn": only q/k/v/o do; each MLP layer
    stays a plain dense layer, returned as the bundle whose W0 is the layer's own weight (the caller's tensor, not a
    copy; every layer its own band), with s = None (unit scale) and U = V = None, which linear_forward,
    linear_forward_group and dense_forward take as they are."""
    if tie_families not in ("all", "attn"):
        raise TBError(TB_ERR_INVALID_ARGUMENT, f"tie_families must be 'all' or 'attn', not {tie_families!r}")
    for fam in weights_by_family:
        if fam not in ATTENTION_FAMILIES + MLP_FAMILIES:
            raise TBError(TB_ERR_INVALID_ARGUMENT, f"unknown projection family {fam!r}")
    out = {}
    for j, (fam, weights) in enumerate(weights_by_family.items()):
        if tie_families == "attn" and fam in MLP_FAMILIES:
            L = len(weights)
            out[fam] = {"W0": list(weights), "band": list(range(L)), "s": [None] * L, "U": [None] * L,
                        "V": [None] * L}
        else:
            out[fam] = decompose(weights, num_bands, rank, oversampling, power_iters, seed + j)
    return out
