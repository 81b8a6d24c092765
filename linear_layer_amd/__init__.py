"""Python binding of the MI355X GEMM / fully-connected C-ABI library.

Argument marshalling only: shape, dtype and layout checks, then the tensors'
device pointers and the current HIP stream go to ``liblinear_layer.so``,
whose HIP kernels do all of the arithmetic. There is no fallback: if the
library is missing, importing the functions raises.

Entry points (same names as the C ABI in ``include/linear_layer.h``):

* ``gemm_f32(A, B, C, alpha=1.0, beta=0.0)`` — C = alpha*A*B + beta*C, fp32.
* ``gemm_f16f32(A, B, C, alpha=1.0, beta=0.0)`` — fp16 A, B; fp32 C.
* ``gemm_bf16f32(A, B, C, alpha=1.0, beta=0.0)`` — bf16 A, B; fp32 C.
* ``linear_bias_act(X, W, bias, act, Y)`` — Y = act(X*W + bias), fp32.
* ``gemm_f32_nt``, ``gemm_f16f32_nt``, ``gemm_bf16f32_nt``, ``linear_bias_act_nt``
  — the same with B (W) given N-by-K: C = alpha*A*B^T + beta*C, Y = act(X*W^T + b)
  (W in the [out_features, in_features] layout of ``torch.nn.Linear.weight``).
* ``linear_bias_act_ws(X, W, bias, act, Y, workspace, w_trans=False)`` — the fused
  layer with a caller workspace (``linear_workspace_size``): stream-K shapes in one
  launch with bias and ReLU in every tile's write-back.
* ``linear_bias_act_noalloc(X, W, bias, act, Y, w_trans=False)`` — the same on the
  library's static per-GPU workspace, for callers that cannot allocate.
* ``gemm_f32_batched``, ``gemm_f16f32_batched``, ``gemm_bf16f32_batched``
  ``(A, B, C, alpha=1.0, beta=0.0, trans_b=False)`` — C[i] = alpha*A[i]*op(B[i])
  + beta*C[i] over 3-D tensors whose first axis is the batch; its stride is the
  batch stride (0, e.g. from ``expand``, shares one matrix among all items).

Matrices are 2-D, row-major with unit column stride (a row stride larger than
the width is a leading dimension), on the current CUDA/HIP device. The calls
are asynchronous on ``torch.cuda.current_stream()`` unless ``stream`` is given.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LinearLayerError", "gemm_f32", "gemm_f16f32", "gemm_bf16f32", "linear_bias_act", "status_string",
    "gemm_f32_nt", "gemm_f16f32_nt", "gemm_bf16f32_nt", "linear_bias_act_nt",
    "gemm_f32_batched", "gemm_f16f32_batched", "gemm_bf16f32_batched",
    "linear_bias_act_ws", "linear_workspace_size", "linear_bias_act_noalloc", "NOALLOC_SCRATCH_BYTES",
    "set_noalloc_limit",
    "library_path", "load", "set_tile", "num_tiles", "tile_name", "chosen_tile",
    "set_split_k", "chosen_split_k", "set_stream_k", "chosen_stream_k",
    "ACT_NONE", "ACT_RELU", "DTYPE_F32", "DTYPE_F16", "PLAN_RELU", "PLAN_B_NK", "PLAN_UNALIGNED",
    "OK", "ERR_INVALID_VALUE", "ERR_NO_DEVICE", "ERR_UNSUPPORTED_ARCH", "ERR_LAUNCH",
]

OK, ERR_INVALID_VALUE, ERR_NO_DEVICE, ERR_UNSUPPORTED_ARCH, ERR_LAUNCH = 0, 1, 2, 3, 4
ACT_NONE, ACT_RELU = 0, 1
DTYPE_F32, DTYPE_F16 = 0, 1
PLAN_RELU, PLAN_B_NK, PLAN_UNALIGNED = 0x100, 0x200, 0x400   # flags OR-ed into dtype for chosen_*
NOALLOC_SCRATCH_BYTES = 65 << 20   # the static workspace of linear_bias_act_noalloc

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-package library, or another build of it named by LINEAR_LAYER_LIBRARY
# (the CPU sanitizer test loads an AddressSanitizer build of the host code
# that way). Either way the file must exist: there is no fallback.
_LIB_PATH = os.environ.get("LINEAR_LAYER_LIBRARY") or os.path.join(_HERE, "liblinear_layer.so")
_lib = None

# Every symbol the C header declares.
EXPORTED = ("gemm_f32", "gemm_f16f32", "gemm_bf16f32", "linear_bias_act", "ll_status_string",
            "gemm_f32_nt", "gemm_f16f32_nt", "gemm_bf16f32_nt", "linear_bias_act_nt",
            "gemm_f32_batched", "gemm_f16f32_batched", "gemm_bf16f32_batched",
            "ll_num_tiles", "ll_tile_name", "ll_set_tile", "ll_chosen_tile",
            "ll_set_split_k", "ll_chosen_split_k", "ll_set_stream_k", "ll_chosen_stream_k",
            "linear_bias_act_ws", "ll_linear_workspace_size", "linear_bias_act_noalloc",
            "ll_set_noalloc_limit")


class LinearLayerError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load liblinear_layer.so (built in-tree by ``python -m linear_layer_amd._build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m linear_layer_amd._build`")
    lib = ctypes.CDLL(_LIB_PATH)
    i32, f32, vp = ctypes.c_int, ctypes.c_float, ctypes.c_void_p
    lib.gemm_f32.argtypes = [i32, i32, i32, f32, vp, i32, vp, i32, f32, vp, i32, vp]
    lib.gemm_f16f32.argtypes = lib.gemm_f32.argtypes
    lib.gemm_bf16f32.argtypes = lib.gemm_f32.argtypes
    lib.linear_bias_act.argtypes = [i32, i32, i32, vp, i32, vp, i32, vp, i32, vp, i32, vp]
    lib.linear_bias_act_ws.argtypes = [i32, i32, i32, vp, i32, vp, i32, i32, vp, i32, vp, i32, vp,
                                       ctypes.c_int64, vp]
    lib.linear_bias_act_ws.restype = i32
    lib.linear_bias_act_noalloc.argtypes = [i32, i32, i32, vp, i32, vp, i32, i32, vp, i32, vp, i32, vp]
    lib.linear_bias_act_noalloc.restype = i32
    lib.ll_set_noalloc_limit.argtypes = [ctypes.c_int64]
    lib.ll_set_noalloc_limit.restype = i32
    lib.ll_linear_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.ll_linear_workspace_size.restype = ctypes.c_int64
    for nt in ("gemm_f32_nt", "gemm_f16f32_nt", "gemm_bf16f32_nt"):
        getattr(lib, nt).argtypes = lib.gemm_f32.argtypes
    lib.linear_bias_act_nt.argtypes = lib.linear_bias_act.argtypes
    i64 = ctypes.c_int64
    for b in ("gemm_f32_batched", "gemm_f16f32_batched", "gemm_bf16f32_batched"):
        getattr(lib, b).argtypes = [i32, i32, i32, i32, f32, vp, i32, i64, vp, i32, i64,
                                    f32, vp, i32, i64, i32, vp]
    for f in (lib.gemm_f32, lib.gemm_f16f32, lib.gemm_bf16f32, lib.linear_bias_act,
              lib.gemm_f32_nt, lib.gemm_f16f32_nt, lib.gemm_bf16f32_nt, lib.linear_bias_act_nt,
              lib.gemm_f32_batched, lib.gemm_f16f32_batched, lib.gemm_bf16f32_batched):
        f.restype = i32
    lib.ll_status_string.argtypes = [i32]
    lib.ll_status_string.restype = ctypes.c_char_p
    lib.ll_num_tiles.argtypes = [i32]
    lib.ll_num_tiles.restype = i32
    lib.ll_tile_name.argtypes = [i32, i32]
    lib.ll_tile_name.restype = ctypes.c_char_p
    lib.ll_set_tile.argtypes = [i32, i32]
    lib.ll_set_tile.restype = i32
    lib.ll_chosen_tile.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.ll_chosen_tile.restype = i32
    lib.ll_chosen_split_k.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.ll_chosen_split_k.restype = i32
    lib.ll_set_split_k.argtypes = [i32]
    lib.ll_set_split_k.restype = i32
    lib.ll_set_stream_k.argtypes = [i32]
    lib.ll_set_stream_k.restype = i32
    lib.ll_chosen_stream_k.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.ll_chosen_stream_k.restype = i32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().ll_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != OK:
        raise LinearLayerError(status, where)


def set_tile(dtype: int, tile: int) -> None:
    """Force a tile shape for later calls of that dtype; -1 = automatic.

    Like set_split_k and set_stream_k, a process-wide override for benchmarks
    and tests (include/linear_layer_tuning.h): it steers every later call from
    every thread and on every stream until reset."""
    _check(load().ll_set_tile(int(dtype), int(tile)), "ll_set_tile")


def num_tiles(dtype: int) -> int:
    return load().ll_num_tiles(int(dtype))


def tile_name(dtype: int, tile: int) -> str:
    return load().ll_tile_name(int(dtype), int(tile)).decode()


def chosen_tile(dtype: int, M: int, N: int, K: int, num_cus: int = 0, batch: int = 1) -> int:
    return load().ll_chosen_tile(int(dtype), int(M), int(N), int(K), int(batch), int(num_cus))


def set_split_k(splits: int) -> None:
    """Force the number of K-splits (1..16) for later calls; -1 = automatic.
    Process-wide, like set_tile."""
    _check(load().ll_set_split_k(int(splits)), "ll_set_split_k")


def chosen_split_k(dtype: int, M: int, N: int, K: int, num_cus: int = 0, batch: int = 1) -> int:
    return load().ll_chosen_split_k(int(dtype), int(M), int(N), int(K), int(batch), int(num_cus))


def set_stream_k(mode: int) -> None:
    """Stream-K for leftover tiles: -1 automatic, 0 never, 1 whenever possible.
    Process-wide, like set_tile."""
    _check(load().ll_set_stream_k(int(mode)), "ll_set_stream_k")


def chosen_stream_k(dtype: int, M: int, N: int, K: int, num_cus: int = 0, batch: int = 1) -> int:
    """Number of tiles the plan shares out with stream-K (0: none)."""
    return load().ll_chosen_stream_k(int(dtype), int(M), int(N), int(K), int(batch), int(num_cus))


# ---- tensor marshalling ---------------------------------------------------

def _torch():
    import torch
    return torch


def _mat(t, dtype, name):
    """(pointer, rows, cols, ld) of a 2-D row-major device tensor."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit column stride (row-major)")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    if rows > 1 and ld < cols:
        raise ValueError(f"{name}: row stride {ld} smaller than width {cols}")
    return t.data_ptr(), rows, cols, max(ld, 1)


def _bmat(t, dtype, name):
    """(pointer, batch, rows, cols, ld, batch stride) of a 3-D tensor of row-major matrices."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != 3:
        raise ValueError(f"{name} must be 3-D (batch, rows, cols), got shape {tuple(t.shape)}")
    nb = t.shape[0]
    if nb == 0:
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        return 0, 0, t.shape[1], t.shape[2], max(t.shape[2], 1), 0
    ptr, rows, cols, ld = _mat(t[0], dtype, name)
    bstride = t.stride(0) if nb > 1 else 0
    if bstride < 0:
        raise ValueError(f"{name}: negative batch stride")
    return t.data_ptr(), nb, rows, cols, ld, bstride


def _gemm_batched(fn_name, in_dtype, A, B, C, alpha, beta, trans_b, stream):
    torch = _torch()
    pa, nb, M, K, lda, sa = _bmat(A, in_dtype, "A")
    if trans_b:
        pb, nb2, N, K2, ldb, sb = _bmat(B, in_dtype, "B")
    else:
        pb, nb2, K2, N, ldb, sb = _bmat(B, in_dtype, "B")
    pc, nb3, M2, N2, ldc, sc = _bmat(C, torch.float32, "C")
    if nb2 != nb or nb3 != nb or K2 != K or M2 != M or N2 != N:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    if nb == 0:
        return C
    st = getattr(load(), fn_name)(int(bool(trans_b)), M, N, K, float(alpha), pa, lda, sa, pb, ldb, sb,
                                  float(beta), pc, ldc, sc, nb, _stream(stream, A, B, C))
    _check(st, fn_name)
    return C


def gemm_f32_batched(A, B, C, alpha: float = 1.0, beta: float = 0.0, trans_b: bool = False,
                     stream=None):
    """C[i] = alpha*A[i]*op(B[i]) + beta*C[i], fp32; op(B) = B^T when trans_b."""
    return _gemm_batched("gemm_f32_batched", _torch().float32, A, B, C, alpha, beta, trans_b, stream)


def gemm_f16f32_batched(A, B, C, alpha: float = 1.0, beta: float = 0.0, trans_b: bool = False,
                        stream=None):
    """Batched product with fp16 A, B and fp32 C."""
    return _gemm_batched("gemm_f16f32_batched", _torch().float16, A, B, C, alpha, beta, trans_b, stream)


def gemm_bf16f32_batched(A, B, C, alpha: float = 1.0, beta: float = 0.0, trans_b: bool = False,
                         stream=None):
    """Batched product with bf16 A, B and fp32 C."""
    return _gemm_batched("gemm_bf16f32_batched", _torch().bfloat16, A, B, C, alpha, beta, trans_b,
                         stream)


_RAW = None


def _raw_getters():
    """(current device index, raw current stream of a device): torch's direct
    getters when it has them (no Stream object per call), else the public API."""
    global _RAW
    if _RAW is None:
        torch = _torch()
        get_dev = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device
        get_raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if get_raw is None:
            def get_raw(index):
                return torch.cuda.current_stream(index).cuda_stream
        _RAW = (get_dev, get_raw)
    return _RAW


def _stream(stream, *tensors):
    if stream is None:
        dev = tensors[0].device
        for t in tensors[1:]:
            if t is not None and t.device != dev:
                raise ValueError("all tensors must be on the same device")
        get_dev, get_raw = _raw_getters()
        if get_dev() != dev.index:
            raise ValueError(f"tensors are on {dev}, but the current device is cuda:{get_dev()}")
        return ctypes.c_void_p(get_raw(dev.index))
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _gemm(fn_name, in_dtype, A, B, C, alpha, beta, stream, bt=False):
    torch = _torch()
    pa, M, K, lda = _mat(A, in_dtype, "A")
    if bt:
        pb, N, K2, ldb = _mat(B, in_dtype, "B")
    else:
        pb, K2, N, ldb = _mat(B, in_dtype, "B")
    pc, M2, N2, ldc = _mat(C, torch.float32, "C")
    if K2 != K or M2 != M or N2 != N:
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)}, C {tuple(C.shape)}")
    st = getattr(load(), fn_name)(M, N, K, float(alpha), pa, lda, pb, ldb, float(beta), pc, ldc,
                                  _stream(stream, A, B, C))
    _check(st, fn_name)
    return C


def gemm_f32(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C = alpha*A*B + beta*C (fp32); C is written in place and returned."""
    return _gemm("gemm_f32", _torch().float32, A, B, C, alpha, beta, stream)


def gemm_f16f32(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C = alpha*A*B + beta*C with fp16 A, B and fp32 C; C returned."""
    return _gemm("gemm_f16f32", _torch().float16, A, B, C, alpha, beta, stream)


def gemm_bf16f32(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C = alpha*A*B + beta*C with bf16 A, B and fp32 C; C returned."""
    return _gemm("gemm_bf16f32", _torch().bfloat16, A, B, C, alpha, beta, stream)


def gemm_f32_nt(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C = alpha*A*B^T + beta*C (fp32) with B given N-by-K; C returned."""
    return _gemm("gemm_f32_nt", _torch().float32, A, B, C, alpha, beta, stream, bt=True)


def gemm_f16f32_nt(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C = alpha*A*B^T + beta*C with fp16 A, B (B N-by-K) and fp32 C."""
    return _gemm("gemm_f16f32_nt", _torch().float16, A, B, C, alpha, beta, stream, bt=True)


def gemm_bf16f32_nt(A, B, C, alpha: float = 1.0, beta: float = 0.0, stream=None):
    """C = alpha*A*B^T + beta*C with bf16 A, B (B N-by-K) and fp32 C."""
    return _gemm("gemm_bf16f32_nt", _torch().bfloat16, A, B, C, alpha, beta, stream, bt=True)


def linear_bias_act_nt(X, W, bias, act: int, Y, stream=None):
    """Y = act(X*W^T + bias) (fp32; W is N-by-K, e.g. a torch Linear weight)."""
    return _linear("linear_bias_act_nt", X, W, bias, act, Y, stream, wt=True)


def linear_bias_act(X, W, bias, act: int, Y, stream=None):
    """Y = act(X*W + bias) (fp32; W is K-by-N row-major; bias may be None)."""
    return _linear("linear_bias_act", X, W, bias, act, Y, stream)


def linear_workspace_size(M: int, N: int, K: int, w_trans: bool = False, act: int = ACT_RELU,
                          num_cus: int = 0) -> int:
    """Bytes of workspace linear_bias_act_ws uses for this shape (0: none)."""
    n = load().ll_linear_workspace_size(int(M), int(N), int(K), int(bool(w_trans)), int(act),
                                        int(num_cus))
    if n < 0:
        raise ValueError("invalid shape, layout or activation")
    return n


def linear_bias_act_ws(X, W, bias, act: int, Y, workspace, w_trans: bool = False, stream=None):
    """Y = act(X*W + bias) (or X*W^T with w_trans) with a workspace tensor (zero-filled
    before its first use; the call leaves it zero-filled), so the epilogue stays
    fused into every tile of a stream-K plan. ``workspace`` may be None."""
    torch = _torch()
    pws, nws = None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        pws, nws = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return _linear("linear_bias_act_ws", X, W, bias, act, Y, stream, wt=w_trans, ws=(pws, nws))


def set_noalloc_limit(nbytes: int) -> None:
    """Lower the workspace linear_bias_act_noalloc may use (process-wide;
    -1 restores the full static array). For tests of its refusal."""
    _check(load().ll_set_noalloc_limit(int(nbytes)), "ll_set_noalloc_limit")


def linear_bias_act_noalloc(X, W, bias, act: int, Y, w_trans: bool = False, stream=None):
    """linear_bias_act_ws on the library's own static workspace (nothing is
    allocated); calls that overlap in time on one GPU race."""
    return _linear("linear_bias_act_noalloc", X, W, bias, act, Y, stream, wt=w_trans, ws="static")


def _linear(fn_name, X, W, bias, act, Y, stream, wt=False, ws=None):
    torch = _torch()
    px, M, K, ldx = _mat(X, torch.float32, "X")
    if wt:
        pw, N, K2, ldw = _mat(W, torch.float32, "W")
    else:
        pw, K2, N, ldw = _mat(W, torch.float32, "W")
    py, M2, N2, ldy = _mat(Y, torch.float32, "Y")
    if K2 != K or M2 != M or N2 != N:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, W {tuple(W.shape)}, Y {tuple(Y.shape)}")
    pbias = None
    if bias is not None:
        if bias.dtype != torch.float32 or bias.dim() != 1 or bias.shape[0] != N or not bias.is_cuda:
            raise ValueError("bias must be a 1-D fp32 device tensor of length N")
        if N > 1 and bias.stride(0) != 1:
            raise ValueError("bias must be contiguous")
        pbias = bias.data_ptr()
    if ws == "static":
        st = getattr(load(), fn_name)(M, N, K, px, ldx, pw, ldw, int(bool(wt)), pbias, int(act), py,
                                      ldy, _stream(stream, X, W, Y, bias))
    elif ws is not None:
        st = getattr(load(), fn_name)(M, N, K, px, ldx, pw, ldw, int(bool(wt)), pbias, int(act), py,
                                      ldy, ws[0], ws[1], _stream(stream, X, W, Y, bias))
    else:
        st = getattr(load(), fn_name)(M, N, K, px, ldx, pw, ldw, pbias, int(act), py, ldy,
                                      _stream(stream, X, W, Y, bias))
    _check(st, fn_name)
    return Y
