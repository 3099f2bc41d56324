"""Python binding of ``libatom.so``, the gfx950 W4A4 mixed-precision linear layer.

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared in
``include/atom.h``.  PyTorch supplies device memory and the current HIP stream.  There is
no CPU fallback: tensors must live on a ROCm device and the library must be built
(``python -m bit_quantized_gemm_amd.build``); otherwise every call raises ``AtomError``.

The function names are the C entry points:

* ``atom_channel_stat(X)``                -> fp64 [K]   outlier statistic (offline)
* ``atom_select_outliers(stat)``          -> int32 [K]  perm, outliers at the tail (offline)
* ``atom_pack_weights(W, perm)``          -> (Wq u8 [N, RB], sw fp16 [G, N])  (offline)
* ``atom_quantize_act(X, perm)``          -> (Xq u8 [M, RB], sx fp16 [G, M])
* ``atom_gemm(Xq, sx, Wq, sw, K)``        -> Y fp16 [M, N]
* ``atom_gemm_group_acc(Xq, Wq, K)``      -> acc int32 [G, M, N]   (verification aid)
* W4A8 variant: ``atom_quantize_act_a8(X, perm)`` -> (Xq u8 [M, K], sx), ``atom_pack_weights_w4a8(W, perm)``
  -> (Wq u8 [N, RB], sw), ``atom_gemm_w4a8(Xq, sx, Wq, sw, K)`` -> Y, ``atom_gemm_w4a8_group_acc(Xq, Wq, K)``
* ``atom_row_bytes(K)``, ``atom_num_groups(K)``, ``atom_strerror(status)``
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "AtomError", "EXPORTS", "GROUP", "OUTLIERS", "MAX_K", "lib_path", "load_library",
    "atom_row_bytes", "atom_num_groups", "atom_strerror", "atom_channel_stat", "atom_select_outliers",
    "atom_pack_weights", "atom_quantize_act", "atom_gemm", "atom_gemm_workspace_bytes", "atom_gemm_ws",
    "atom_gemm_group_acc", "linear", "atom_quantize_act_a8", "atom_pack_weights_w4a8", "atom_gemm_w4a8",
    "atom_gemm_w4a8_group_acc", "atom_gemm_w4a8_workspace_bytes", "atom_gemm_w4a8_ws",
]

GROUP = 128
OUTLIERS = 128
MAX_K = 32768

# Every symbol declared in include/atom.h.
EXPORTS = (
    "atom_row_bytes", "atom_num_groups", "atom_strerror", "atom_channel_stat", "atom_select_outliers",
    "atom_pack_weights", "atom_quantize_act", "atom_gemm", "atom_gemm_workspace_bytes", "atom_gemm_ws",
    "atom_gemm_group_acc", "atom_quantize_act_a8", "atom_pack_weights_w4a8", "atom_gemm_w4a8",
    "atom_gemm_w4a8_group_acc", "atom_gemm_w4a8_workspace_bytes", "atom_gemm_w4a8_ws",
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class AtomError(RuntimeError):
    """A non-OK status from libatom, a missing library, or a tensor the ABI cannot take."""


def lib_path() -> str:
    return os.environ.get("ATOM_LIB", os.path.join(_HERE, "libatom.so"))


def load_library():
    """Load libatom.so (once) and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise AtomError(f"{path} is not built; run `python -m bit_quantized_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "atom_row_bytes": (i64, [i32]),
        "atom_num_groups": (i32, [i32]),
        "atom_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "atom_channel_stat": (ctypes.c_int, [vp, i32, i32, vp, vp]),
        "atom_select_outliers": (ctypes.c_int, [vp, i32, vp, vp]),
        "atom_pack_weights": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp]),
        "atom_quantize_act": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp]),
        "atom_gemm": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp]),
        "atom_gemm_workspace_bytes": (i64, [i32, i32, i32]),
        "atom_gemm_ws": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp, i64, vp]),
        "atom_gemm_group_acc": (ctypes.c_int, [vp, vp, i32, i32, i32, vp, vp]),
        "atom_quantize_act_a8": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp]),
        "atom_pack_weights_w4a8": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp]),
        "atom_gemm_w4a8": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp]),
        "atom_gemm_w4a8_group_acc": (ctypes.c_int, [vp, vp, i32, i32, i32, vp, vp]),
        "atom_gemm_w4a8_workspace_bytes": (i64, [i32, i32, i32]),
        "atom_gemm_w4a8_ws": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp, i64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def atom_row_bytes(K: int) -> int:
    return int(load_library().atom_row_bytes(K))


def atom_num_groups(K: int) -> int:
    return int(load_library().atom_num_groups(K))


def atom_strerror(status: int) -> str:
    return load_library().atom_strerror(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise AtomError(f"{what}: {atom_strerror(status)} (status {status})")


# ----------------------------------------------------------------------------- tensor plumbing
def _torch():
    import torch
    return torch


def _dev(t, name, dtype):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise AtomError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise AtomError(f"{name} must be a ROCm device tensor (got {t.device}); there is no CPU path")
    if t.dtype != dtype:
        raise AtomError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise AtomError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------------------- entry points
def atom_channel_stat(X, stat=None, stream=None):
    torch = _torch()
    M, K = X.shape
    if stat is None:
        stat = _empty((K,), torch.float64, X)
    st = load_library().atom_channel_stat(_dev(X, "X", torch.float16), M, K, _dev(stat, "stat", torch.float64),
                                          _stream(stream, X.device))
    _check(st, "atom_channel_stat")
    return stat


def atom_select_outliers(stat, perm=None, stream=None):
    torch = _torch()
    (K,) = stat.shape
    if perm is None:
        perm = _empty((K,), torch.int32, stat)
    st = load_library().atom_select_outliers(_dev(stat, "stat", torch.float64), K, _dev(perm, "perm", torch.int32),
                                             _stream(stream, stat.device))
    _check(st, "atom_select_outliers")
    return perm


def _rows_out(rows, K, like, q, s):
    torch = _torch()
    rb = atom_row_bytes(K)
    g = atom_num_groups(K)
    if rb < 0 or g < 0:
        _check(-rb if rb < 0 else -g, "shape")
    if q is None:
        q = _empty((rows, rb), torch.uint8, like)
    if s is None:
        s = _empty((g, rows), torch.float16, like)
    return q, s


def atom_pack_weights(W, perm, Wq=None, sw=None, stream=None):
    torch = _torch()
    N, K = W.shape
    Wq, sw = _rows_out(N, K, W, Wq, sw)
    st = load_library().atom_pack_weights(_dev(W, "W", torch.float16), _dev(perm, "perm", torch.int32), N, K,
                                          _dev(Wq, "Wq", torch.uint8), _dev(sw, "sw", torch.float16),
                                          _stream(stream, W.device))
    _check(st, "atom_pack_weights")
    return Wq, sw


def atom_quantize_act(X, perm, Xq=None, sx=None, stream=None):
    torch = _torch()
    M, K = X.shape
    Xq, sx = _rows_out(M, K, X, Xq, sx)
    st = load_library().atom_quantize_act(_dev(X, "X", torch.float16), _dev(perm, "perm", torch.int32), M, K,
                                          _dev(Xq, "Xq", torch.uint8), _dev(sx, "sx", torch.float16),
                                          _stream(stream, X.device))
    _check(st, "atom_quantize_act")
    return Xq, sx


def atom_gemm(Xq, sx, Wq, sw, K, Y=None, stream=None):
    torch = _torch()
    M = Xq.shape[0]
    N = Wq.shape[0]
    if Y is None:
        Y = _empty((M, N), torch.float16, Xq)
    st = load_library().atom_gemm(_dev(Xq, "Xq", torch.uint8), _dev(sx, "sx", torch.float16),
                                  _dev(Wq, "Wq", torch.uint8), _dev(sw, "sw", torch.float16), M, N, K,
                                  _dev(Y, "Y", torch.float16), _stream(stream, Xq.device))
    _check(st, "atom_gemm")
    return Y


def atom_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    r = load_library().atom_gemm_workspace_bytes(M, N, K)
    if r < 0:
        raise AtomError(f"atom_gemm_workspace_bytes: {atom_strerror(-r)}")
    return r


def atom_gemm_ws(Xq, sx, Wq, sw, K, workspace, Y=None, stream=None):
    """atom_gemm with a caller-allocated workspace (uint8 tensor on the same device, or None)."""
    torch = _torch()
    M = Xq.shape[0]
    N = Wq.shape[0]
    if Y is None:
        Y = _empty((M, N), torch.float16, Xq)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    st = load_library().atom_gemm_ws(_dev(Xq, "Xq", torch.uint8), _dev(sx, "sx", torch.float16),
                                     _dev(Wq, "Wq", torch.uint8), _dev(sw, "sw", torch.float16), M, N, K,
                                     _dev(Y, "Y", torch.float16), ws_ptr, ws_bytes, _stream(stream, Xq.device))
    _check(st, "atom_gemm_ws")
    return Y


def atom_gemm_group_acc(Xq, Wq, K, acc=None, stream=None):
    torch = _torch()
    M = Xq.shape[0]
    N = Wq.shape[0]
    if acc is None:
        acc = _empty((K // GROUP, M, N), torch.int32, Xq)
    st = load_library().atom_gemm_group_acc(_dev(Xq, "Xq", torch.uint8), _dev(Wq, "Wq", torch.uint8), M, N, K,
                                            _dev(acc, "acc", torch.int32), _stream(stream, Xq.device))
    _check(st, "atom_gemm_group_acc")
    return acc


def linear(X, perm, Wq, sw, Y=None, stream=None, workspace=None):
    """Runtime forward of the layer: quantize X, then the grouped GEMM (one stream).  The GEMM
    uses split-K scratch when the shape needs it: `workspace` if given, else a torch buffer."""
    torch = _torch()
    Xq, sx = atom_quantize_act(X, perm, stream=stream)
    K = X.shape[1]
    need = atom_gemm_workspace_bytes(X.shape[0], Wq.shape[0], K)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    return atom_gemm_ws(Xq, sx, Wq, sw, K, workspace if need else None, Y=Y, stream=stream)


# --------------------------------------------------------------------------- W4A8 variant
def atom_quantize_act_a8(X, perm, Xq=None, sx=None, stream=None):
    """INT8 codes in every group: (Xq u8 [M, K], sx fp16 [G, M])."""
    torch = _torch()
    M, K = X.shape
    _, sx = _rows_out(M, K, X, torch.empty(0), sx)
    if Xq is None:
        Xq = _empty((M, K), torch.uint8, X)
    st = load_library().atom_quantize_act_a8(_dev(X, "X", torch.float16), _dev(perm, "perm", torch.int32), M, K,
                                             _dev(Xq, "Xq", torch.uint8), _dev(sx, "sx", torch.float16),
                                             _stream(stream, X.device))
    _check(st, "atom_quantize_act_a8")
    return Xq, sx


def atom_pack_weights_w4a8(W, perm, Wq=None, sw=None, stream=None):
    """W4 rule, offset-binary INT4 layout for the W4A8 GEMM: (Wq u8 [N, RB], sw fp16 [G, N])."""
    torch = _torch()
    N, K = W.shape
    Wq, sw = _rows_out(N, K, W, Wq, sw)
    st = load_library().atom_pack_weights_w4a8(_dev(W, "W", torch.float16), _dev(perm, "perm", torch.int32), N, K,
                                               _dev(Wq, "Wq", torch.uint8), _dev(sw, "sw", torch.float16),
                                               _stream(stream, W.device))
    _check(st, "atom_pack_weights_w4a8")
    return Wq, sw


def atom_gemm_w4a8(Xq, sx, Wq, sw, K, Y=None, stream=None):
    torch = _torch()
    M = Xq.shape[0]
    N = Wq.shape[0]
    if Y is None:
        Y = _empty((M, N), torch.float16, Xq)
    st = load_library().atom_gemm_w4a8(_dev(Xq, "Xq", torch.uint8), _dev(sx, "sx", torch.float16),
                                       _dev(Wq, "Wq", torch.uint8), _dev(sw, "sw", torch.float16), M, N, K,
                                       _dev(Y, "Y", torch.float16), _stream(stream, Xq.device))
    _check(st, "atom_gemm_w4a8")
    return Y


def atom_gemm_w4a8_group_acc(Xq, Wq, K, acc=None, stream=None):
    torch = _torch()
    M = Xq.shape[0]
    N = Wq.shape[0]
    if acc is None:
        acc = _empty((K // GROUP, M, N), torch.int32, Xq)
    st = load_library().atom_gemm_w4a8_group_acc(_dev(Xq, "Xq", torch.uint8), _dev(Wq, "Wq", torch.uint8), M, N, K,
                                                 _dev(acc, "acc", torch.int32), _stream(stream, Xq.device))
    _check(st, "atom_gemm_w4a8_group_acc")
    return acc


def atom_gemm_w4a8_workspace_bytes(M: int, N: int, K: int) -> int:
    r = load_library().atom_gemm_w4a8_workspace_bytes(M, N, K)
    if r < 0:
        raise AtomError(f"atom_gemm_w4a8_workspace_bytes: {atom_strerror(-r)}")
    return r


def atom_gemm_w4a8_ws(Xq, sx, Wq, sw, K, workspace, Y=None, stream=None):
    """atom_gemm_w4a8 with a caller-allocated split-K workspace (uint8 tensor, or None)."""
    torch = _torch()
    M = Xq.shape[0]
    N = Wq.shape[0]
    if Y is None:
        Y = _empty((M, N), torch.float16, Xq)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _dev(workspace, "workspace", torch.uint8)
        ws_bytes = workspace.numel()
    st = load_library().atom_gemm_w4a8_ws(_dev(Xq, "Xq", torch.uint8), _dev(sx, "sx", torch.float16),
                                          _dev(Wq, "Wq", torch.uint8), _dev(sw, "sw", torch.float16), M, N, K,
                                          _dev(Y, "Y", torch.float16), ws_ptr, ws_bytes, _stream(stream, Xq.device))
    _check(st, "atom_gemm_w4a8_ws")
    return Y
