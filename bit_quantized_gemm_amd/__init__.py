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
* ``atom_linear(X, perm, Wq, sw, workspace)`` -> (Y, Xq, sx): quantize + GEMM, one persistent launch
  where the shape allows (``atom_linear_workspace_bytes(M, N, K)``; the workspace starts zeroed)
* ``atom_row_bytes(K)``, ``atom_num_groups(K)``, ``atom_strerror(status)``
"""
from __future__ import annotations

import ctypes
import functools
import os

__all__ = [
    "AtomError", "EXPORTS", "GROUP", "OUTLIERS", "MAX_K", "lib_path", "load_library",
    "atom_row_bytes", "atom_num_groups", "atom_strerror", "atom_channel_stat", "atom_select_outliers",
    "atom_pack_weights", "atom_quantize_act", "atom_gemm", "atom_gemm_workspace_bytes", "atom_gemm_ws",
    "atom_gemm_group_acc", "linear", "atom_quantize_act_a8", "atom_pack_weights_w4a8", "atom_gemm_w4a8",
    "atom_gemm_w4a8_group_acc", "atom_gemm_w4a8_workspace_bytes", "atom_gemm_w4a8_ws",
    "atom_linear_workspace_bytes", "atom_linear", "linear_timed_out", "atom_gemm_noalloc",
]

GROUP = 128
OUTLIERS = 128
MAX_K = 65536

# Every symbol declared in include/atom.h.
EXPORTS = (
    "atom_row_bytes", "atom_num_groups", "atom_strerror", "atom_channel_stat", "atom_select_outliers",
    "atom_pack_weights", "atom_quantize_act", "atom_gemm", "atom_gemm_workspace_bytes", "atom_gemm_ws",
    "atom_gemm_group_acc", "atom_quantize_act_a8", "atom_pack_weights_w4a8", "atom_gemm_w4a8",
    "atom_gemm_w4a8_group_acc", "atom_gemm_w4a8_workspace_bytes", "atom_gemm_w4a8_ws",
    "atom_linear_workspace_bytes", "atom_linear", "atom_gemm_noalloc",
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
        "atom_linear_workspace_bytes": (i64, [i32, i32, i32]),
        "atom_linear": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, i64, vp]),
        "atom_gemm_noalloc": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, i32, vp, vp]),
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
# The C ABI sees only pointers, so the sizes the kernels will read and write are checked here,
# before the call: every tensor must have exactly the shape the entry point implies (a wrong
# shape would otherwise be an out-of-bounds device access), the expected dtype, be contiguous
# and live on the same ROCm device as the first operand.
def _torch():
    import torch
    return torch


def _ptrs(*specs):
    """Check every (tensor, name, dtype, shape) and return their device pointers.

    Sizes, dtypes and contiguity of all arguments are checked first, then that they all live
    on the first tensor's ROCm device, so a mis-sized argument is reported as such wherever it
    lives.  ``shape=None`` skips the shape check; ``tensor=None`` passes a NULL pointer.

    One pass over the arguments accepts them when every check holds (the common case, a few
    microseconds cheaper per call than two passes, which matters for launches of small
    shapes); otherwise the two-pass check below names the first problem."""
    Tensor = _torch().Tensor
    out = []
    dev = None
    for t, _, dtype, shape in specs:
        if t is None:
            out.append(None)
            continue
        if (not isinstance(t, Tensor) or (shape is not None and t.shape != shape) or t.dtype != dtype
                or not t.is_contiguous() or not t.is_cuda):
            break
        d = t.get_device()
        if dev is None:
            dev = d
        elif d != dev:
            break
        out.append(t.data_ptr())
    else:
        return out
    return _ptrs_checked(*specs)


def _ptrs_checked(*specs):
    """The two-pass check of :func:`_ptrs` (sizes, dtypes and contiguity first, then devices),
    raising AtomError for the first argument that fails."""
    torch = _torch()
    for t, name, dtype, shape in specs:
        if t is None:
            continue
        if not isinstance(t, torch.Tensor):
            raise AtomError(f"{name} must be a torch.Tensor")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise AtomError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype != dtype:
            raise AtomError(f"{name} must be {dtype} (got {t.dtype})")
        if not t.is_contiguous():
            raise AtomError(f"{name} must be contiguous")
    device = None
    out = []
    for t, name, _, _ in specs:
        if t is None:
            out.append(None)
            continue
        if t.device.type != "cuda":
            raise AtomError(f"{name} must be a ROCm device tensor (got {t.device}); there is no CPU path")
        if device is None:
            device = t.device
        elif t.device != device:
            raise AtomError(f"{name} is on {t.device}, the other operands on {device}")
        out.append(ctypes.c_void_p(t.data_ptr()))
    return out


def _mat(t, name):
    """(rows, cols) of a 2-D tensor argument."""
    if getattr(t, "dim", lambda: -1)() != 2:
        raise AtomError(f"{name} must be a 2-D tensor")
    return int(t.shape[0]), int(t.shape[1])


@functools.lru_cache(maxsize=64)
def _shape_k_valid(K):
    return atom_row_bytes(K), atom_num_groups(K)


def _shape_k(K):
    """(row bytes, groups) of a valid K, else AtomError."""
    rb, g = _shape_k_valid(int(K))
    if rb < 0 or g < 0:
        _check(-rb if rb < 0 else -g, f"K={K}")
    return rb, g


def _stream(stream, device):
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _empty(shape, dtype, like):
    return _torch().empty(shape, dtype=dtype, device=like.device)


# ----------------------------------------------------------------------------- entry points
def atom_channel_stat(X, stat=None, stream=None):
    torch = _torch()
    M, K = _mat(X, "X")
    if stat is None:
        stat = _empty((K,), torch.float64, X)
    pX, pS = _ptrs((X, "X", torch.float16, None), (stat, "stat", torch.float64, (K,)))
    _check(load_library().atom_channel_stat(pX, M, K, pS, _stream(stream, X.device)), "atom_channel_stat")
    return stat


def atom_select_outliers(stat, perm=None, stream=None):
    torch = _torch()
    if getattr(stat, "dim", lambda: -1)() != 1:
        raise AtomError("stat must be a 1-D tensor")
    K = int(stat.shape[0])
    if perm is None:
        perm = _empty((K,), torch.int32, stat)
    pS, pP = _ptrs((stat, "stat", torch.float64, None), (perm, "perm", torch.int32, (K,)))
    _check(load_library().atom_select_outliers(pS, K, pP, _stream(stream, stat.device)), "atom_select_outliers")
    return perm


def _row_quantize(fn, what, X, perm, q, s, stream, a8=False):
    """Shared marshalling of the row quantize calls: X fp16 [rows, K], perm int32 [K] ->
    codes u8 [rows, K (A8) or row bytes], scales fp16 [G, rows]."""
    torch = _torch()
    rows, K = _mat(X, "X")
    rb, g = _shape_k(K)
    if a8:
        rb = K
    if q is None:
        q = _empty((rows, rb), torch.uint8, X)
    if s is None:
        s = _empty((g, rows), torch.float16, X)
    pX, pP, pQ, pS = _ptrs((X, "X", torch.float16, None), (perm, "perm", torch.int32, (K,)),
                           (q, "codes", torch.uint8, (rows, rb)), (s, "scales", torch.float16, (g, rows)))
    _check(fn(pX, pP, rows, K, pQ, pS, _stream(stream, X.device)), what)
    return q, s


def atom_pack_weights(W, perm, Wq=None, sw=None, stream=None):
    return _row_quantize(load_library().atom_pack_weights, "atom_pack_weights", W, perm, Wq, sw, stream)


def atom_quantize_act(X, perm, Xq=None, sx=None, stream=None):
    return _row_quantize(load_library().atom_quantize_act, "atom_quantize_act", X, perm, Xq, sx, stream)


def _gemm_args(Xq, sx, Wq, sw, K, out, out_name, out_dtype, workspace=None, a8=False, acc=False):
    """Check the GEMM operands against K and return (pointers, M, N, out tensor, workspace bytes).

    Xq u8 [M, row bytes] (A8: [M, K]), sx fp16 [G, M], Wq u8 [N, row bytes], sw fp16 [G, N];
    the output is fp16 Y [M, N], or int32 acc [G, M, N] (acc=True, no scales); the workspace a
    1-D uint8 tensor or None."""
    torch = _torch()
    rb, g = _shape_k(K)
    M, _ = _mat(Xq, "Xq")
    N, _ = _mat(Wq, "Wq")
    oshape = (g, M, N) if acc else (M, N)
    if out is None:
        out = _empty(oshape, out_dtype, Xq)
    if workspace is not None and getattr(workspace, "dim", lambda: -1)() != 1:
        raise AtomError("workspace must be a 1-D uint8 tensor")
    ptrs = _ptrs((Xq, "Xq", torch.uint8, (M, K if a8 else rb)),
                 (None if acc else sx, "sx", torch.float16, (g, M)),
                 (Wq, "Wq", torch.uint8, (N, rb)),
                 (None if acc else sw, "sw", torch.float16, (g, N)),
                 (out, out_name, out_dtype, oshape),
                 (workspace, "workspace", torch.uint8, None))
    return ptrs, M, N, out, (int(workspace.numel()) if workspace is not None else 0)


def atom_gemm(Xq, sx, Wq, sw, K, Y=None, stream=None):
    torch = _torch()
    (pX, pSx, pW, pSw, pY, _), M, N, Y, _ = _gemm_args(Xq, sx, Wq, sw, K, Y, "Y", torch.float16)
    _check(load_library().atom_gemm(pX, pSx, pW, pSw, M, N, K, pY, _stream(stream, Xq.device)), "atom_gemm")
    return Y


def atom_gemm_workspace_bytes(M: int, N: int, K: int) -> int:
    r = load_library().atom_gemm_workspace_bytes(M, N, K)
    if r < 0:
        raise AtomError(f"atom_gemm_workspace_bytes: {atom_strerror(-r)}")
    return r


def atom_gemm_ws(Xq, sx, Wq, sw, K, workspace, Y=None, stream=None):
    """atom_gemm with a caller-allocated workspace (uint8 tensor on the same device, or None)."""
    torch = _torch()
    (pX, pSx, pW, pSw, pY, pWs), M, N, Y, nws = _gemm_args(Xq, sx, Wq, sw, K, Y, "Y", torch.float16, workspace)
    _check(load_library().atom_gemm_ws(pX, pSx, pW, pSw, M, N, K, pY, pWs, nws, _stream(stream, Xq.device)),
           "atom_gemm_ws")
    return Y


def atom_gemm_noalloc(Xq, sx, Wq, sw, K, Y=None, stream=None):
    """atom_gemm with the library's static split-K scratch: the C call allocates nothing (pass Y to
    allocate nothing here either)."""
    torch = _torch()
    (pX, pSx, pW, pSw, pY, _), M, N, Y, _ = _gemm_args(Xq, sx, Wq, sw, K, Y, "Y", torch.float16)
    _check(load_library().atom_gemm_noalloc(pX, pSx, pW, pSw, M, N, K, pY, _stream(stream, Xq.device)),
           "atom_gemm_noalloc")
    return Y


def atom_gemm_group_acc(Xq, Wq, K, acc=None, stream=None):
    torch = _torch()
    (pX, _, pW, _, pA, _), M, N, acc, _ = _gemm_args(Xq, None, Wq, None, K, acc, "acc", torch.int32, acc=True)
    _check(load_library().atom_gemm_group_acc(pX, pW, M, N, K, pA, _stream(stream, Xq.device)),
           "atom_gemm_group_acc")
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


# --------------------------------------------------------------------------- fused forward
def atom_linear_workspace_bytes(M: int, N: int, K: int) -> int:
    r = load_library().atom_linear_workspace_bytes(M, N, K)
    if r < 0:
        raise AtomError(f"atom_linear_workspace_bytes: {atom_strerror(-r)}")
    return r


def atom_linear(X, perm, Wq, sw, workspace, Xq=None, sx=None, Y=None, stream=None):
    """Quantize X and run the grouped GEMM in one call (one persistent launch where the shape
    allows).  ``workspace``: 1-D uint8 tensor of at least atom_linear_workspace_bytes(M, N, K)
    bytes, zero before its first use (torch.zeros); calls leave it zero.  Returns (Y, Xq, sx)."""
    torch = _torch()
    M, K = _mat(X, "X")
    N, _ = _mat(Wq, "Wq")
    rb, g = _shape_k(K)
    if Xq is None:
        Xq = _empty((M, rb), torch.uint8, X)
    if sx is None:
        sx = _empty((g, M), torch.float16, X)
    if Y is None:
        Y = _empty((M, N), torch.float16, X)
    if getattr(workspace, "dim", lambda: -1)() != 1:
        raise AtomError("workspace must be a 1-D uint8 tensor")
    ptrs = _ptrs((X, "X", torch.float16, None), (perm, "perm", torch.int32, (K,)), (Wq, "Wq", torch.uint8, (N, rb)),
                 (sw, "sw", torch.float16, (g, N)), (Xq, "Xq", torch.uint8, (M, rb)),
                 (sx, "sx", torch.float16, (g, M)), (Y, "Y", torch.float16, (M, N)),
                 (workspace, "workspace", torch.uint8, None))
    _check(load_library().atom_linear(ptrs[0], ptrs[1], ptrs[2], ptrs[3], M, N, K, ptrs[4], ptrs[5], ptrs[6], ptrs[7],
                                      int(workspace.numel()), _stream(stream, X.device)), "atom_linear")
    return Y, Xq, sx


def linear_timed_out(workspace) -> bool:
    """True if a bounded wait of an atom_linear call using this workspace gave up (int32 word 9;
    read after the stream has completed)."""
    return bool(workspace[36:40].view(_torch().int32).item())


# --------------------------------------------------------------------------- W4A8 variant
def atom_quantize_act_a8(X, perm, Xq=None, sx=None, stream=None):
    """INT8 codes in every group: (Xq u8 [M, K], sx fp16 [G, M])."""
    return _row_quantize(load_library().atom_quantize_act_a8, "atom_quantize_act_a8", X, perm, Xq, sx, stream,
                         a8=True)


def atom_pack_weights_w4a8(W, perm, Wq=None, sw=None, stream=None):
    """W4 rule, offset-binary INT4 layout for the W4A8 GEMM: (Wq u8 [N, RB], sw fp16 [G, N])."""
    return _row_quantize(load_library().atom_pack_weights_w4a8, "atom_pack_weights_w4a8", W, perm, Wq, sw, stream)


def atom_gemm_w4a8(Xq, sx, Wq, sw, K, Y=None, stream=None):
    torch = _torch()
    (pX, pSx, pW, pSw, pY, _), M, N, Y, _ = _gemm_args(Xq, sx, Wq, sw, K, Y, "Y", torch.float16, a8=True)
    _check(load_library().atom_gemm_w4a8(pX, pSx, pW, pSw, M, N, K, pY, _stream(stream, Xq.device)),
           "atom_gemm_w4a8")
    return Y


def atom_gemm_w4a8_group_acc(Xq, Wq, K, acc=None, stream=None):
    torch = _torch()
    (pX, _, pW, _, pA, _), M, N, acc, _ = _gemm_args(Xq, None, Wq, None, K, acc, "acc", torch.int32, a8=True,
                                                     acc=True)
    _check(load_library().atom_gemm_w4a8_group_acc(pX, pW, M, N, K, pA, _stream(stream, Xq.device)),
           "atom_gemm_w4a8_group_acc")
    return acc


def atom_gemm_w4a8_workspace_bytes(M: int, N: int, K: int) -> int:
    r = load_library().atom_gemm_w4a8_workspace_bytes(M, N, K)
    if r < 0:
        raise AtomError(f"atom_gemm_w4a8_workspace_bytes: {atom_strerror(-r)}")
    return r


def atom_gemm_w4a8_ws(Xq, sx, Wq, sw, K, workspace, Y=None, stream=None):
    """atom_gemm_w4a8 with a caller-allocated split-K workspace (uint8 tensor, or None)."""
    torch = _torch()
    (pX, pSx, pW, pSw, pY, pWs), M, N, Y, nws = _gemm_args(Xq, sx, Wq, sw, K, Y, "Y", torch.float16, workspace,
                                                           a8=True)
    _check(load_library().atom_gemm_w4a8_ws(pX, pSx, pW, pSw, M, N, K, pY, pWs, nws, _stream(stream, Xq.device)),
           "atom_gemm_w4a8_ws")
    return Y
