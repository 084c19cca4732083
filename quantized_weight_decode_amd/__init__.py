"""MI355X (gfx950) quantized-weight GEMV: Python binding of libqgemv.so.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libqgemv.so``; there is no CPU or PyTorch fallback: if the
library is missing or a call is refused, an exception is raised.

Two layers:
* ``qgemv_*`` -- the C ABI under the same names, taking raw device pointers
  (ints), sizes and a stream handle, returning the status code;
* ``i4g``, ``fp8b128``, ``mq4v2``, ``fwht256``, ``moe_topk``, ``dequant_*`` --
  take torch tensors on the current CUDA (HIP) device, allocate the output
  with ``torch.empty``, launch on ``torch.cuda.current_stream()`` and raise
  ``QgemvError`` on a refusal.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqgemv.so")

QGEMV_MAX_S = 8

# every entry point declared in include/qgemv.h
_SIGS = {
    "qgemv_strerror": (C.c_char_p, [C.c_int]),
    "qgemv_version": (C.c_char_p, []),
    "qgemv_i4g": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                            C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_i4g_prefill": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_int, C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_fp8b128": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_fp8b128_ue8m0": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_mq4v2": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_mq4v1": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_mq4c": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                             C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_mq4v2_encode": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_mq4v2_rot": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                  C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_fwht256": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                                C.c_int, C.c_int, C.c_void_p]),
    "qgemv_router_topk": (C.c_int, [C.c_void_p, C.c_int, C.c_int, C.c_int, C.c_int,
                                    C.c_void_p, C.c_void_p, C.c_void_p]),
    "qgemv_moe_topk_workspace": (C.c_size_t, [C.c_int, C.c_int, C.c_int]),
    "qgemv_moe_topk": (C.c_int, [C.c_void_p, C.c_void_p, C.c_longlong, C.c_longlong,
                                 C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                 C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                 C.c_void_p, C.c_size_t, C.c_void_p]),
    "qgemv_moe_topk_error": (C.c_int, [C.c_void_p, C.POINTER(C.c_int), C.c_void_p]),
    "qgemv_moe_topk_noalloc": (C.c_int, [C.c_void_p, C.c_void_p, C.c_longlong, C.c_longlong,
                                         C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_int,
                                         C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_int,
                                         C.c_void_p]),
    "qgemv_dequant_i4g": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                                    C.c_int, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_dequant_fp8b128": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                                        C.c_int, C.c_int, C.c_void_p]),
    "qgemv_dequant_fp8b128_ue8m0": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p,
                                              C.c_int, C.c_int, C.c_void_p]),
    "qgemv_dequant_mq4v2": (C.c_int, [C.c_void_p, C.c_void_p,
                                      C.c_int, C.c_int, C.c_void_p]),
    "qgemv_dequant_mq4v1": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]),
    "qgemv_dequant_mq4c": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int, C.c_int, C.c_void_p]),
}

ENTRY_POINTS = tuple(_SIGS)


class QgemvError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


_lib = None


def lib(path: str = LIB_PATH):
    """The loaded libqgemv.so (raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built: run quantized_weight_decode_amd.build.build()")
        L = C.CDLL(path)
        for name, (res, args) in _SIGS.items():
            if not hasattr(L, name):
                continue  # reported by exported_symbols(); calling it raises
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols(path: str = LIB_PATH):
    """Entry points of include/qgemv.h that the built library exports."""
    L = lib(path)
    return [n for n in ENTRY_POINTS if hasattr(L, n)]


def strerror(status: int) -> str:
    return lib().qgemv_strerror(status).decode()


def version() -> str:
    return lib().qgemv_version().decode()


def _call(name, *args):
    st = getattr(lib(), name)(*args)
    if st != 0:
        raise QgemvError(name, st, strerror(st))
    return st


# -- raw C ABI, same names -------------------------------------------------
def qgemv_i4g(w, scales, x, y, S, I, O, gs, stream):
    return lib().qgemv_i4g(w, scales, x, y, S, I, O, gs, stream)


def qgemv_i4g_prefill(w, scales, x, y, S, I, O, gs, stream):
    return lib().qgemv_i4g_prefill(w, scales, x, y, S, I, O, gs, stream)


def qgemv_fp8b128(w, scale_inv, x, y, S, I, O, stream):
    return lib().qgemv_fp8b128(w, scale_inv, x, y, S, I, O, stream)


def qgemv_fp8b128_ue8m0(w, scale_e8m0, x, y, S, I, O, stream):
    return lib().qgemv_fp8b128_ue8m0(w, scale_e8m0, x, y, S, I, O, stream)


def qgemv_mq4v2(w, x_rot, y, S, I, O, stream):
    return lib().qgemv_mq4v2(w, x_rot, y, S, I, O, stream)


def qgemv_mq4v1(w, x_rot, y, S, I, O, stream):
    return lib().qgemv_mq4v1(w, x_rot, y, S, I, O, stream)


def qgemv_mq4c(w, x_rot, y, S, I, O, stream):
    return lib().qgemv_mq4c(w, x_rot, y, S, I, O, stream)


def qgemv_mq4v2_encode(W, w_out, I, O, stream):
    return lib().qgemv_mq4v2_encode(W, w_out, I, O, stream)


def qgemv_mq4v2_rot(w, x, signs, y, S, I, O, stream):
    return lib().qgemv_mq4v2_rot(w, x, signs, y, S, I, O, stream)


def qgemv_fwht256(x, signs, x_rot, S, I, stream):
    return lib().qgemv_fwht256(x, signs, x_rot, S, I, stream)


def qgemv_router_topk(logits, T, E, ld, K, ids, gates, stream):
    return lib().qgemv_router_topk(logits, T, E, ld, K, ids, gates, stream)


def qgemv_moe_topk_workspace(T, K, O):
    return lib().qgemv_moe_topk_workspace(T, K, O)


def qgemv_moe_topk(w, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs,
                   workspace, ws_bytes, stream):
    return lib().qgemv_moe_topk(w, scales, w_stride, s_stride, E, ids, gates, T, K, x, y,
                                I, O, gs, workspace, ws_bytes, stream)


def qgemv_moe_topk_noalloc(w, scales, w_stride, s_stride, E, ids, gates, T, K, x, y, I, O, gs,
                           stream):
    return lib().qgemv_moe_topk_noalloc(w, scales, w_stride, s_stride, E, ids, gates, T, K, x, y,
                                        I, O, gs, stream)


def qgemv_dequant_i4g(w, scales, W, I, O, gs, stream):
    return lib().qgemv_dequant_i4g(w, scales, W, I, O, gs, stream)


def qgemv_dequant_fp8b128(w, scale_inv, W, I, O, stream):
    return lib().qgemv_dequant_fp8b128(w, scale_inv, W, I, O, stream)


def qgemv_dequant_fp8b128_ue8m0(w, scale_e8m0, W, I, O, stream):
    return lib().qgemv_dequant_fp8b128_ue8m0(w, scale_e8m0, W, I, O, stream)


def qgemv_dequant_mq4v2(w, W, I, O, stream):
    return lib().qgemv_dequant_mq4v2(w, W, I, O, stream)


def qgemv_dequant_mq4v1(w, W, I, O, stream):
    return lib().qgemv_dequant_mq4v1(w, W, I, O, stream)


def qgemv_dequant_mq4c(w, W, I, O, stream):
    return lib().qgemv_dequant_mq4c(w, W, I, O, stream)


# -- torch-tensor layer ----------------------------------------------------
def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _dev(t, name, dtype=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _shape(t, name, shape):
    """t must have exactly this shape (a tuple of ints)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _one_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")


def _out(out, S, O, like):
    """The caller's y (checked: f32 [S][O] on like's device) or a new one."""
    torch = _torch()
    if out is None:
        return torch.empty((S, O), dtype=torch.float32, device=like.device)
    if out.numel() != S * O or out.dim() not in (1, 2) or \
            (out.dim() == 2 and tuple(out.shape) != (S, O)) or (out.dim() == 1 and S != 1):
        raise ValueError(f"out must have shape ({S}, {O})" + (f" or ({O},)" if S == 1 else ""))
    return out


def _gs(gs):
    import operator
    gs = operator.index(gs)
    if gs < 2 or gs % 2:
        raise QgemvError("argument check", 3, "group size must be an even number >= 2")
    return gs


def _vecs(x, I, name="x"):
    if x.dim() == 1:
        return 1
    if x.dim() == 2 and x.shape[1] == I:
        return x.shape[0]
    raise ValueError(f"{name} must be [I] or [S, I]")


def _i4g_check(w, scales, x, gs, S, I):
    O = w.shape[0]
    _gs(gs)
    _shape(w, "w", (O, (I + 1) // 2))
    if scales.numel() != O * ((I + gs - 1) // gs):
        raise ValueError(f"scales must hold {O} x {(I + gs - 1) // gs} floats")
    return O


def i4g(w, scales, x, gs, out=None):
    """y[S][O] = grouped-int4 W[O][I] . x[S][I]; w u8 [O][(I+1)//2], scales f32 [O][ng]."""
    torch = _torch()
    I = x.shape[-1]
    S = _vecs(x, I)
    O = _i4g_check(w, scales, x, gs, S, I)
    _one_device(w, scales, x, out)
    y = _out(out, S, O, x)
    _call("qgemv_i4g", _dev(w, "w", torch.uint8), _dev(scales, "scales", torch.float32),
          _dev(x, "x", torch.float32), _dev(y, "y", torch.float32), S, I, O, gs, _stream())
    return y


def i4g_prefill(w, scales, x, gs, out=None):
    """Grouped-int4 product for many tokens (MFMA): x f32 [S][I] -> y f32 [S][O]."""
    torch = _torch()
    I = x.shape[-1]
    S = x.reshape(-1, I).shape[0]
    O = _i4g_check(w, scales, x, gs, S, I)
    _one_device(w, scales, x, out)
    y = _out(out, S, O, x)
    _call("qgemv_i4g_prefill", _dev(w, "w", torch.uint8), _dev(scales, "scales", torch.float32),
          _dev(x, "x", torch.float32), _dev(y, "y", torch.float32), S, I, O, gs, _stream())
    return y


def _fp8_check(w, sc, I, name):
    O = w.shape[0]
    _shape(w, "w", (O, I))
    if sc.numel() != ((O + 127) // 128) * ((I + 127) // 128):
        raise ValueError(f"{name} must hold {(O + 127) // 128} x {(I + 127) // 128} block scales")
    return O


def fp8b128(w, scale_inv, x, out=None):
    torch = _torch()
    I = x.shape[-1]
    S = _vecs(x, I)
    O = _fp8_check(w, scale_inv, I, "scale_inv")
    _one_device(w, scale_inv, x, out)
    y = _out(out, S, O, x)
    _call("qgemv_fp8b128", _dev(w, "w", torch.uint8), _dev(scale_inv, "scale_inv", torch.float32),
          _dev(x, "x", torch.float32), _dev(y, "y", torch.float32), S, I, O, _stream())
    return y


def fp8b128_ue8m0(w, scale_e8m0, x, out=None):
    """fp8-e4m3 GEMV with UE8M0 (power-of-two byte) block scales."""
    torch = _torch()
    I = x.shape[-1]
    S = _vecs(x, I)
    O = _fp8_check(w, scale_e8m0, I, "scale_e8m0")
    _one_device(w, scale_e8m0, x, out)
    y = _out(out, S, O, x)
    _call("qgemv_fp8b128_ue8m0", _dev(w, "w", torch.uint8),
          _dev(scale_e8m0, "scale_e8m0", torch.uint8), _dev(x, "x", torch.float32),
          _dev(y, "y", torch.float32), S, I, O, _stream())
    return y


def _mq4_check(w, I):
    O = w.shape[0]
    if I % 256 == 0:  # otherwise the library refuses the call by name
        if w.numel() != O * (I // 256) * 136:
            raise ValueError(f"w must hold {O} rows of {I // 256} 136-byte groups")
    return O


def mq4v2(w, x_rot, out=None):
    torch = _torch()
    I = x_rot.shape[-1]
    S = _vecs(x_rot, I, "x_rot")
    O = _mq4_check(w, I)
    _one_device(w, x_rot, out)
    y = _out(out, S, O, x_rot)
    _call("qgemv_mq4v2", _dev(w, "w", torch.uint8), _dev(x_rot, "x_rot", torch.float32),
          _dev(y, "y", torch.float32), S, I, O, _stream())
    return y


def _mq4_any(fn, w, x_rot, out):
    torch = _torch()
    I = x_rot.shape[-1]
    S = _vecs(x_rot, I, "x_rot")
    O = _mq4_check(w, I)
    _one_device(w, x_rot, out)
    y = _out(out, S, O, x_rot)
    _call(fn, _dev(w, "w", torch.uint8), _dev(x_rot, "x_rot", torch.float32),
          _dev(y, "y", torch.float32), S, I, O, _stream())
    return y


def mq4v1(w, x_rot, out=None):
    """MQ4 v1 (f32 scale and zero per 256 weights) GEMV on rotated x."""
    return _mq4_any("qgemv_mq4v1", w, x_rot, out)


def mq4c(w, x_rot, out=None):
    """MQ4C pad (one fp16 scale/zero pair per 256 weights) GEMV on rotated x."""
    return _mq4_any("qgemv_mq4c", w, x_rot, out)


def mq4v2_encode(W, out=None):
    """MQ4-v2 groups [O][I/256*136] u8 from rotated-space weights W f32 [O][I]."""
    torch = _torch()
    O, I = W.shape
    _one_device(W, out)
    if out is not None and out.numel() != O * (I // 256) * 136:
        raise ValueError(f"out must hold {O} rows of {I // 256} 136-byte groups")
    w = out if out is not None else torch.empty((O, (I // 256) * 136), dtype=torch.uint8,
                                                 device=W.device)
    _call("qgemv_mq4v2_encode", _dev(W, "W", torch.float32), _dev(w, "w_out", torch.uint8),
          I, O, _stream())
    return w


def mq4v2_rot(w, x, signs, out=None):
    """MQ4-v2 GEMV on unrotated x: the FWHT-256 pre-rotation fused in."""
    torch = _torch()
    I = x.shape[-1]
    S = _vecs(x, I)
    O = _mq4_check(w, I)
    if signs.numel() != I:
        raise ValueError(f"signs must hold {I} values")
    _one_device(w, x, signs, out)
    y = _out(out, S, O, x)
    _call("qgemv_mq4v2_rot", _dev(w, "w", torch.uint8), _dev(x, "x", torch.float32),
          _dev(signs, "signs", torch.int8), _dev(y, "y", torch.float32), S, I, O, _stream())
    return y


def fwht256(x, signs, out=None):
    torch = _torch()
    I = x.shape[-1]
    S = _vecs(x, I)
    if signs.numel() != I:
        raise ValueError(f"signs must hold {I} values")
    _one_device(x, signs, out)
    if out is not None and out.numel() != x.numel():
        raise ValueError(f"out must hold {x.numel()} floats")
    y = out if out is not None else torch.empty_like(x)
    _call("qgemv_fwht256", _dev(x, "x", torch.float32), _dev(signs, "signs", torch.int8),
          _dev(y, "x_rot", torch.float32), S, I, _stream())
    return y


def router_topk(logits, E, K):
    """logits f32 [T][ld] (experts 0..E-1 valid) -> (ids int32 [T][K], gates f32 [T][K])."""
    torch = _torch()
    T, ld = logits.shape
    if not (1 <= E <= ld):
        raise ValueError(f"E must be in 1..{ld} (the row stride of logits)")
    ids = torch.empty((T, K), dtype=torch.int32, device=logits.device)
    gates = torch.empty((T, K), dtype=torch.float32, device=logits.device)
    _call("qgemv_router_topk", _dev(logits, "logits", torch.float32), T, E, ld, K,
          _dev(ids, "ids", torch.int32), _dev(gates, "gates", torch.float32), _stream())
    return ids, gates


def moe_topk_workspace(T, K, O, device):
    torch = _torch()
    n = qgemv_moe_topk_workspace(T, K, O)
    return torch.zeros(max(int(n), 1), dtype=torch.uint8, device=device)


def moe_topk(w, scales, ids, gates, x, gs, workspace=None, out=None):
    """w u8 [E][O][rb], scales f32 [E][O][ng], ids int32 [T][K], gates f32 [T][K], x f32 [T][I]."""
    torch = _torch()
    E, O = w.shape[0], w.shape[1]
    T, K = ids.shape
    I = x.shape[-1]
    _gs(gs)
    _shape(w, "w", (E, O, (I + 1) // 2))
    _shape(scales, "scales", (E, O, (I + gs - 1) // gs))
    _shape(gates, "gates", (T, K))
    _shape(x, "x", (T, I))
    _one_device(w, scales, ids, gates, x, workspace, out)
    ws = workspace if workspace is not None else moe_topk_workspace(T, K, O, x.device)
    if ws.numel() < qgemv_moe_topk_workspace(T, K, O):
        raise ValueError(f"workspace must hold {qgemv_moe_topk_workspace(T, K, O)} bytes")
    y = _out(out, T, O, x)
    _call("qgemv_moe_topk", _dev(w, "w", torch.uint8), _dev(scales, "scales", torch.float32),
          w[0].numel(), scales[0].numel(), E, _dev(ids, "ids", torch.int32),
          _dev(gates, "gates", torch.float32), T, K, _dev(x, "x", torch.float32),
          _dev(y, "y", torch.float32), I, O, gs, _dev(ws, "workspace", torch.uint8),
          ws.numel(), _stream())
    return y


def moe_topk_error(workspace):
    flag = C.c_int(0)
    _call("qgemv_moe_topk_error", _dev(workspace, "workspace"), C.byref(flag), _stream())
    return flag.value


def dequant_i4g(w, scales, I, gs):
    torch = _torch()
    O = _i4g_check(w, scales, None, gs, 1, I)
    _one_device(w, scales)
    W = torch.empty((O, I), dtype=torch.float32, device=w.device)
    _call("qgemv_dequant_i4g", _dev(w, "w", torch.uint8), _dev(scales, "scales", torch.float32),
          _dev(W, "W"), I, O, gs, _stream())
    return W


def dequant_fp8b128(w, scale_inv):
    torch = _torch()
    O, I = w.shape
    _fp8_check(w, scale_inv, I, "scale_inv")
    _one_device(w, scale_inv)
    W = torch.empty((O, I), dtype=torch.float32, device=w.device)
    _call("qgemv_dequant_fp8b128", _dev(w, "w", torch.uint8),
          _dev(scale_inv, "scale_inv", torch.float32), _dev(W, "W"), I, O, _stream())
    return W


def dequant_fp8b128_ue8m0(w, scale_e8m0):
    torch = _torch()
    O, I = w.shape
    _fp8_check(w, scale_e8m0, I, "scale_e8m0")
    _one_device(w, scale_e8m0)
    W = torch.empty((O, I), dtype=torch.float32, device=w.device)
    _call("qgemv_dequant_fp8b128_ue8m0", _dev(w, "w", torch.uint8),
          _dev(scale_e8m0, "scale_e8m0", torch.uint8), _dev(W, "W"), I, O, _stream())
    return W


def _dequant_mq4_any(fn, w, I):
    torch = _torch()
    O = _mq4_check(w, I)
    W = torch.empty((O, I), dtype=torch.float32, device=w.device)
    _call(fn, _dev(w, "w", torch.uint8), _dev(W, "W"), I, O, _stream())
    return W


def dequant_mq4v1(w, I):
    return _dequant_mq4_any("qgemv_dequant_mq4v1", w, I)


def dequant_mq4c(w, I):
    return _dequant_mq4_any("qgemv_dequant_mq4c", w, I)


def dequant_mq4v2(w, I):
    torch = _torch()
    O = _mq4_check(w, I)
    W = torch.empty((O, I), dtype=torch.float32, device=w.device)
    _call("qgemv_dequant_mq4v2", _dev(w, "w", torch.uint8), _dev(W, "W"), I, O, _stream())
    return W
