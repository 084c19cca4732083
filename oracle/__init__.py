"""CPU oracle for the quantized-weight GEMV path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg use this
package.  It wraps ``qref.c`` (plain C11, double accumulation) through ctypes
and shares nothing with the GPU library.

``build()`` compiles ``libqref.so`` next to this file with gcc;
``build_mutant(n, dir)`` compiles the same source with the planted mistake
number ``n`` so tests can show that their pins catch it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qref.c")
LIB = os.path.join(HERE, "libqref.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC"]


# AddressSanitizer and UndefinedBehaviorSanitizer build (host code only); any
# report aborts the process
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g",
            "-fno-omit-frame-pointer"]


def build(out: str = LIB, mutate: int = 0, sanitize: bool = False) -> str:
    """Compile qref.c (optionally with planted mistake ``mutate``, or with the
    address and undefined-behaviour sanitizers) to ``out``."""
    cmd = ["gcc", *CFLAGS, *(SANITIZE if sanitize else []), f"-DQREF_MUTATE={int(mutate)}", SRC,
           "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def build_mutant(n: int, directory: str) -> str:
    return build(os.path.join(directory, f"libqref_mut{n}.so"), mutate=n)


_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_i8p = np.ctypeslib.ndpointer(dtype=np.int8, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_rowsp = C.c_void_p


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise FileNotFoundError(f"oracle library {path} is not built (oracle.build())")
        L = C.CDLL(path)
        self.lib = L
        self.path = path
        L.qref_e4m3.restype = C.c_double
        L.qref_e4m3.argtypes = [C.c_uint8]
        L.qref_e8m0.restype = C.c_double
        L.qref_e8m0.argtypes = [C.c_uint8]
        L.qref_f16.restype = C.c_double
        L.qref_f16.argtypes = [C.c_uint16]
        L.qref_set_threads.argtypes = [C.c_int]
        L.qref_get_threads.restype = C.c_int
        L.qref_mutation.restype = C.c_int
        I = C.c_int
        L.qref_i4g_dequant.argtypes = [_u8p, _f32p, I, I, I, _f32p]
        L.qref_i4g_gemv.argtypes = [_u8p, _f32p, _f32p, _f32p, I, I, I, I, _rowsp, I]
        L.qref_fp8b128_dequant.argtypes = [_u8p, _f32p, I, I, _f32p]
        L.qref_fp8b128_gemv.argtypes = [_u8p, _f32p, _f32p, _f32p, I, I, I, _rowsp, I]
        L.qref_fp8ue8m0_dequant.argtypes = [_u8p, _u8p, I, I, _f32p]
        L.qref_fp8ue8m0_gemv.argtypes = [_u8p, _u8p, _f32p, _f32p, I, I, I, _rowsp, I]
        L.qref_mq4v2_dequant.argtypes = [_u8p, I, I, _f32p]
        L.qref_mq4v2_gemv.argtypes = [_u8p, _f32p, _f32p, I, I, I, _rowsp, I]
        L.qref_fwht256.argtypes = [_f32p, _i8p, _f32p, I, I]
        L.qref_mq4v1_dequant.argtypes = [_u8p, I, I, _f32p]
        L.qref_mq4c_dequant.argtypes = [_u8p, I, I, _f32p]
        L.qref_mq4v1_gemv.argtypes = [_u8p, _f32p, _f32p, I, I, I, _rowsp, I]
        L.qref_mq4c_gemv.argtypes = [_u8p, _f32p, _f32p, I, I, I, _rowsp, I]
        L.qref_mq4v2_encode.argtypes = [_f32p, I, I, _u8p]
        L.qref_router_topk.argtypes = [_f32p, I, I, I, I, _i32p, _f32p]
        L.qref_f32_to_f16.restype = C.c_uint16
        L.qref_f32_to_f16.argtypes = [C.c_float]
        L.qref_moe_i4g.argtypes = [_u8p, _f32p, C.c_longlong, C.c_longlong, I, _i32p,
                                   _f32p, I, I, _f32p, _f32p, I, I, I, _rowsp, I]
        for f in (L.qref_i4g_dequant, L.qref_i4g_gemv, L.qref_fp8b128_dequant,
                  L.qref_fp8b128_gemv, L.qref_fp8ue8m0_dequant, L.qref_fp8ue8m0_gemv,
                  L.qref_mq4v2_dequant, L.qref_mq4v2_gemv,
                  L.qref_fwht256, L.qref_moe_i4g, L.qref_set_threads,
                  L.qref_mq4v1_dequant, L.qref_mq4c_dequant, L.qref_mq4v1_gemv,
                  L.qref_mq4c_gemv, L.qref_mq4v2_encode, L.qref_router_topk):
            f.restype = None

    # -- scalars ---------------------------------------------------------
    def e4m3(self, b: int) -> float:
        return self.lib.qref_e4m3(b)

    def e8m0(self, e: int) -> float:
        return self.lib.qref_e8m0(e)

    def f16(self, h: int) -> float:
        return self.lib.qref_f16(h)

    @property
    def mutation(self) -> int:
        return self.lib.qref_mutation()

    def set_threads(self, n: int) -> None:
        self.lib.qref_set_threads(int(n))

    @property
    def threads(self) -> int:
        return self.lib.qref_get_threads()

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _rows(rows):
        if rows is None:
            return None, None, 0
        r = np.ascontiguousarray(rows, dtype=np.int32)
        return r, r.ctypes.data_as(C.c_void_p), int(r.size)

    @staticmethod
    def _c(a, dt):
        return np.ascontiguousarray(a, dtype=dt)

    # -- grouped int4 ----------------------------------------------------
    def i4g_dequant(self, w, s, O, I, gs):
        W = np.empty((O, I), np.float32)
        self.lib.qref_i4g_dequant(self._c(w, np.uint8), self._c(s, np.float32), O, I, gs, W)
        return W

    def i4g_gemv(self, w, s, x, O, I, gs, rows=None):
        x = self._c(x, np.float32).reshape(-1, I)
        keep, rp, n = self._rows(rows)
        y = np.empty((x.shape[0], n if rows is not None else O), np.float32)
        self.lib.qref_i4g_gemv(self._c(w, np.uint8), self._c(s, np.float32), x, y,
                               x.shape[0], I, O, gs, rp, n)
        return y

    # -- fp8 block-scaled ------------------------------------------------
    def fp8b128_dequant(self, w, sc, O, I):
        W = np.empty((O, I), np.float32)
        self.lib.qref_fp8b128_dequant(self._c(w, np.uint8), self._c(sc, np.float32), O, I, W)
        return W

    def fp8b128_gemv(self, w, sc, x, O, I, rows=None):
        x = self._c(x, np.float32).reshape(-1, I)
        keep, rp, n = self._rows(rows)
        y = np.empty((x.shape[0], n if rows is not None else O), np.float32)
        self.lib.qref_fp8b128_gemv(self._c(w, np.uint8), self._c(sc, np.float32), x, y,
                                   x.shape[0], I, O, rp, n)
        return y

    # -- MQ4-v2 ----------------------------------------------------------
    # -- fp8 with UE8M0 block scales ----------------------------------------
    def fp8ue8m0_dequant(self, w, se, O, I):
        W = np.empty((O, I), np.float32)
        self.lib.qref_fp8ue8m0_dequant(self._c(w, np.uint8), self._c(se, np.uint8), O, I, W)
        return W

    def fp8ue8m0_gemv(self, w, se, x, O, I, rows=None):
        x = self._c(x, np.float32).reshape(-1, I)
        r, rp, n = self._rows(rows)
        y = np.empty((x.shape[0], n if rows is not None else O), np.float32)
        self.lib.qref_fp8ue8m0_gemv(self._c(w, np.uint8), self._c(se, np.uint8), x, y,
                                    x.shape[0], I, O, rp, n)
        return y

    def mq4v2_dequant(self, w, O, I):
        W = np.empty((O, I), np.float32)
        self.lib.qref_mq4v2_dequant(self._c(w, np.uint8), O, I, W)
        return W

    def mq4v2_gemv(self, w, x, O, I, rows=None):
        x = self._c(x, np.float32).reshape(-1, I)
        keep, rp, n = self._rows(rows)
        y = np.empty((x.shape[0], n if rows is not None else O), np.float32)
        self.lib.qref_mq4v2_gemv(self._c(w, np.uint8), x, y, x.shape[0], I, O, rp, n)
        return y

    # -- MQ4 v1 (f32 header per 256) and MQ4C (fp16 pair per 256 + pad) ---
    def _mq4g_dequant(self, fn, w, O, I):
        W = np.empty((O, I), np.float32)
        fn(self._c(w, np.uint8), O, I, W)
        return W

    def _mq4g_gemv(self, fn, w, x, O, I, rows):
        x = self._c(x, np.float32).reshape(-1, I)
        keep, rp, n = self._rows(rows)
        y = np.empty((x.shape[0], n if rows is not None else O), np.float32)
        fn(self._c(w, np.uint8), x, y, x.shape[0], I, O, rp, n)
        return y

    def mq4v1_dequant(self, w, O, I):
        return self._mq4g_dequant(self.lib.qref_mq4v1_dequant, w, O, I)

    def mq4c_dequant(self, w, O, I):
        return self._mq4g_dequant(self.lib.qref_mq4c_dequant, w, O, I)

    def mq4v1_gemv(self, w, x, O, I, rows=None):
        return self._mq4g_gemv(self.lib.qref_mq4v1_gemv, w, x, O, I, rows)

    def mq4c_gemv(self, w, x, O, I, rows=None):
        return self._mq4g_gemv(self.lib.qref_mq4c_gemv, w, x, O, I, rows)

    def mq4v2_encode(self, W, O, I):
        out = np.empty(O * (I // 256) * 136, np.uint8)
        self.lib.qref_mq4v2_encode(self._c(W, np.float32), O, I, out)
        return out.reshape(O, (I // 256) * 136)

    def router_topk(self, logits, E, K):
        """logits f32 [T][ld] (ld >= E) -> ids int32 [T][K], gates f32 [T][K]."""
        lg = self._c(logits, np.float32)
        T, ld = lg.shape
        ids = np.empty((T, K), np.int32)
        gates = np.empty((T, K), np.float32)
        self.lib.qref_router_topk(lg, T, E, ld, K, ids, gates)
        return ids, gates

    def f32_to_f16(self, f: float) -> int:
        return self.lib.qref_f32_to_f16(f)

    def fwht256(self, x, signs, I):
        x = self._c(x, np.float32).reshape(-1, I)
        out = np.empty_like(x)
        self.lib.qref_fwht256(x, self._c(signs, np.int8), out, x.shape[0], I)
        return out

    # -- routed experts --------------------------------------------------
    def moe_i4g(self, w, s, ids, gates, x, E, O, I, gs, rows=None):
        """``w`` u8[E][O][rb], ``s`` f32[E][O][ng]; returns y f32[T][O or nrows]."""
        w = self._c(w, np.uint8)
        s = self._c(s, np.float32)
        ids = self._c(ids, np.int32)
        T, K = ids.shape
        x = self._c(x, np.float32).reshape(T, I)
        w_stride = w.size // E
        s_stride = s.size // E
        keep, rp, n = self._rows(rows)
        y = np.empty((T, n if rows is not None else O), np.float32)
        self.lib.qref_moe_i4g(w, s, w_stride, s_stride, E, ids, self._c(gates, np.float32),
                              T, K, x, y, I, O, gs, rp, n)
        return y


_default = None


def load() -> Oracle:
    """The oracle built next to this file (built on first use if missing), or
    the library the environment variable QREF_LIB names (a sanitizer build)."""
    global _default
    if _default is None:
        path = os.environ.get("QREF_LIB", LIB)
        if path == LIB and not os.path.exists(LIB):
            build()
        _default = Oracle(path)
    return _default
