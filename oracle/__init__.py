"""Python view of the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The GPU library never does, and this package never imports the
GPU library.

Arrays cross as numpy arrays holding the raw storage of the dtype:
float32 for "f32", uint16 bit patterns for "bf16" and "f16".
"""
import ctypes
import os

import numpy as np

from .build import LIB, build as _build

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
OPS = {"fwd": 0, "dx": 1, "dw": 2}
STORAGE = {"f32": np.float32, "bf16": np.uint16, "f16": np.uint16}


class Oracle:
    """Handle on one build of the oracle's shared object."""

    def __init__(self, path=LIB):
        L = ctypes.CDLL(path)
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [
            ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ]
        L.oracle_round.restype = ctypes.c_int
        L.oracle_round.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        L.oracle_env_ok.restype = ctypes.c_int
        L.oracle_version.restype = ctypes.c_int
        vp, i64 = ctypes.c_void_p, ctypes.c_int64
        L.oracle_gemm_cr.restype = ctypes.c_int
        L.oracle_gemm_cr.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, i64, i64, i64, vp, i64, vp]
        L.oracle_exact_sum.restype = ctypes.c_int
        L.oracle_exact_sum.argtypes = [vp, i64, ctypes.c_int, vp]
        L.oracle_layernorm_fwd.restype = ctypes.c_int
        L.oracle_layernorm_fwd.argtypes = [ctypes.c_int, vp, vp, vp, i64, i64, ctypes.c_double, vp, vp, vp, vp]
        L.oracle_layernorm_bwd.restype = ctypes.c_int
        L.oracle_layernorm_bwd.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp]
        if L.oracle_env_ok() != 1:
            raise RuntimeError("oracle: floating-point environment is not IEEE RNE without FTZ/DAZ")
        self.L = L
        self.path = path

    def gemm(self, op, dt, A, B, m, k, n, bias=None, rows=None, want_r=False, want_S=False):
        """Evaluate output rows of op in {"fwd","dx","dw"}; shapes are always (m,k,n) of the forward.

        fwd: A = X[m,k], B = W[k,n] -> Y[m,n] (+ bias[n]);  dx: A = dY[m,n], B = W[k,n] -> dX[m,k];
        dw : A = X[m,k], B = dY[m,n] -> dW[k,n].  Returns (y, r, S); r and S are float64 or None.
        """
        o = OPS[op]
        a_shape = (m, k) if op in ("fwd", "dw") else (m, n)
        b_shape = (k, n) if op in ("fwd", "dx") else (m, n)
        _check(A, dt, a_shape, "A")
        _check(B, dt, b_shape, "B")
        if bias is not None:
            _check(bias, dt, (n,), "bias")
        out_rows = k if op == "dw" else m
        cols = k if op == "dx" else n
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            nrows = rows.shape[0]
        else:
            nrows = out_rows
        y = np.zeros((nrows, cols), dtype=STORAGE[dt])
        r = np.zeros((nrows, cols), dtype=np.float64) if want_r else None
        S = np.zeros((nrows, cols), dtype=np.float64) if want_S else None
        rc = self.L.oracle_gemm(o, DTYPES[dt], _ptr(A), _ptr(B), _ptr(bias), m, k, n,
                                _ptr(rows), nrows, _ptr(y), _ptr(r), _ptr(S))
        if rc != 0:
            raise ValueError("oracle_gemm rejected its arguments")
        return y, r, S

    def fwd(self, dt, x, w, bias=None, rows=None, **kw):
        m, k = x.shape
        return self.gemm("fwd", dt, x, w, m, k, w.shape[1], bias=bias, rows=rows, **kw)

    def dx(self, dt, dy, w, rows=None, **kw):
        m, n = dy.shape
        return self.gemm("dx", dt, dy, w, m, w.shape[0], n, rows=rows, **kw)

    def dw(self, dt, x, dy, rows=None, **kw):
        m, k = x.shape
        return self.gemm("dw", dt, x, dy, m, k, dy.shape[1], rows=rows, **kw)

    def dw_out(self, dt, out_dt, x, dy, rows=None, **kw):
        """dW rounded once to out_dt (dt itself, or "f32" for f32 master weights): the float64
        value r of dw, then one RNE rounding to out_dt. Returns (y, r, S) like gemm."""
        _, r, S = self.dw(dt, x, dy, rows=rows, want_r=True, want_S=kw.get("want_S", False))
        return self.round_to(out_dt, r), (r if kw.get("want_r") else None), S

    def db(self, dt, dy, out_dt=None, want_r=False, want_S=False):
        """Bias gradient db[n] = sum_i dy[i, n], defined as dW of a column of ones (the
        reduction over i in tiles of 32 rows, Neumaier across tiles), rounded once to out_dt
        (default dt). Returns (y[n], r[n] or None, S[n] or None)."""
        m, n = dy.shape
        ones = self.round_to(dt, np.ones((m, 1)))
        _, r, S = self.gemm("dw", dt, ones, dy, m, 1, n, want_r=True, want_S=want_S)
        y = self.round_to(out_dt or dt, r[0])
        return y, (r[0] if want_r else None), (S[0] if want_S else None)

    def gemm_cr(self, op, dt, A, B, m, k, n, bias=None, rows=None):
        """Correctly rounded tier: each output is the exact value of its dot product (+ bias)
        rounded once (RNE) to dt. Shapes and operands as gemm; returns y."""
        a_shape = (m, k) if op in ("fwd", "dw") else (m, n)
        b_shape = (k, n) if op in ("fwd", "dx") else (m, n)
        _check(A, dt, a_shape, "A")
        _check(B, dt, b_shape, "B")
        if bias is not None:
            _check(bias, dt, (n,), "bias")
        out_rows = k if op == "dw" else m
        cols = k if op == "dx" else n
        if rows is not None:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            nrows = rows.shape[0]
        else:
            nrows = out_rows
        y = np.zeros((nrows, cols), dtype=STORAGE[dt])
        if self.L.oracle_gemm_cr(OPS[op], DTYPES[dt], _ptr(A), _ptr(B), _ptr(bias), m, k, n, _ptr(rows), nrows,
                                 _ptr(y)) != 0:
            raise ValueError("oracle_gemm_cr rejected its arguments")
        return y

    def exact_sum(self, dt, values):
        """The exact sum of float64 values rounded once to dt (raw storage scalar)."""
        v = np.ascontiguousarray(values, dtype=np.float64)
        out = np.zeros(1, dtype=STORAGE[dt])
        if self.L.oracle_exact_sum(_ptr(v) if v.size else None, v.size, DTYPES[dt], _ptr(out)) != 0:
            raise ValueError("oracle_exact_sum rejected its arguments")
        return out[0]

    def layernorm_fwd(self, dt, x, gamma=None, beta=None, eps=1e-5, want_r=False):
        """LayerNorm over the last dim of x[rows, h] with float64 statistics (the row sums are
        the matmul's tiled compensated sum). Returns (y, mean, rstd, r or None)."""
        rows, h = x.shape
        _check(x, dt, (rows, h), "x")
        for v, name in ((gamma, "gamma"), (beta, "beta")):
            if v is not None:
                _check(v, dt, (h,), name)
        y = np.zeros((rows, h), dtype=STORAGE[dt])
        mean = np.zeros(rows)
        rstd = np.zeros(rows)
        r = np.zeros((rows, h)) if want_r else None
        if self.L.oracle_layernorm_fwd(DTYPES[dt], _ptr(x), _ptr(gamma), _ptr(beta), rows, h, float(eps),
                                       _ptr(y), _ptr(mean), _ptr(rstd), _ptr(r)) != 0:
            raise ValueError("oracle_layernorm_fwd rejected its arguments")
        return y, mean, rstd, r

    def layernorm_bwd(self, dt, dy, x, mean, rstd, gamma=None, pdt=None, want_r=False):
        """Gradients of layernorm_fwd: (dx in dt, dgamma and dbeta in pdt (default dt), r of dx or None)."""
        rows, h = x.shape
        _check(x, dt, (rows, h), "x")
        _check(dy, dt, (rows, h), "dy")
        if gamma is not None:
            _check(gamma, dt, (h,), "gamma")
        mean = np.ascontiguousarray(mean, dtype=np.float64)
        rstd = np.ascontiguousarray(rstd, dtype=np.float64)
        if mean.shape != (rows,) or rstd.shape != (rows,):
            raise ValueError("oracle: mean and rstd must have one value per row")
        pdt = pdt or dt
        dx = np.zeros((rows, h), dtype=STORAGE[dt])
        dg = np.zeros(h, dtype=STORAGE[pdt])
        dbt = np.zeros(h, dtype=STORAGE[pdt])
        r = np.zeros((rows, h)) if want_r else None
        if self.L.oracle_layernorm_bwd(DTYPES[dt], DTYPES[pdt], _ptr(dy), _ptr(x), _ptr(mean), _ptr(rstd),
                                       _ptr(gamma), rows, h, _ptr(dx), _ptr(dg), _ptr(dbt), _ptr(r)) != 0:
            raise ValueError("oracle_layernorm_bwd rejected its arguments")
        return dx, dg, dbt, r

    def round_to(self, dt, r):
        """Single RNE rounding of float64 values to dt (raw storage out)."""
        r = np.ascontiguousarray(r, dtype=np.float64)
        out = np.zeros(r.shape, dtype=STORAGE[dt])
        if self.L.oracle_round(_ptr(r), r.size, DTYPES[dt], _ptr(out)) != 0:
            raise ValueError("oracle_round rejected its arguments")
        return out


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(a, dt, shape, name):
    if a.dtype != STORAGE[dt] or tuple(a.shape) != tuple(shape) or not a.flags.c_contiguous:
        raise ValueError(f"oracle: {name} must be a C-contiguous {STORAGE[dt].__name__} array of shape {shape}")


_default = None


def default():
    """The oracle built from oracle.cpp in this directory (built on first use if absent)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB):
            _build()
        _default = Oracle(LIB)
    return _default


def gemm(*a, **kw):
    return default().gemm(*a, **kw)


def fwd(*a, **kw):
    return default().fwd(*a, **kw)


def dx(*a, **kw):
    return default().dx(*a, **kw)


def dw(*a, **kw):
    return default().dw(*a, **kw)


def round_to(*a, **kw):
    return default().round_to(*a, **kw)


def dw_out(*a, **kw):
    return default().dw_out(*a, **kw)


def db(*a, **kw):
    return default().db(*a, **kw)


def layernorm_fwd(*a, **kw):
    return default().layernorm_fwd(*a, **kw)


def layernorm_bwd(*a, **kw):
    return default().layernorm_bwd(*a, **kw)


def gemm_cr(*a, **kw):
    return default().gemm_cr(*a, **kw)


def exact_sum(*a, **kw):
    return default().exact_sum(*a, **kw)
