"""Python binding of libdetgemm.so: argument marshalling only.

The C entry points (include/det_gemm.h) are exposed under the same names and
take raw device pointers (ints) or torch tensors, plus an explicit stream, as
the sgemm-bi 0.1.2 PyPI page's low-level engine does ("Use": raw pointers,
explicit stream). On top of them sit a functional form, an autograd function
and a drop-in layer with the weight stored [in, out] (same page, "Use"). Every
GEMM runs in the library's HIP kernels; there is no fallback path, and a
missing library raises at first use.
"""
import ctypes
import os

__all__ = [
    "det_gemm_fwd", "det_gemm_dx", "det_gemm_dw", "det_gemm_dw_out", "det_gemm_dw_noalloc", "det_gemm_db",
    "det_gemm_strerror",
    "det_gemm_last_error", "det_gemm_version", "det_gemm_debug_force_family", "det_gemm_debug_force_exact_kernel",
    "det_gemm_debug_force_db_chunk", "det_gemm_debug_force_cr_fallback", "det_gemm_debug_force_arch",
    "det_gemm_debug_round_f32", "det_gemm_debug_round_f64", "det_gemm_debug_round_f64_grouped", "DetGemmError", "LIB_PATH", "fwd", "dx", "dw", "db", "deterministic_linear", "Linear", "DTYPES", "TIERS",
    "det_layernorm_fwd", "det_layernorm_bwd", "layer_norm", "layer_norm_backward", "deterministic_layer_norm",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdetgemm.so")

DTYPES = {"f32": 0, "bf16": 1, "f16": 2}
TIERS = {"exact": 0, "fast": 1, "cr": 2}
STATUS = {0: "DET_OK", -1: "DET_EINVAL", -2: "DET_EDTYPE", -3: "DET_ETIER", -4: "DET_EDEVICE", -5: "DET_ELAUNCH"}


class DetGemmError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libdetgemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        # torch bundles its own HIP runtime (same soname). Load it first so that
        # libdetgemm.so binds to that one runtime instead of a second copy from
        # /opt/rocm, which would not know torch's device memory or streams.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                              "(hipcc, gfx950); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.det_gemm_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.det_gemm_dx.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.det_gemm_dw.argtypes = [vp, vp, vp, i64, i64, i64, ci, ci, vp]
        L.det_gemm_dw_out.argtypes = [vp, ci, vp, vp, i64, i64, i64, ci, ci, vp]
        L.det_gemm_dw_noalloc.argtypes = [vp, ci, vp, vp, i64, i64, i64, ci, ci, vp]
        L.det_gemm_db.argtypes = [vp, ci, vp, i64, i64, ci, ci, vp]
        L.det_layernorm_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, ctypes.c_double, ci, vp]
        L.det_layernorm_bwd.argtypes = [vp, vp, vp, ci, vp, vp, vp, vp, vp, i64, i64, ci, vp]
        for f in (L.det_gemm_fwd, L.det_gemm_dx, L.det_gemm_dw, L.det_gemm_dw_out, L.det_gemm_dw_noalloc, L.det_gemm_db,
                  L.det_layernorm_fwd, L.det_layernorm_bwd):
            f.restype = ci
        L.det_gemm_strerror.argtypes = [ci]
        L.det_gemm_strerror.restype = ctypes.c_char_p
        L.det_gemm_last_error.argtypes = []
        L.det_gemm_last_error.restype = ctypes.c_char_p
        L.det_gemm_version.restype = ci
        L.det_gemm_debug_force_family.argtypes = [ci]
        L.det_gemm_debug_force_family.restype = ci
        L.det_gemm_debug_force_exact_kernel.argtypes = [ci]
        L.det_gemm_debug_force_exact_kernel.restype = ci
        L.det_gemm_debug_force_db_chunk.argtypes = [i64]
        L.det_gemm_debug_force_db_chunk.restype = ci
        L.det_gemm_debug_force_cr_fallback.argtypes = [ci]
        L.det_gemm_debug_force_cr_fallback.restype = ci
        L.det_gemm_debug_force_arch.argtypes = [ctypes.c_char_p]
        L.det_gemm_debug_force_arch.restype = ci
        L.det_gemm_debug_round_f32.argtypes = [vp, ctypes.c_uint32, i64, ci, vp]
        L.det_gemm_debug_round_f32.restype = ci
        L.det_gemm_debug_round_f64.argtypes = [vp, vp, i64, ci, vp]
        L.det_gemm_debug_round_f64.restype = ci
        L.det_gemm_debug_round_f64_grouped.argtypes = [vp, vp, i64, ci, vp]
        L.det_gemm_debug_round_f64_grouped.restype = ci
        _lib = L
    return _lib


def _p(v):
    """Pointer value of a torch tensor, an int or None."""
    if v is None:
        return None
    if isinstance(v, int):
        return v
    return v.data_ptr()


def _code(table, v, what):
    if isinstance(v, int):
        return v
    try:
        return table[v]
    except KeyError:
        raise ValueError(f"unknown {what} {v!r}") from None


def _check(status):
    if status != 0:
        raise DetGemmError(status, lib().det_gemm_last_error().decode())


def det_gemm_fwd(y, x, w, bias, m, k, n, dtype, tier, stream=0):
    _check(lib().det_gemm_fwd(_p(y), _p(x), _p(w), _p(bias), m, k, n,
                              _code(DTYPES, dtype, "dtype"), _code(TIERS, tier, "tier"), _p(stream)))


def det_gemm_dx(dx_, dy, w, m, k, n, dtype, tier, stream=0):
    _check(lib().det_gemm_dx(_p(dx_), _p(dy), _p(w), m, k, n,
                             _code(DTYPES, dtype, "dtype"), _code(TIERS, tier, "tier"), _p(stream)))


def det_gemm_dw(dw_, x, dy, m, k, n, dtype, tier, stream=0):
    _check(lib().det_gemm_dw(_p(dw_), _p(x), _p(dy), m, k, n,
                             _code(DTYPES, dtype, "dtype"), _code(TIERS, tier, "tier"), _p(stream)))


def det_gemm_dw_out(dw_, dw_dtype, x, dy, m, k, n, dtype, tier, stream=0):
    _check(lib().det_gemm_dw_out(_p(dw_), _code(DTYPES, dw_dtype, "dtype"), _p(x), _p(dy), m, k, n,
                                 _code(DTYPES, dtype, "dtype"), _code(TIERS, tier, "tier"), _p(stream)))


def det_gemm_dw_noalloc(dw_, dw_dtype, x, dy, m, k, n, dtype, tier, stream=0):
    _check(lib().det_gemm_dw_noalloc(_p(dw_), _code(DTYPES, dw_dtype, "dtype"), _p(x), _p(dy), m, k, n,
                                     _code(DTYPES, dtype, "dtype"), _code(TIERS, tier, "tier"), _p(stream)))


def det_gemm_db(db_, db_dtype, dy, m, n, dtype, tier, stream=0):
    _check(lib().det_gemm_db(_p(db_), _code(DTYPES, db_dtype, "dtype"), _p(dy), m, n,
                             _code(DTYPES, dtype, "dtype"), _code(TIERS, tier, "tier"), _p(stream)))


def det_layernorm_fwd(y, mean, rstd, x, gamma, beta, rows, h, eps, dtype, stream=0):
    _check(lib().det_layernorm_fwd(_p(y), _p(mean), _p(rstd), _p(x), _p(gamma), _p(beta), rows, h, float(eps),
                                   _code(DTYPES, dtype, "dtype"), _p(stream)))


def det_layernorm_bwd(dx, dgamma, dbeta, param_dtype, dy, x, mean, rstd, gamma, rows, h, dtype, stream=0):
    _check(lib().det_layernorm_bwd(_p(dx), _p(dgamma), _p(dbeta), _code(DTYPES, param_dtype, "dtype"), _p(dy), _p(x),
                                   _p(mean), _p(rstd), _p(gamma), rows, h, _code(DTYPES, dtype, "dtype"), _p(stream)))


def det_gemm_strerror(status):
    return lib().det_gemm_strerror(status).decode()


def det_gemm_last_error():
    return lib().det_gemm_last_error().decode()


def det_gemm_version():
    return lib().det_gemm_version()


def det_gemm_debug_force_family(family):
    _check(lib().det_gemm_debug_force_family(family))


def det_gemm_debug_force_exact_kernel(variant):
    _check(lib().det_gemm_debug_force_exact_kernel(variant))


def det_gemm_debug_force_db_chunk(tiles):
    _check(lib().det_gemm_debug_force_db_chunk(tiles))


def det_gemm_debug_force_cr_fallback(on):
    _check(lib().det_gemm_debug_force_cr_fallback(int(on)))


def det_gemm_debug_force_arch(arch):
    """Test hook: check `arch` (a string) instead of the device's architecture; None restores it."""
    _check(lib().det_gemm_debug_force_arch(None if arch is None else arch.encode()))


def det_gemm_debug_round_f32(first, count, dt, device="cuda:0"):
    """Test hook: the fast tier's output rounding of the f32 values with bits
    first .. first + count - 1 (mod 2^32), on the device; returns a uint16 (bf16,
    f16) or float32 (f32) tensor of raw output bits."""
    import torch
    storage = torch.float32 if dt == "f32" else torch.int16
    out = torch.empty(count, dtype=storage, device=device)
    stream = torch.cuda.current_stream(out.device).cuda_stream
    _check(lib().det_gemm_debug_round_f32(_p(out), first & 0xffffffff, count, DTYPES[dt], stream))
    return out


def _debug_round_f64(fn, values, dt):
    import torch
    if values.dtype != torch.float64 or not values.is_cuda or not values.is_contiguous():
        raise ValueError("values must be a contiguous float64 device tensor")
    storage = torch.float32 if dt == "f32" else torch.int16
    out = torch.empty(values.numel(), dtype=storage, device=values.device)
    stream = torch.cuda.current_stream(values.device).cuda_stream
    _check(fn(_p(out), _p(values), values.numel(), DTYPES[dt], stream))
    return out


def det_gemm_debug_round_f64(values, dt):
    """Test hook: the exact tier's output rounding of a float64 device tensor, on
    the device; returns raw output bits as int16 (bf16, f16) or float32 (f32)."""
    return _debug_round_f64(lib().det_gemm_debug_round_f64, values, dt)


def det_gemm_debug_round_f64_grouped(values, dt):
    """Test hook: the LayerNorm forward's grouped rounding of the same values
    (eight per lane); the bits must equal det_gemm_debug_round_f64's."""
    return _debug_round_f64(lib().det_gemm_debug_round_f64_grouped, values, dt)


# ---------------------------------------------------------------- torch layer

def _torch_dtype_name(t):
    import torch
    names = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}
    if t.dtype not in names:
        raise TypeError(f"unsupported dtype {t.dtype}; use float32, bfloat16 or float16")
    return names[t.dtype]


def _prep(*ts):
    import torch
    out = []
    dev = None
    for t in ts:
        if t is None:
            out.append(None)
            continue
        if not t.is_cuda:
            raise ValueError("det_gemm operates on device tensors")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")
        out.append(t.contiguous())
    if len({t.dtype for t in out if t is not None}) != 1:
        raise TypeError("all tensors must share one dtype")
    return out, torch.cuda.current_stream(dev).cuda_stream


def _out(out, shape, dtype, device):
    """The output tensor: a new one, or the caller's `out` after checking that the kernels may
    write exactly shape x dtype into it (contiguous, on the operands' device); a mismatch raises
    ValueError before anything is launched."""
    import torch
    if out is None:
        return torch.empty(shape, dtype=dtype, device=device)
    if out.dtype != dtype or tuple(out.shape) != tuple(shape) or not out.is_contiguous() or out.device != device:
        raise ValueError(f"out must be a contiguous {tuple(shape)} tensor of {dtype} on {device}; got "
                         f"{tuple(out.shape)} {out.dtype} on {out.device} (contiguous={out.is_contiguous()})")
    return out


def fwd(x, w, bias=None, tier="exact", out=None):
    """y[m,n] = x[m,k] @ w[k,n] (+ bias[n]) on the current stream."""
    (x, w, bias), stream = _prep(x, w, bias)
    m, k = x.shape
    k2, n = w.shape
    if k2 != k or (bias is not None and tuple(bias.shape) != (n,)):
        raise ValueError("shape mismatch")
    y = _out(out, (m, n), x.dtype, x.device)
    det_gemm_fwd(y, x, w, bias, m, k, n, _torch_dtype_name(x), tier, stream)
    return y


def dx(dy, w, tier="exact", out=None):
    """dx[m,k] = dy[m,n] @ w[k,n]^T on the current stream."""
    (dy, w), stream = _prep(dy, w)
    m, n = dy.shape
    k, n2 = w.shape
    if n2 != n:
        raise ValueError("shape mismatch")
    g = _out(out, (m, k), dy.dtype, dy.device)
    det_gemm_dx(g, dy, w, m, k, n, _torch_dtype_name(dy), tier, stream)
    return g


def dw(x, dy, tier="exact", out=None, out_dtype=None):
    """dw[k,n] = x[m,k]^T @ dy[m,n] on the current stream; out_dtype=torch.float32 writes
    f32 gradients (for f32 master weights) from bf16/f16 inputs."""
    import torch
    (x, dy), stream = _prep(x, dy)
    m, k = x.shape
    m2, n = dy.shape
    if m2 != m:
        raise ValueError("shape mismatch")
    odt = out_dtype or x.dtype
    g = _out(out, (k, n), odt, x.device)
    if odt == x.dtype:
        det_gemm_dw(g, x, dy, m, k, n, _torch_dtype_name(x), tier, stream)
    else:
        det_gemm_dw_out(g, _torch_dtype_name(g), x, dy, m, k, n, _torch_dtype_name(x), tier, stream)
    return g


def db(dy, tier="exact", out=None, out_dtype=None):
    """db[n] = sum_i dy[i,n] on the current stream (the exact tier's column sum in either tier);
    out_dtype=torch.float32 writes f32 from bf16/f16 inputs."""
    import torch
    (dy,), stream = _prep(dy)
    m, n = dy.shape
    odt = out_dtype or dy.dtype
    g = _out(out, (n,), odt, dy.device)
    det_gemm_db(g, _torch_dtype_name(g), dy, m, n, _torch_dtype_name(dy), tier, stream)
    return g


def layer_norm(x, gamma=None, beta=None, eps=1e-5, out=None):
    """LayerNorm over the last dim of x[rows, h] with float64 statistics on the current stream.
    Returns (y, mean, rstd); mean and rstd are float64 [rows] for layer_norm_backward."""
    import torch
    (x, gamma, beta), stream = _prep(x, gamma, beta)
    rows, h = x.shape
    for v in (gamma, beta):
        if v is not None and tuple(v.shape) != (h,):
            raise ValueError("gamma and beta must have h elements")
    y = _out(out, (rows, h), x.dtype, x.device)
    mean = torch.empty(rows, dtype=torch.float64, device=x.device)
    rstd = torch.empty(rows, dtype=torch.float64, device=x.device)
    det_layernorm_fwd(y, mean, rstd, x, gamma, beta, rows, h, eps, _torch_dtype_name(x), stream)
    return y, mean, rstd


def layer_norm_backward(dy, x, mean, rstd, gamma=None, param_dtype=None, need_dx=True, need_params=True):
    """(dx, dgamma, dbeta) of layer_norm; dgamma/dbeta in param_dtype (x's dtype or torch.float32)."""
    import torch
    (dy, x, gamma), stream = _prep(dy, x, gamma)
    rows, h = x.shape
    if tuple(dy.shape) != (rows, h) or mean.dtype != torch.float64 or rstd.dtype != torch.float64:
        raise ValueError("dy must match x; mean and rstd must be float64")
    mean, rstd = mean.contiguous(), rstd.contiguous()
    pdt = param_dtype or x.dtype
    gx = torch.empty_like(x) if need_dx else None
    gg = torch.empty(h, dtype=pdt, device=x.device) if need_params and gamma is not None else None
    gb = torch.empty(h, dtype=pdt, device=x.device) if need_params else None
    det_layernorm_bwd(gx, gg, gb, _torch_dtype_name(gb if gb is not None else x), dy, x, mean, rstd, gamma,
                      rows, h, _torch_dtype_name(x), stream)
    return gx, gg, gb


def _autograd_fn():
    import torch

    class DeterministicLinearFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, weight, bias, tier):
            ctx.save_for_backward(x, weight)
            ctx.tier = tier
            ctx.has_bias = bias is not None
            return fwd(x, weight, bias, tier)

        @staticmethod
        def backward(ctx, gy):
            x, weight = ctx.saved_tensors
            gy = gy.contiguous()
            gx = dx(gy, weight, ctx.tier) if ctx.needs_input_grad[0] else None
            gw = dw(x, gy, ctx.tier) if ctx.needs_input_grad[1] else None
            gb = None
            if ctx.has_bias and ctx.needs_input_grad[2]:
                gb = db(gy, ctx.tier)   # column sum in the exact tier's fixed order
            return gx, gw, gb, None

    return DeterministicLinearFn


_FN = None
_LN = None


def _ln_fn():
    import torch

    class DeterministicLayerNormFn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, gamma, beta, eps):
            y, mean, rstd = layer_norm(x, gamma, beta, eps)
            ctx.save_for_backward(x, gamma, mean, rstd)
            ctx.has_beta = beta is not None
            return y

        @staticmethod
        def backward(ctx, gy):
            x, gamma, mean, rstd = ctx.saved_tensors
            need_params = ctx.needs_input_grad[1] or ctx.needs_input_grad[2]
            gx, gg, gb = layer_norm_backward(gy.contiguous(), x, mean, rstd, gamma,
                                             need_dx=ctx.needs_input_grad[0], need_params=need_params)
            return gx, gg, (gb if ctx.has_beta else None), None

    return DeterministicLayerNormFn


def deterministic_layer_norm(x, gamma=None, beta=None, eps=1e-5):
    """LayerNorm over the last dim (leading dims flattened) with float64 statistics, differentiable."""
    global _LN
    if _LN is None:
        _LN = _ln_fn()
    lead = x.shape[:-1]
    return _LN.apply(x.reshape(-1, x.shape[-1]), gamma, beta, eps).reshape(*lead, x.shape[-1])


def deterministic_linear(x, weight, bias=None, tier="exact"):
    """y = x @ weight (+ bias) with weight stored [in, out]; leading dims of x are flattened."""
    global _FN
    if _FN is None:
        _FN = _autograd_fn()
    lead = x.shape[:-1]
    y = _FN.apply(x.reshape(-1, x.shape[-1]), weight, bias, tier)
    return y.reshape(*lead, weight.shape[1])


def _make_linear():
    import torch

    class Linear(torch.nn.Module):
        """Drop-in linear layer with the weight stored [in_features, out_features]."""

        def __init__(self, in_features, out_features, bias=True, device=None, dtype=None, tier="exact"):
            super().__init__()
            self.in_features, self.out_features, self.tier = in_features, out_features, tier
            self.weight = torch.nn.Parameter(torch.empty((in_features, out_features), device=device, dtype=dtype))
            self.bias = torch.nn.Parameter(torch.zeros(out_features, device=device, dtype=dtype)) if bias else None
            bound = 1.0 / (in_features ** 0.5)
            with torch.no_grad():
                self.weight.uniform_(-bound, bound)

        @classmethod
        def from_torch(cls, layer, tier="exact"):
            m = cls(layer.in_features, layer.out_features, layer.bias is not None,
                    layer.weight.device, layer.weight.dtype, tier)
            with torch.no_grad():
                m.weight.copy_(layer.weight.t())
                if layer.bias is not None:
                    m.bias.copy_(layer.bias)
            return m

        def forward(self, x):
            return deterministic_linear(x, self.weight, self.bias, self.tier)

    return Linear


def __getattr__(name):
    if name == "Linear":
        cls = _make_linear()
        globals()["Linear"] = cls
        return cls
    raise AttributeError(name)
