"""Binding of libdetpeak.so (include/det_peak.h): the peak-rate microkernels the
benchmark states each tier against. Measurement only; the GEMM library does not
contain or load them."""
import ctypes
import os

PEAK_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdetpeak.so")
KINDS = {0: "float64 4x4x4 MFMA", 1: "float64 vector fma", 2: "bf16 32x32x16 MFMA"}

_lib = None


def lib():
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (bind to torch's HIP runtime first, as the GEMM library does)
        if not os.path.exists(PEAK_LIB_PATH):
            raise ImportError(f"{PEAK_LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(PEAK_LIB_PATH)
        L.det_peak_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int64,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
        L.det_peak_run.restype = ctypes.c_int
        _lib = L
    return _lib


def run(kind, iters, out, out_len, stream):
    """One microkernel launch; returns the flops it performs."""
    fl = ctypes.c_double(0.0)
    st = lib().det_peak_run(kind, iters, out if isinstance(out, int) else out.data_ptr(), out_len,
                            ctypes.byref(fl), stream)
    if st != 0:
        raise RuntimeError(f"det_peak_run({kind}) returned {st}")
    return fl.value


def measure(kind, iters, reps=5, device=None):
    """Sustained TFLOP/s of microkernel `kind` on the current stream: one warm-up launch, then
    `reps` launches between two events."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(cus * 512, dtype=torch.float64, device=dev)
    stream = torch.cuda.current_stream(dev)
    run(kind, iters, out, out.numel(), stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    flops = 0.0
    for _ in range(reps):
        flops += run(kind, iters, out, out.numel(), stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
