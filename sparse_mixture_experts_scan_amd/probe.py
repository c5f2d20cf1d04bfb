"""ctypes binding of libmoe_probe.so (include/moe_probe.h): HBM-read, copy
and bf16-MFMA microbenchmarks that give measured ceilings beside MI355X's
datasheet peaks.  Argument marshalling only; raises if the library is not
built."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(PKG, "libmoe_probe.so")
EXPORTED = ("moe_probe_read", "moe_probe_copy", "moe_probe_mfma", "moe_probe_mfma_flops")

_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is not built: run "
                               "`python -m sparse_mixture_experts_scan_amd.build` first")
        L = ctypes.CDLL(PROBE_LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.moe_probe_read.argtypes = [vp, sz, vp, i32, vp]
        L.moe_probe_read.restype = i32
        L.moe_probe_copy.argtypes = [vp, vp, sz, i32, vp]
        L.moe_probe_copy.restype = i32
        L.moe_probe_mfma.argtypes = [vp, i32, i32, vp]
        L.moe_probe_mfma.restype = i32
        L.moe_probe_mfma_flops.argtypes = [i32, i32]
        L.moe_probe_mfma_flops.restype = ctypes.c_double
        _lib = L
    return _lib


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed")


def measured_peaks(device=None, read_gib: int = 4, reps: int = 5) -> dict:
    """Time the three microbenchmarks on the current torch stream and return
    {"hbm_read_GBs", "hbm_copy_GBs", "mfma_bf16_TFLOPs"} (best of `reps`
    launches each) with a description of each."""
    import torch
    dev = device or torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev)
    s = ctypes.c_void_p(stream.cuda_stream)
    L = lib()
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    nbytes = read_gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    src.fill_(1)
    blocks = cus * 16
    sink = torch.empty(max(blocks, cus * 8 * 8), dtype=torch.int32, device=dev)

    def timed(fn):
        best = float("inf")
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            best = min(best, a.elapsed_time(b) * 1e-3)
        return best

    _check(L.moe_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, s), "read probe")
    t_read = timed(lambda: _check(L.moe_probe_read(src.data_ptr(), nbytes, sink.data_ptr(),
                                                   blocks, s), "read probe"))
    half = nbytes // 2
    t_copy = timed(lambda: _check(L.moe_probe_copy(src.data_ptr(), src.data_ptr() + half, half,
                                                   blocks, s), "copy probe"))
    del src
    mblocks, iters = cus, 16384
    fsink = torch.empty(mblocks * 8, dtype=torch.float32, device=dev)
    _check(L.moe_probe_mfma(fsink.data_ptr(), mblocks, 16, s), "mfma probe")
    t_mfma = timed(lambda: _check(L.moe_probe_mfma(fsink.data_ptr(), mblocks, iters, s),
                                  "mfma probe"))
    flops = L.moe_probe_mfma_flops(mblocks, iters)
    torch.cuda.synchronize()
    return {
        "hbm_read_GBs": nbytes / t_read / 1e9,
        "hbm_copy_GBs": 2 * half / t_copy / 1e9,
        "mfma_bf16_TFLOPs": flops / t_mfma / 1e12,
        "how": (f"best of {reps}: a {read_gib} GiB 16-byte streaming read over {blocks} blocks; "
                f"a {read_gib // 2} GiB copy (read + write bytes); {mblocks} blocks x 8 waves "
                f"x {iters} x 8 independent v_mfma_f32_32x32x16_bf16 on register operands"),
    }
