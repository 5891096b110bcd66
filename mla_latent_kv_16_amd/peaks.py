"""Same-run achievable peaks of the device, from libmla_peaks.so (include/mla_peaks.h).

measure(torch, dev) returns
  hbm_stream_read_GBps    plain 16-byte vector loads over a 4 GiB buffer
  lds_dma_stream_GBps     the split-KV kernel's own load path (direct global->LDS
                          copies into a four-slot 36 KB ring, one workgroup per CU)
                          over the same buffer
  mfma_bf16_TFLOPs        v_mfma_f32_32x32x16_bf16 chains on register operands
each the mean over back-to-back launches timed with HIP events on the current
stream, after untimed launches.  ctypes marshalling only; the kernels are HIP.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_peaks.so")
STREAM_BYTES = 4 << 30

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mla_latent_kv_16_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        for name in ("mla_peak_stream_read", "mla_peak_dma_stream"):
            getattr(L, name).argtypes = [vp, sz, vp, i32, vp]
            getattr(L, name).restype = i32
        L.mla_peak_dma_stream_bytes.argtypes = [sz, i32]
        L.mla_peak_dma_stream_bytes.restype = sz
        L.mla_peak_mfma_bf16.argtypes = [i32, vp, i32, vp]
        L.mla_peak_mfma_bf16.restype = i32
        L.mla_peak_mfma_bf16_flops.argtypes = [i32, i32]
        L.mla_peak_mfma_bf16_flops.restype = ctypes.c_double
        _lib = L
    return _lib


def _timed(torch, launch, reps, warm=2):
    for _ in range(warm):
        launch()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        launch()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3 / reps


def measure(torch, dev, cus=None):
    L = lib()
    cus = cus or torch.cuda.get_device_properties(dev).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    buf = torch.empty(STREAM_BYTES, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    bp, sp = ctypes.c_void_p(buf.data_ptr()), ctypes.c_void_p(sink.data_ptr())

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what} returned {st}")

    wg_stream = cus * 8
    t_read = _timed(torch, lambda: check(L.mla_peak_stream_read(bp, STREAM_BYTES, sp, wg_stream,
                                                                 stream), "stream read"), 10)
    dma_bytes = L.mla_peak_dma_stream_bytes(STREAM_BYTES, cus)
    t_dma = _timed(torch, lambda: check(L.mla_peak_dma_stream(bp, STREAM_BYTES, sp, cus, stream),
                                        "dma stream"), 10)
    del buf
    iters, wg_mfma = 2000, cus * 8
    t_mfma = _timed(torch, lambda: check(L.mla_peak_mfma_bf16(iters, sp, wg_mfma, stream),
                                         "mfma"), 5)
    flops = L.mla_peak_mfma_bf16_flops(iters, wg_mfma)
    torch.cuda.synchronize()
    del sink
    return {"hbm_stream_read_GBps": round(STREAM_BYTES / t_read / 1e9, 1),
            "lds_dma_stream_GBps": round(dma_bytes / t_dma / 1e9, 1),
            "mfma_bf16_TFLOPs": round(flops / t_mfma / 1e12, 1),
            "how": f"HIP microbenchmarks of libmla_peaks.so: {STREAM_BYTES >> 30} GiB read with "
                   f"16-byte loads ({wg_stream} workgroups) and with the split-KV kernel's "
                   f"global->LDS copies ({cus} workgroups); {wg_mfma} workgroups x 4 waves of "
                   f"bf16 32x32x16 MFMA chains"}
