"""ctypes binding of libw4a8_probe.so: roofline probes timed with HIP events
on the current stream (argument marshalling and timing only)."""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libw4a8_probe.so")
_lib = None

MFMA_FLOPS = 2 * 16 * 16 * 128  # one v_mfma_scale_f32_16x16x128_f8f6f4


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built (python -m moe_grouped_precision_amd.build)")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.w4a8_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
        lib.w4a8_probe_mfma.restype = ctypes.c_int
        lib.w4a8_probe_mfma_data.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.w4a8_probe_mfma_data.restype = ctypes.c_int
        lib.w4a8_probe_mfma_promote.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p]
        lib.w4a8_probe_mfma_promote.restype = ctypes.c_int
        lib.w4a8_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
        lib.w4a8_probe_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def _time(fn, reps):
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(x.elapsed_time(y) for x, y in ts)
    return ms[len(ms) // 2]


def mfma_tflops(fmt_a: int, fmt_b: int, iters: int = 4096, reps: int = 5) -> float:
    """Sustained TFLOP/s of the scaled 16x16x128 MFMA for a format pair
    (0 = FP8 E4M3, 4 = FP4 E2M1), eight waves per SIMD."""
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * 8
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        st = lib.w4a8_probe_mfma(fmt_a, fmt_b, iters, blocks, ctypes.c_void_p(sink.data_ptr()), stream)
        if st != 0:
            raise RuntimeError(f"w4a8_probe_mfma status {st}")

    ms = _time(run, reps)
    flops = blocks * 4 * iters * 8 * MFMA_FLOPS
    return flops / (ms * 1e-3) / 1e12


def mfma_tflops_random(fmt_a: int, fmt_b: int, iters: int = 4096, reps: int = 5, seed: int = 0) -> float:
    """Sustained TFLOP/s of the same MFMA stream on random operand bits (one
    set per thread, fixed over the loop), eight waves per SIMD."""
    lib = load()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks = cus * 8
    g = torch.Generator(device="cuda").manual_seed(seed)
    ops = torch.randint(-2**31, 2**31 - 1, (blocks * 256 * 16,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        st = lib.w4a8_probe_mfma_data(fmt_a, fmt_b, iters, blocks, ctypes.c_void_p(ops.data_ptr()),
                                      ctypes.c_void_p(sink.data_ptr()), stream)
        if st != 0:
            raise RuntimeError(f"w4a8_probe_mfma_data status {st}")

    ms = _time(run, reps)
    flops = blocks * 4 * iters * 8 * MFMA_FLOPS
    return flops / (ms * 1e-3) / 1e12


def mfma_promote_tflops(promote: bool, iters: int = 4096, reps: int = 5, seed: int = 0) -> float:
    """Sustained TFLOP/s (MFMA flops only) of the GEMM's MFMA-phase pattern
    without memory traffic: FP4 x FP8 MFMAs with a zero accumulator input on
    random operands, each followed (promote) by four fp32 promotion FMAs;
    one 512-thread workgroup per CU (two waves per SIMD, as the GEMM)."""
    lib = load()
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    g = torch.Generator(device="cuda").manual_seed(seed)
    ops = torch.randint(-2**31, 2**31 - 1, (blocks * 512 * 16,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        st = lib.w4a8_probe_mfma_promote(int(promote), iters, blocks, ctypes.c_void_p(ops.data_ptr()),
                                         ctypes.c_void_p(sink.data_ptr()), stream)
        if st != 0:
            raise RuntimeError(f"w4a8_probe_mfma_promote status {st}")

    ms = _time(run, reps)
    flops = blocks * 8 * iters * 8 * MFMA_FLOPS
    return flops / (ms * 1e-3) / 1e12


def read_gbs(nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Sustained GB/s of a plain streaming read of nbytes (larger than the
    last-level cache, so the reads come from HBM): one workgroup of 256
    threads per CU, eight nontemporal 16-byte loads in flight per thread (32
    KB per CU), the fastest of the launch shapes measured (more bytes in
    flight per CU read slower)."""
    lib = load()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def run():
        st = lib.w4a8_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, cus,
                                 ctypes.c_void_p(sink.data_ptr()), stream)
        if st != 0:
            raise RuntimeError(f"w4a8_probe_read status {st}")

    ms = _time(run, reps)
    del buf
    return nbytes / (ms * 1e-3) / 1e9
