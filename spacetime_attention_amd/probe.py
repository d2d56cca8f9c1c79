"""The matrix-core rate probe (libvdit_probe.so, declared in include/vdit_probe.h).

It is no part of the attention path: the benchmark calls it to state, on the
same device and in the same run, the bf16 MFMA rate the part sustains with
near-constant operands and with random full-mantissa operands. Device memory
and the stream come from PyTorch; the kernel and its timing counters are the
library's.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(_HERE, "libvdit_probe.so")
PROBE_EXPORTS = ("vdit_probe_mfma_bf16",)
FLOP_PER_MFMA = 32 * 32 * 16 * 2   # v_mfma_f32_32x32x16_bf16
SIMDS = 256 * 4                    # 256 compute units x 4 SIMDs

_plib = None


def load_probe_library(path: str = PROBE_LIB_PATH) -> ctypes.CDLL:
    global _plib
    if _plib is not None:
        return _plib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m spacetime_attention_amd.build`")
    lib = ctypes.CDLL(path)
    lib.vdit_probe_mfma_bf16.restype = ctypes.c_int
    lib.vdit_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
    _plib = lib
    return lib


def mfma_rate(random_operands: bool, launches: int = 4, warmup: int = 8, iters: int = 10000,
              nblocks: int = 2048) -> dict:
    """Sustained v_mfma_f32_32x32x16_bf16 rate over `launches` timed launches,
    after `warmup` untimed ones (~100 ms, which lets the clock settle)."""
    import torch

    lib = load_probe_library()
    ticks = torch.zeros(2 * nblocks, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def launch():
        rc = lib.vdit_probe_mfma_bf16(1 if random_operands else 0, iters, nblocks,
                                      ctypes.c_void_p(ticks.data_ptr()), sp)
        if rc != 0:
            raise RuntimeError(f"vdit_probe_mfma_bf16 returned {rc}")

    for _ in range(warmup):
        launch()
    torch.cuda.synchronize()
    ms, clk = [], []
    for _ in range(launches):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
        t = ticks.view(nblocks, 2).double().sum(0).tolist()
        clk.append(t[0] / t[1] * 100.0)   # shader clocks per 10 ns tick -> MHz
    flop = float(nblocks) * 4 * 8 * iters * FLOP_PER_MFMA
    ms_mean = sum(ms) / len(ms)
    mhz = sum(clk) / len(clk)
    tflops = flop / ms_mean / 1e9
    # Clocks between MFMA issues on one SIMD, all SIMDs busy.
    cyc = mhz * 1e6 * SIMDS * FLOP_PER_MFMA / (tflops * 1e12)
    return {"tflops": tflops, "clock_mhz": mhz, "clocks_per_mfma": cyc, "ms": ms_mean}
