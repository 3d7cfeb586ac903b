"""Binding of the measurement probes (include/qa_probe.h, libqaprobe.so):
argument marshalling only. Used by bench.py to state practical ceilings."""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqaprobe.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: run quantized_attention_quantize_amd/build.py")
lib = ctypes.CDLL(_LIB_PATH)
lib.qa_probe_stream_read.restype = ctypes.c_int
lib.qa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
lib.qa_probe_mfma.restype = ctypes.c_int
lib.qa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
lib.qa_probe_valu.restype = ctypes.c_int
lib.qa_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
EXPORTED = ("qa_probe_stream_read", "qa_probe_mfma", "qa_probe_valu")

# ops per round of one wave, by kind (see qa_probe.h)
MFMA_KINDS = {
    0: ("i8_32x32x32", 4 * 65536),
    1: ("f16_32x32x16", 4 * 32768),
    2: ("i8_16x16x64", 8 * 32768),
    3: ("f16_16x16x32", 8 * 16384),
    4: ("i8_16x16x64_acc16", 16 * 32768),
    5: ("f16_16x16x32_acc16", 16 * 16384),
    6: ("i8_16x16x64_acc4", 4 * 32768),
    7: ("f16_16x16x32_acc4", 4 * 16384),
    8: ("fp8_32x32x64", 4 * 131072),
}

VALU_KINDS = {0: "exp_f32", 1: "fma_f32"}


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed with status {rc}")


def stream_read(src, wgs: int, sink, stream) -> None:
    """Launch one streaming read over the whole tensor `src` (bytes a multiple
    of 16) on `stream` (a raw hipStream_t value); `sink` holds >= wgs int32."""
    nbytes = src.numel() * src.element_size()
    _check(lib.qa_probe_stream_read(src.data_ptr(), nbytes, wgs, sink.data_ptr(), stream), "qa_probe_stream_read")


def mfma(kind: int, iters: int, wgs: int, sink, stream) -> float:
    """Launch one matrix-throughput loop; returns its total ops. `sink` holds
    >= wgs * 256 float32."""
    _check(lib.qa_probe_mfma(kind, iters, wgs, sink.data_ptr(), stream), "qa_probe_mfma")
    return float(MFMA_KINDS[kind][1]) * iters * 4 * wgs


def valu(kind: int, iters: int, wgs: int, sink, stream) -> float:
    """Launch one vector-ALU throughput loop; returns its total lane
    operations. `sink` holds >= wgs * 256 float32."""
    _check(lib.qa_probe_valu(kind, iters, wgs, sink.data_ptr(), stream), "qa_probe_valu")
    return 8.0 * iters * 256 * wgs
