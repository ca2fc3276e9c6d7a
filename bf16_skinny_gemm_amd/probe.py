"""ctypes binding of the read-stream probe, libskinny_stream_probe.so
(include/skinny_stream_probe.h): one kernel that reads a device buffer once, to
measure the HBM read rate a plain streaming kernel reaches on this device.
Measurement only; the GEMM does not use it."""
from __future__ import annotations

import ctypes
import os
import threading

import torch  # noqa: F401  (binds the library to torch's HIP runtime, as the main binding does)

from .build import PROBE_LIB_PATH

_lock = threading.Lock()
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(PROBE_LIB_PATH):
                raise ImportError(f"{PROBE_LIB_PATH} is missing: build it first "
                                  "(python -m bf16_skinny_gemm_amd.build)")
            L = ctypes.CDLL(PROBE_LIB_PATH)
            L.skinny_probe_sink_words.argtypes = [ctypes.c_int]
            L.skinny_probe_sink_words.restype = ctypes.c_size_t
            L.skinny_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
            L.skinny_probe_read.restype = ctypes.c_int
            L.skinny_probe_tiles_sink_words.argtypes = [ctypes.c_size_t, ctypes.c_int, ctypes.c_int]
            L.skinny_probe_tiles_sink_words.restype = ctypes.c_size_t
            L.skinny_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                                  ctypes.c_void_p]
            L.skinny_probe_read_tiles.restype = ctypes.c_int
            L.skinny_probe_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
            L.skinny_probe_empty.restype = ctypes.c_int
            _lib = L
        return _lib


def sink_words(grid_blocks: int) -> int:
    return int(lib().skinny_probe_sink_words(grid_blocks))


def read(buf: torch.Tensor, sink: torch.Tensor, nontemporal: bool = True,
         grid_blocks: int = 2048) -> None:
    """Enqueue one read of all of `buf` on the current stream; `sink` is an int32
    device tensor of at least sink_words(grid_blocks) elements."""
    if not (buf.is_cuda and sink.is_cuda and buf.device == sink.device):
        raise ValueError("buf and sink must be tensors on the same GPU")
    if not buf.is_contiguous() or sink.dtype != torch.int32 or not sink.is_contiguous():
        raise ValueError("buf must be contiguous and sink a contiguous int32 tensor")
    if sink.numel() < sink_words(grid_blocks):
        raise ValueError(f"sink needs {sink_words(grid_blocks)} words")
    stream = torch.cuda.current_stream(buf.device).cuda_stream
    st = lib().skinny_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(),
                                 1 if nontemporal else 0, grid_blocks, sink.data_ptr(), stream)
    if st != 0:
        raise RuntimeError(f"skinny_probe_read failed with status {st}")


def tiles_sink_words(nbytes: int, loads: int, threads: int) -> int:
    return int(lib().skinny_probe_tiles_sink_words(nbytes, loads, threads))


def read_tiles(buf: torch.Tensor, sink: torch.Tensor, loads: int = 4, threads: int = 256,
               nontemporal: bool = True) -> None:
    """Enqueue one read of all of `buf`, one block per tile of threads/64 * loads KiB
    (the M = 1 GEMV's load schedule without arithmetic), on the current stream;
    `sink` is an int32 device tensor of at least tiles_sink_words() elements."""
    if not (buf.is_cuda and sink.is_cuda and buf.device == sink.device):
        raise ValueError("buf and sink must be tensors on the same GPU")
    if not buf.is_contiguous() or sink.dtype != torch.int32 or not sink.is_contiguous():
        raise ValueError("buf must be contiguous and sink a contiguous int32 tensor")
    nbytes = buf.numel() * buf.element_size()
    need = tiles_sink_words(nbytes, loads, threads)
    if need == 0 or sink.numel() < need:
        raise ValueError(f"sink needs {need} words (loads {loads}, threads {threads})")
    stream = torch.cuda.current_stream(buf.device).cuda_stream
    st = lib().skinny_probe_read_tiles(buf.data_ptr(), nbytes, 1 if nontemporal else 0, loads,
                                       threads, sink.data_ptr(), stream)
    if st != 0:
        raise RuntimeError(f"skinny_probe_read_tiles failed with status {st}")


def empty(grid_blocks: int, threads: int = 256, device=None) -> None:
    """Enqueue one launch of a kernel that does nothing, on the current stream."""
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream(dev).cuda_stream
    st = lib().skinny_probe_empty(grid_blocks, threads, stream)
    if st != 0:
        raise RuntimeError(f"skinny_probe_empty failed with status {st}")
