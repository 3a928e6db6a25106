"""Binding of libdg_probe.so (include/dg_probe.h): measurement kernels for the achievable
HBM and bf16 matrix ceilings, not part of the denoising step. Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg_probe.so")
EXPORTS = ["dg_probe_read", "dg_probe_copy", "dg_probe_mfma_bf16"]
_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_denoising_step_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.dg_probe_read.argtypes = [vp, sz, vp, ctypes.c_int, vp]
    lib.dg_probe_copy.argtypes = [vp, vp, sz, ctypes.c_int, vp]
    lib.dg_probe_mfma_bf16.argtypes = [vp, vp, ctypes.c_int, ctypes.c_int, vp]
    for n in EXPORTS:
        getattr(lib, n).restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ok(rc: int, name: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{name} failed ({rc})")


def read(src: torch.Tensor, sink: torch.Tensor, blocks: int, stream=None) -> None:
    _ok(load().dg_probe_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), blocks,
                             _stream(stream)), "dg_probe_read")


def copy(dst: torch.Tensor, src: torch.Tensor, blocks: int, stream=None) -> None:
    _ok(load().dg_probe_copy(dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(), blocks,
                             _stream(stream)), "dg_probe_copy")


def mfma_bf16(sink: torch.Tensor, blocks: int, iters: int, ops: torch.Tensor = None, stream=None) -> None:
    """ops: [blocks * 256 * 8 * 8] bf16 operands (4 A and 4 B vectors per lane), or None
    for one fixed operand pair."""
    _ok(load().dg_probe_mfma_bf16(None if ops is None else ops.data_ptr(), sink.data_ptr(), blocks, iters,
                                  _stream(stream)), "dg_probe_mfma_bf16")
