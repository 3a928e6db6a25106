"""Python binding of libdg, the HIP (gfx950) hot path of one block-diffusion
denoising step: mixed-mode attention, the DiffusionSampler step and the
self-conditioning embedding average.

The binding only marshals arguments: torch tensors give device pointers and the
current HIP stream, and every step of the computation runs in libdg's kernels.
There is no fallback: if libdg.so is missing or cannot be loaded, every call
raises. Build it with `python -m block_denoising_step_amd.build`.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg.so")

DG_OK, DG_ERR_INVALID_ARG, DG_ERR_UNSUPPORTED, DG_ERR_WORKSPACE, DG_ERR_HIP = 0, 1, 2, 3, 4
ABI_VERSION = 3  # DG_ABI_VERSION of the include/dg.h these structs mirror
DG_F32, DG_BF16 = 0, 1
DG_CAUSAL, DG_BIDIR = 0, 1
DG_CONF_NEG_ENTROPY, DG_CONF_MAX_PROB = 0, 1
DG_CONV_AND, DG_CONV_OR = 0, 1
DG_ENTROPY_IN, DG_INIT_CANVAS, DG_SKIP_SELECT, DG_SELECT_ONLY = 1, 2, 4, 8
DG_MAX_SEQS = DG_MAX_REQS = 64
DG_MAX_CANVAS = 1024
DG_PROB_BLOCK = 8192
DG_NOALLOC_SCRATCH_BYTES = 4 << 20

_c_int32, _c_int64, _c_uint32, _c_uint64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_uint64
_vp, _fp = ctypes.c_void_p, ctypes.c_void_p


class DgSeq(ctypes.Structure):
    _fields_ = [("q_start", _c_int32), ("num_q", _c_int32), ("kv_start", _c_int32),
                ("prefix_len", _c_int32), ("mode", _c_int32)]


class DgAttnArgs(ctypes.Structure):
    _fields_ = [("num_seqs", _c_int32), ("seqs", ctypes.POINTER(DgSeq)), ("window", _c_int32),
                ("num_q_heads", _c_int32), ("num_kv_heads", _c_int32), ("head_dim", _c_int32),
                ("scale", ctypes.c_float), ("dtype", _c_int32), ("total_q", _c_int64), ("total_kv", _c_int64),
                ("q", _vp), ("k", _vp), ("v", _vp), ("out", _vp), ("lse", _vp), ("kv_chunk", _c_int32),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("block_size", _c_int32), ("block_table", _vp), ("block_table_len", _c_int64),
                ("kv_fp8", _c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class DgKvSeq(ctypes.Structure):
    _fields_ = [("src_start", _c_int32), ("num", _c_int32), ("table_start", _c_int32), ("pos", _c_int32)]


class DgKvWriteArgs(ctypes.Structure):
    _fields_ = [("num_seqs", _c_int32), ("seqs", ctypes.POINTER(DgKvSeq)), ("num_kv_heads", _c_int32),
                ("head_dim", _c_int32), ("dtype", _c_int32), ("block_size", _c_int32), ("block_table", _vp),
                ("block_table_len", _c_int64), ("total_new", _c_int64), ("pool_rows", _c_int64),
                ("k_new", _vp), ("v_new", _vp), ("k_pool", _vp), ("v_pool", _vp),
                ("pool_fp8", _c_int32), ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class DgSreq(ctypes.Structure):
    _fields_ = [("row_start", _c_int32), ("num_rows", _c_int32), ("seed", _c_uint64), ("step", _c_int32),
                ("reserved", _c_int32)]


class DgSamplerArgs(ctypes.Structure):
    _fields_ = [("num_reqs", _c_int32), ("reqs", ctypes.POINTER(DgSreq)), ("num_rows", _c_int32),
                ("vocab", _c_int32), ("dtype", _c_int32), ("logits", _vp), ("ld", _c_int64),
                ("budget", ctypes.c_float), ("min_accept", _c_int32), ("conf_mode", _c_int32),
                ("renoise", _c_int32), ("stable_k", _c_int32), ("tau", ctypes.c_float), ("step_limit", _c_int32),
                ("combine", _c_int32), ("flags", _c_uint32),
                ("entropy", _vp), ("conf", _vp), ("row_max", _vp), ("row_sum", _vp), ("argmax", _vp),
                ("cand", _vp), ("accept", _vp), ("canvas", _vp), ("prev_argmax", _vp),
                ("stable_count", _vp), ("num_accepted", _vp), ("converged", _vp), ("mean_entropy", _vp),
                ("probs", _vp), ("ldq", _c_int64), ("probs_scale", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("step_counter", _vp)]


class DgSelfcondArgs(ctypes.Structure):
    _fields_ = [("M", _c_int32), ("V", _c_int32), ("d", _c_int32), ("dtype", _c_int32),
                ("p", _vp), ("ldp", _c_int64), ("row_max", _vp), ("row_sum", _vp), ("p_scale", _vp),
                ("embed", _vp), ("lde", _c_int64), ("out", _vp), ("ldo", _c_int64),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t)]


class DgInjectArgs(ctypes.Structure):
    _fields_ = [("M", _c_int32), ("d", _c_int32), ("hidden", _c_int32), ("vocab", _c_int32), ("dtype", _c_int32),
                ("tokens", _vp), ("embed", _vp), ("s", _vp), ("w_gate_up", _vp), ("w_down", _vp), ("out", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t)]


EXPORTS = ["dg_attn_mixed", "dg_attn_workspace_size", "dg_sampler_step", "dg_sampler_workspace_size",
           "dg_sampler_step_noalloc",
           "dg_selfcond_embed", "dg_selfcond_workspace_size", "dg_kv_write", "dg_selfcond_inject",
           "dg_selfcond_inject_workspace_size", "dg_status_string", "dg_last_error",
           "dg_abi_version", "dg_test_force_register_staged", "dg_test_wide_min_sub"]

_lib = None


class DgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_string(status)}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load libdg.so (once). Raises if it is not built: there is no other path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_denoising_step_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.dg_attn_mixed.argtypes = [ctypes.POINTER(DgAttnArgs), _vp]
    lib.dg_attn_mixed.restype = ctypes.c_int
    lib.dg_attn_workspace_size.argtypes = [ctypes.POINTER(DgAttnArgs)]
    lib.dg_attn_workspace_size.restype = ctypes.c_size_t
    lib.dg_sampler_step.argtypes = [ctypes.POINTER(DgSamplerArgs), _vp]
    lib.dg_sampler_step.restype = ctypes.c_int
    lib.dg_sampler_step_noalloc.argtypes = [ctypes.POINTER(DgSamplerArgs), _vp]
    lib.dg_sampler_step_noalloc.restype = ctypes.c_int
    lib.dg_sampler_workspace_size.argtypes = [ctypes.POINTER(DgSamplerArgs)]
    lib.dg_sampler_workspace_size.restype = ctypes.c_size_t
    lib.dg_selfcond_embed.argtypes = [ctypes.POINTER(DgSelfcondArgs), _vp]
    lib.dg_selfcond_embed.restype = ctypes.c_int
    lib.dg_selfcond_workspace_size.argtypes = [ctypes.POINTER(DgSelfcondArgs)]
    lib.dg_selfcond_workspace_size.restype = ctypes.c_size_t
    lib.dg_selfcond_inject.argtypes = [ctypes.POINTER(DgInjectArgs), _vp]
    lib.dg_selfcond_inject.restype = ctypes.c_int
    lib.dg_selfcond_inject_workspace_size.argtypes = [ctypes.POINTER(DgInjectArgs)]
    lib.dg_selfcond_inject_workspace_size.restype = ctypes.c_size_t
    lib.dg_kv_write.argtypes = [ctypes.POINTER(DgKvWriteArgs), _vp]
    lib.dg_kv_write.restype = ctypes.c_int
    lib.dg_status_string.argtypes = [ctypes.c_int]
    lib.dg_status_string.restype = ctypes.c_char_p
    lib.dg_last_error.argtypes = []
    lib.dg_last_error.restype = ctypes.c_char_p
    lib.dg_abi_version.argtypes = []
    lib.dg_abi_version.restype = ctypes.c_int
    lib.dg_test_force_register_staged.argtypes = [ctypes.c_int]
    lib.dg_test_force_register_staged.restype = ctypes.c_int
    lib.dg_test_wide_min_sub.argtypes = [ctypes.c_int]
    lib.dg_test_wide_min_sub.restype = ctypes.c_int
    if lib.dg_abi_version() != ABI_VERSION:
        # the structs above would not match the library's: refuse rather than pass garbage
        raise RuntimeError(f"{LIB_PATH} has ABI version {lib.dg_abi_version()}, this binding needs {ABI_VERSION}; "
                           "rebuild it")
    _lib = lib
    return lib


class wide_min_sub:
    """Test hook as a context manager: inside it, a head_dim-256 request (bf16 or FP8 K/V)
    runs on a 64-rows-per-wave attention kernel from `n` sub-tiles per work group
    (dg_test_wide_min_sub)."""

    def __init__(self, n: int):
        self._n = n

    def __enter__(self):
        self._prev = load().dg_test_wide_min_sub(self._n)
        return self

    def __exit__(self, *exc):
        load().dg_test_wide_min_sub(self._prev)
        return False


class force_register_staged:
    """Test hook as a context manager: inside it, dg_attn_mixed plans every request on the
    register-staged attention kernel (dg_test_force_register_staged)."""

    def __enter__(self):
        self._prev = load().dg_test_force_register_staged(1)
        return self

    def __exit__(self, *exc):
        load().dg_test_force_register_staged(self._prev)
        return False


def status_string(status: int) -> str:
    return load().dg_status_string(status).decode()


def last_error() -> str:
    return load().dg_last_error().decode()


def _check(status: int) -> None:
    if status != DG_OK:
        raise DgError(status, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DG_BF16
    if t.dtype == torch.float32:
        return DG_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _is_fp8(t: torch.Tensor) -> bool:
    """E4M3 codes: torch.float8_e4m3fn, or raw codes in uint8."""
    return t.dtype in (torch.float8_e4m3fn, torch.uint8)


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _workspace(nbytes: int, like: torch.Tensor, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == ctypes.c_size_t(-1).value:
        return workspace  # invalid args: the call itself reports the error
    if nbytes == 0:
        return workspace
    if workspace is not None and workspace.numel() * workspace.element_size() >= nbytes:
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


# ---- dg_attn_mixed ---------------------------------------------------------------

def make_attn_args(q, k, v, out, seqs: Sequence, window: int, num_q_heads: int, num_kv_heads: int,
                   lse=None, scale: float = 0.0, kv_chunk: int = 0, workspace=None, block_table=None,
                   block_size: int = 0, k_scale: float = 1.0, v_scale: float = 1.0):
    """block_size > 0: k/v are paged pools and block_table an int32 device tensor; each
    request's kv_start is then the index of its first table entry. k/v of dtype
    float8_e4m3fn (or uint8) hold E4M3 codes whose values are code * k_scale / v_scale."""
    seq_arr = (DgSeq * max(1, len(seqs)))()
    for i, s in enumerate(seqs):
        f = (s.q_start, s.num_q, s.kv_start, s.prefix_len, s.mode) if hasattr(s, "q_start") else tuple(s)
        seq_arr[i] = DgSeq(*f)
    a = DgAttnArgs()
    a.num_seqs = len(seqs)
    a.seqs = ctypes.cast(seq_arr, ctypes.POINTER(DgSeq))
    a.window = window
    a.num_q_heads, a.num_kv_heads = num_q_heads, num_kv_heads
    a.head_dim = q.shape[-1]
    a.scale = scale
    a.dtype = _dtype(q)
    a.total_q, a.total_kv = q.shape[0], k.shape[0]
    a.q, a.k, a.v, a.out, a.lse = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse)
    a.kv_chunk = kv_chunk
    a.kv_fp8 = int(_is_fp8(k))
    if a.kv_fp8 != int(_is_fp8(v)):
        raise TypeError("k and v must both hold E4M3 codes, or neither")
    a.k_scale, a.v_scale = (k_scale, v_scale) if a.kv_fp8 else (0.0, 0.0)
    a.block_size = block_size
    if block_size:
        if block_table is None or block_table.dtype != torch.int32:
            raise TypeError("paged attention needs an int32 block_table tensor")
        a.block_table, a.block_table_len = _ptr(block_table), block_table.numel()
    a._keep = seq_arr  # keep the host array alive with the struct
    return a


def attn_workspace_size(args: DgAttnArgs) -> int:
    return load().dg_attn_workspace_size(ctypes.byref(args))


def dg_attn_mixed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, seqs: Sequence,
                  window: int, num_q_heads: int, num_kv_heads: int, lse: Optional[torch.Tensor] = None,
                  scale: float = 0.0, kv_chunk: int = 0, workspace: Optional[torch.Tensor] = None,
                  stream=None, block_table: Optional[torch.Tensor] = None, block_size: int = 0,
                  k_scale: float = 1.0, v_scale: float = 1.0) -> Optional[torch.Tensor]:
    """Mixed-mode attention (see include/dg.h). q [T, Hq, D], k/v [S, Hkv, D], out like q,
    lse [T, Hq] fp32 or None; with block_size > 0, k/v are paged pools read through
    block_table; k/v in float8_e4m3fn (or uint8) are E4M3 codes with scales k_scale and
    v_scale. Returns the workspace tensor used (reusable)."""
    a = make_attn_args(q, k, v, out, seqs, window, num_q_heads, num_kv_heads, lse, scale, kv_chunk,
                       block_table=block_table, block_size=block_size, k_scale=k_scale, v_scale=v_scale)
    ws = _workspace(attn_workspace_size(a), q, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().dg_attn_mixed(ctypes.byref(a), _stream(stream)))
    return ws


# ---- dg_kv_write -----------------------------------------------------------------

def make_kv_write_args(k_new, v_new, k_pool, v_pool, seqs: Sequence, block_table, block_size: int,
                       k_scale: float = 1.0, v_scale: float = 1.0):
    """seqs: (src_start, num, table_start, pos) per request. Pools of dtype float8_e4m3fn
    (or uint8) take E4M3 codes of the new values at scales k_scale and v_scale."""
    if block_table.dtype != torch.int32:
        raise TypeError("block_table must be an int32 tensor")
    arr = (DgKvSeq * max(1, len(seqs)))()
    for i, s in enumerate(seqs):
        arr[i] = DgKvSeq(*tuple(s))
    a = DgKvWriteArgs()
    a.num_seqs = len(seqs)
    a.seqs = ctypes.cast(arr, ctypes.POINTER(DgKvSeq))
    a.num_kv_heads, a.head_dim = k_new.shape[1], k_new.shape[2]
    a.dtype = _dtype(k_new)
    a.block_size = block_size
    a.block_table, a.block_table_len = _ptr(block_table), block_table.numel()
    a.total_new, a.pool_rows = k_new.shape[0], k_pool.shape[0]
    a.k_new, a.v_new, a.k_pool, a.v_pool = _ptr(k_new), _ptr(v_new), _ptr(k_pool), _ptr(v_pool)
    a.pool_fp8 = int(_is_fp8(k_pool))
    if a.pool_fp8 != int(_is_fp8(v_pool)):
        raise TypeError("k_pool and v_pool must both hold E4M3 codes, or neither")
    a.k_scale, a.v_scale = (k_scale, v_scale) if a.pool_fp8 else (0.0, 0.0)
    a._keep = arr
    return a


def dg_kv_write(k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                seqs: Sequence, block_table: torch.Tensor, block_size: int, stream=None, k_scale: float = 1.0,
                v_scale: float = 1.0) -> None:
    """Scatter new K/V rows [T, Hkv, D] into paged pools [rows, Hkv, D] (see include/dg.h);
    pools of E4M3 codes take the quantized values."""
    a = make_kv_write_args(k_new, v_new, k_pool, v_pool, seqs, block_table, block_size, k_scale, v_scale)
    _check(load().dg_kv_write(ctypes.byref(a), _stream(stream)))


def prepare_kv_write(k_new, v_new, k_pool, v_pool, seqs, block_table, block_size, k_scale=1.0, v_scale=1.0):
    a = make_kv_write_args(k_new, v_new, k_pool, v_pool, seqs, block_table, block_size, k_scale, v_scale)
    return Prepared(load().dg_kv_write, a, ())


# ---- dg_selfcond_inject ------------------------------------------------------------

def make_inject_args(tokens, embed, s, w_gate_up, w_down, out):
    """tokens [M] int32; embed [V, d]; s [M, d]; w_gate_up [d, 2h]; w_down [h, d]; out [M, d]."""
    if tokens.dtype != torch.int32:
        raise TypeError("tokens must be int32")
    a = DgInjectArgs()
    a.M, a.d = s.shape[0], s.shape[1]
    a.hidden = w_down.shape[0]
    a.vocab = embed.shape[0]
    a.dtype = _dtype(s)
    a.tokens, a.embed, a.s, a.w_gate_up, a.w_down, a.out = (_ptr(tokens), _ptr(embed), _ptr(s), _ptr(w_gate_up),
                                                            _ptr(w_down), _ptr(out))
    return a


def inject_workspace_size(args: DgInjectArgs) -> int:
    return load().dg_selfcond_inject_workspace_size(ctypes.byref(args))


def dg_selfcond_inject(tokens, embed, s, w_gate_up, w_down, out, workspace=None, stream=None):
    """out = embed[tokens] + GeGLU(s) (see include/dg.h). Returns the workspace used."""
    a = make_inject_args(tokens, embed, s, w_gate_up, w_down, out)
    ws = _workspace(inject_workspace_size(a), s, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().dg_selfcond_inject(ctypes.byref(a), _stream(stream)))
    return ws


def prepare_inject(tokens, embed, s, w_gate_up, w_down, out):
    a = make_inject_args(tokens, embed, s, w_gate_up, w_down, out)
    ws = _workspace(inject_workspace_size(a), s, None)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel()
    return Prepared(load().dg_selfcond_inject, a, (ws,))


# ---- dg_sampler_step -------------------------------------------------------------

class SamplerBuffers:
    """Device buffers of one sampler call: per-row outputs and per-request state."""

    def __init__(self, num_rows: int, num_reqs: int, device, vocab: int = 0, probs_dtype=None):
        f = dict(dtype=torch.float32, device=device)
        i = dict(dtype=torch.int32, device=device)
        self.entropy = torch.zeros(num_rows, **f)
        self.conf = torch.zeros(num_rows, **f)
        self.row_max = torch.zeros(num_rows, **f)
        self.row_sum = torch.zeros(num_rows, **f)
        self.argmax = torch.zeros(num_rows, **i)
        self.cand = torch.zeros(num_rows, **i)
        self.accept = torch.zeros(num_rows, dtype=torch.uint8, device=device)
        self.canvas = torch.zeros(num_rows, **i)
        self.prev_argmax = torch.full((num_rows,), -1, **i)
        self.stable_count = torch.zeros(num_reqs, **i)
        self.num_accepted = torch.zeros(num_reqs, **i)
        self.converged = torch.zeros(num_reqs, **i)
        self.mean_entropy = torch.zeros(num_reqs, **f)
        self.workspace: Optional[torch.Tensor] = None
        # block-scaled probabilities (optional): w [num_rows, vocab] and scales
        self.probs = self.probs_scale = None
        if vocab and probs_dtype is not None:
            ld = (vocab + 7) // 8 * 8
            self.probs = torch.empty(num_rows, ld, dtype=probs_dtype, device=device)[:, :vocab]
            self.probs_scale = torch.empty(num_rows, (vocab + DG_PROB_BLOCK - 1) // DG_PROB_BLOCK, **f)


def make_sampler_args(logits: Optional[torch.Tensor], reqs: Sequence[Tuple[int, int, int, int]], vocab: int,
                      bufs: SamplerBuffers, budget: float, min_accept: int = 1,
                      conf_mode: int = DG_CONF_NEG_ENTROPY, renoise: int = 1, stable_k: int = 3, tau: float = 0.05,
                      step_limit: int = 48, combine: int = DG_CONV_AND, flags: int = 0, num_rows: Optional[int] = None,
                      probs: Optional[torch.Tensor] = None, probs_scale: Optional[torch.Tensor] = None,
                      step_counter: Optional[torch.Tensor] = None):
    """step_counter: an int32 device tensor [num_reqs] that holds each request's step
    (read and advanced by the kernels; see include/dg.h), or None."""
    if step_counter is not None and (step_counter.dtype != torch.int32 or step_counter.numel() < len(reqs)):
        raise TypeError("step_counter must be an int32 tensor with one entry per request")
    req_arr = (DgSreq * max(1, len(reqs)))()
    for i, (row_start, n, seed, step) in enumerate(reqs):
        req_arr[i] = DgSreq(row_start, n, seed, step, 0)
    a = DgSamplerArgs()
    a.num_reqs = len(reqs)
    a.reqs = ctypes.cast(req_arr, ctypes.POINTER(DgSreq))
    a.num_rows = num_rows if num_rows is not None else (logits.shape[0] if logits is not None else bufs.canvas.shape[0])
    a.vocab = vocab
    a.dtype = _dtype(logits) if logits is not None else DG_BF16
    a.logits = _ptr(logits)
    a.ld = logits.stride(0) if logits is not None else vocab
    a.budget, a.min_accept, a.conf_mode, a.renoise = budget, min_accept, conf_mode, renoise
    a.stable_k, a.tau, a.step_limit, a.combine, a.flags = stable_k, tau, step_limit, combine, flags
    for name in ("entropy", "conf", "row_max", "row_sum", "argmax", "cand", "accept", "canvas", "prev_argmax",
                 "stable_count", "num_accepted", "converged", "mean_entropy"):
        setattr(a, name, _ptr(getattr(bufs, name)))
    a.probs, a.probs_scale = _ptr(probs), _ptr(probs_scale)
    a.ldq = probs.stride(0) if probs is not None else 0
    a.step_counter = _ptr(step_counter)
    a._keep = req_arr
    return a


def sampler_workspace_size(args: DgSamplerArgs) -> int:
    return load().dg_sampler_workspace_size(ctypes.byref(args))


def dg_sampler_step(logits: Optional[torch.Tensor], reqs: Sequence[Tuple[int, int, int, int]], vocab: int,
                    bufs: SamplerBuffers, budget: float, stream=None, **kw) -> None:
    """One DiffusionSampler denoise step (see include/dg.h). reqs: (row_start, num_rows,
    seed, step) per request. Outputs and state live in `bufs` (block-scaled
    probabilities too, when bufs holds them)."""
    kw.setdefault("probs", bufs.probs)
    kw.setdefault("probs_scale", bufs.probs_scale)
    a = make_sampler_args(logits, reqs, vocab, bufs, budget, **kw)
    like = logits if logits is not None else bufs.canvas
    bufs.workspace = _workspace(sampler_workspace_size(a), like, bufs.workspace)
    a.workspace = _ptr(bufs.workspace)
    a.workspace_bytes = 0 if bufs.workspace is None else bufs.workspace.numel()
    _check(load().dg_sampler_step(ctypes.byref(a), _stream(stream)))


def dg_sampler_step_noalloc(logits: Optional[torch.Tensor], reqs: Sequence[Tuple[int, int, int, int]], vocab: int,
                            bufs: SamplerBuffers, budget: float, stream=None, **kw) -> None:
    """dg_sampler_step on the library's static scratch (no workspace, nothing allocated;
    see include/dg.h): same arguments and results."""
    kw.setdefault("probs", bufs.probs)
    kw.setdefault("probs_scale", bufs.probs_scale)
    a = make_sampler_args(logits, reqs, vocab, bufs, budget, **kw)
    _check(load().dg_sampler_step_noalloc(ctypes.byref(a), _stream(stream)))


# ---- dg_selfcond_embed -----------------------------------------------------------

def make_selfcond_args(p: torch.Tensor, embed: torch.Tensor, out: torch.Tensor, row_max=None, row_sum=None,
                       num_cols: Optional[int] = None, p_scale=None):
    a = DgSelfcondArgs()
    a.M = p.shape[0]
    a.V = num_cols if num_cols is not None else p.shape[1]
    a.d = embed.shape[1]
    a.dtype = _dtype(p)
    a.p, a.ldp = _ptr(p), p.stride(0)
    a.row_max, a.row_sum = _ptr(row_max), _ptr(row_sum)
    a.p_scale = _ptr(p_scale)
    a.embed, a.lde = _ptr(embed), embed.stride(0)
    a.out, a.ldo = _ptr(out), out.stride(0)
    return a


def selfcond_workspace_size(args: DgSelfcondArgs) -> int:
    return load().dg_selfcond_workspace_size(ctypes.byref(args))


def dg_selfcond_embed(p: torch.Tensor, embed: torch.Tensor, out: torch.Tensor,
                      row_max: Optional[torch.Tensor] = None, row_sum: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None,
                      p_scale: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """out = P . E with P given, rebuilt from logits and row stats, or block-scaled
    (p holds w, p_scale the per-block scales; see include/dg.h). Returns the
    workspace tensor used (reusable)."""
    a = make_selfcond_args(p, embed, out, row_max, row_sum, p_scale=p_scale)
    ws = _workspace(selfcond_workspace_size(a), p, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(load().dg_selfcond_embed(ctypes.byref(a), _stream(stream)))
    return ws


# ---- prepared calls (argument structs built once, reused every step) ----------------

class Prepared:
    """A libdg call with its argument struct and workspace fixed; calling it only
    passes the struct and the stream. `args` stays editable (e.g. a request's step)."""

    def __init__(self, fn, args, keep=()):
        self._fn = fn
        self.args = args
        self._keep = keep

    def __call__(self, stream=None) -> None:
        _check(self._fn(ctypes.byref(self.args), _stream(stream)))


def prepare_attn(q, k, v, out, seqs, window, num_q_heads, num_kv_heads, lse=None, scale=0.0, kv_chunk=0,
                 block_table=None, block_size=0, k_scale=1.0, v_scale=1.0):
    a = make_attn_args(q, k, v, out, seqs, window, num_q_heads, num_kv_heads, lse, scale, kv_chunk,
                       block_table=block_table, block_size=block_size, k_scale=k_scale, v_scale=v_scale)
    ws = _workspace(attn_workspace_size(a), q, None)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel()
    return Prepared(load().dg_attn_mixed, a, (ws,))


def prepare_sampler(logits, reqs, vocab, bufs, budget, **kw):
    if logits is not None:
        kw.setdefault("probs", bufs.probs)
        kw.setdefault("probs_scale", bufs.probs_scale)
    a = make_sampler_args(logits, reqs, vocab, bufs, budget, **kw)
    like = logits if logits is not None else bufs.canvas
    bufs.workspace = _workspace(sampler_workspace_size(a), like, bufs.workspace)
    a.workspace = _ptr(bufs.workspace)
    a.workspace_bytes = 0 if bufs.workspace is None else bufs.workspace.numel()
    return Prepared(load().dg_sampler_step, a, (bufs,))


def prepare_selfcond(p, embed, out, row_max=None, row_sum=None, p_scale=None, workspace=None):
    """workspace: a uint8 device tensor to reuse when it is large enough (calls that never
    run concurrently can share one)."""
    a = make_selfcond_args(p, embed, out, row_max, row_sum, p_scale=p_scale)
    ws = _workspace(selfcond_workspace_size(a), p, workspace)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel()
    return Prepared(load().dg_selfcond_embed, a, (ws,))
