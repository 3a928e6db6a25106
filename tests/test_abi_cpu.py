"""Host-only checks of the C ABI (no GPU needed, no kernel launched): libdg.so loads,
exports every function include/dg.h declares, sizes workspaces, and maps every
invalid argument to its dg_status with a message, before anything is launched.
Device pointers here are fake aligned addresses: every call below fails
validation, which happens before any HIP call."""
import ctypes
import os
import re

import pytest

import block_denoising_step_amd as dg
from workloads import pack_seqs, BIDIR, CAUSAL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced


def _declared():
    with open(os.path.join(ROOT, "include", "dg.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dg_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = dg.load()
    names = _declared()
    assert set(names) == set(dg.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dg_abi_version() == 3
    for s in range(5):
        assert lib.dg_status_string(s).decode().startswith("DG_")


class _T:
    """Stand-in for a tensor: only what the binding reads."""

    def __init__(self, shape, ptr=FAKE, dtype="bf16"):
        self.shape = shape
        self._ptr = ptr
        import torch
        self.dtype = {"bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32,
                      "fp8": torch.float8_e4m3fn}[dtype]

    def data_ptr(self):
        return self._ptr

    def numel(self):
        n = 1
        for x in self.shape:
            n *= x
        return n

    def stride(self, i):
        s = 1
        for x in self.shape[i + 1:]:
            s *= x
        return s


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without libdg.so every entry point raises."""
    monkeypatch.setattr(dg, "_lib", None)
    monkeypatch.setattr(dg, "LIB_PATH", str(tmp_path / "libdg.so"))
    with pytest.raises(RuntimeError):
        dg.load()
    with pytest.raises(RuntimeError):
        dg.attn_workspace_size(dg.DgAttnArgs())


def test_binding_matches_the_library_abi():
    assert dg.ABI_VERSION == dg.load().dg_abi_version()


def _attn(**over):
    seqs = over.pop("seqs", pack_seqs([(64, 32, BIDIR)]))
    q = over.pop("q", _T((32, 4, 64)))
    k = over.pop("k", _T((96, 2, 64)))
    a = dg.make_attn_args(q, k, _T(k.shape), _T(q.shape), seqs, over.pop("window", -1),
                          over.pop("hq", 4), over.pop("hkv", 2))
    for key, val in over.items():
        setattr(a, key[6:] if key.startswith("field_") else key, val)
    return a


def _status(a):
    lib = dg.load()
    return lib.dg_attn_mixed(ctypes.byref(a), None)


@pytest.mark.parametrize("change,status", [
    (dict(num_seqs=0), dg.DG_ERR_INVALID_ARG),
    (dict(num_seqs=65), dg.DG_ERR_INVALID_ARG),
    (dict(hq=6, hkv=4), dg.DG_ERR_INVALID_ARG),
    (dict(hq=12, hkv=4), dg.DG_ERR_UNSUPPORTED),  # G = 3
    (dict(head_dim=96), dg.DG_ERR_UNSUPPORTED),
    (dict(window=-2), dg.DG_ERR_INVALID_ARG),
    (dict(scale=float("nan")), dg.DG_ERR_INVALID_ARG),
    (dict(scale=-1.0), dg.DG_ERR_INVALID_ARG),
    (dict(dtype=7), dg.DG_ERR_INVALID_ARG),
    (dict(field_q=None), dg.DG_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), dg.DG_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), dg.DG_ERR_INVALID_ARG),
    (dict(kv_chunk=100), dg.DG_ERR_INVALID_ARG),
    (dict(total_q=31), dg.DG_ERR_INVALID_ARG),
    (dict(total_kv=95), dg.DG_ERR_INVALID_ARG),
    (dict(seqs=pack_seqs([(64, 32, 5)])), dg.DG_ERR_INVALID_ARG),
    (dict(seqs=[(0, 16, 0, 8, BIDIR), (8, 16, 24, 8, BIDIR)], q=_T((24, 4, 64)), k=_T((96, 2, 64))),
     dg.DG_ERR_INVALID_ARG),  # overlapping query ranges
])
def test_attn_validation(change, status):
    a = _attn(**change)
    if "head_dim" in change:
        a.head_dim = change["head_dim"]
    assert _status(a) == status
    assert dg.last_error()


def test_attn_fp32_head_dim_256_unsupported_and_workspace():
    a = _attn(q=_T((32, 4, 256), dtype="f32"), k=_T((96, 2, 256), dtype="f32"))
    assert _status(a) == dg.DG_ERR_UNSUPPORTED
    # a long prefix splits keys into chunks, which need a workspace; too small is an error
    seqs = pack_seqs([(8192, 256, BIDIR)])
    a = _attn(seqs=seqs, q=_T((256, 16, 256)), k=_T((8448, 8, 256)), hq=16, hkv=8)
    need = dg.attn_workspace_size(a)
    assert 0 < need < 2**40
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert _status(a) == dg.DG_ERR_WORKSPACE
    bad = _attn(num_seqs=0)
    assert dg.attn_workspace_size(bad) == ctypes.c_size_t(-1).value


def test_attn_workspace_single_chunk_is_zero():
    # a chunk covering all 96 keys leaves one chunk per q tile: no partials
    a = _attn()
    a.kv_chunk = 128
    assert dg.attn_workspace_size(a) == 0
    # left to the planner, a request this small is split into one-tile chunks
    a.kv_chunk = 0
    assert dg.attn_workspace_size(a) > 0


@pytest.mark.parametrize("change", [
    dict(block_size=32), dict(block_size=96), dict(block_size=-64),  # not a power of two >= 64
    dict(block_size=64, block_table=None),
    dict(block_size=64, block_table=FAKE + 2),
    dict(block_size=64, block_table_len=0),
    dict(block_size=64, block_table_len=1),  # the request needs ceil(96 / 64) = 2 entries
    dict(block_size=64, total_kv=100),  # not a multiple of block_size
])
def test_attn_paged_validation(change):
    a = _attn()
    a.block_table, a.block_table_len = FAKE, 2
    for key, val in change.items():
        setattr(a, key, val)
    assert _status(a) == dg.DG_ERR_INVALID_ARG
    assert dg.last_error()


def test_attn_paged_sizes_a_workspace_and_ignores_the_contiguous_span():
    """In paged mode kv_start indexes the table: rows past total_kv are no error."""
    a = _attn(seqs=[(0, 32, 5, 64, BIDIR)])
    a.block_size, a.block_table, a.block_table_len, a.total_kv = 64, FAKE, 7, 64
    assert dg.attn_workspace_size(a) != ctypes.c_size_t(-1).value
    a.block_table_len = 6
    assert dg.attn_workspace_size(a) == ctypes.c_size_t(-1).value


def _attn_fp8(**over):
    q = over.pop("q", _T((32, 4, 64)))
    a = dg.make_attn_args(q, _T((96, 2, 64), dtype="fp8"), _T((96, 2, 64), dtype="fp8"), _T(q.shape),
                          pack_seqs([(64, 32, BIDIR)]), -1, 4, 2, k_scale=0.5, v_scale=2.0)
    for key, val in over.items():
        setattr(a, key, val)
    return a


def test_attn_fp8_fields_and_validation():
    a = _attn_fp8()
    assert a.kv_fp8 == 1 and a.k_scale == 0.5 and a.v_scale == 2.0
    assert dg.attn_workspace_size(a) != ctypes.c_size_t(-1).value
    for change, status in [(dict(kv_fp8=2), dg.DG_ERR_INVALID_ARG), (dict(k_scale=0.0), dg.DG_ERR_INVALID_ARG),
                           (dict(v_scale=-1.0), dg.DG_ERR_INVALID_ARG),
                           (dict(k_scale=float("inf")), dg.DG_ERR_INVALID_ARG),
                           (dict(v_scale=float("nan")), dg.DG_ERR_INVALID_ARG),
                           (dict(dtype=dg.DG_F32), dg.DG_ERR_UNSUPPORTED)]:
        b = _attn_fp8(**change)
        assert _status(b) == status, change
        assert dg.last_error()
    # the binding refuses a K/V pair of which only one holds codes
    with pytest.raises(TypeError):
        dg.make_attn_args(_T((32, 4, 64)), _T((96, 2, 64), dtype="fp8"), _T((96, 2, 64)), _T((32, 4, 64)),
                          pack_seqs([(64, 32, BIDIR)]), -1, 4, 2)
    # without codes the scales are not read: zero scales are no error
    plain = _attn()
    assert plain.kv_fp8 == 0 and plain.k_scale == 0.0
    assert dg.attn_workspace_size(plain) != ctypes.c_size_t(-1).value


def test_kv_write_fp8_validation():
    a = dg.make_kv_write_args(_T((32, 2, 64)), _T((32, 2, 64)), _T((256, 2, 64), dtype="fp8"),
                              _T((256, 2, 64), dtype="fp8"), [(0, 32, 0, 10)], _T((4,), dtype="i32"), 64,
                              k_scale=0.25, v_scale=4.0)
    assert a.pool_fp8 == 1 and a.k_scale == 0.25
    lib = dg.load()
    for field, val in [("k_scale", 0.0), ("v_scale", float("nan")), ("pool_fp8", 3)]:
        old = getattr(a, field)
        setattr(a, field, val)
        assert lib.dg_kv_write(ctypes.byref(a), None) == dg.DG_ERR_INVALID_ARG, field
        assert dg.last_error()
        setattr(a, field, old)
    a.seqs[0].num = 0
    assert lib.dg_kv_write(ctypes.byref(a), None) == dg.DG_OK


def _kv(**over):
    seqs = over.pop("seqs", [(0, 32, 0, 10)])
    a = dg.make_kv_write_args(_T((32, 2, 64)), _T((32, 2, 64)), _T((256, 2, 64)), _T((256, 2, 64)), seqs,
                              _T((4,), dtype="i32"), 64)
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("change,status", [
    (dict(num_seqs=0), dg.DG_ERR_INVALID_ARG), (dict(num_seqs=65), dg.DG_ERR_INVALID_ARG),
    (dict(block_size=48), dg.DG_ERR_INVALID_ARG), (dict(block_size=0), dg.DG_ERR_INVALID_ARG),
    (dict(pool_rows=200), dg.DG_ERR_INVALID_ARG), (dict(head_dim=12), dg.DG_ERR_INVALID_ARG),
    (dict(num_kv_heads=0), dg.DG_ERR_INVALID_ARG), (dict(dtype=5), dg.DG_ERR_INVALID_ARG),
    (dict(block_table=None), dg.DG_ERR_INVALID_ARG), (dict(k_pool=FAKE + 8), dg.DG_ERR_INVALID_ARG),
    (dict(seqs=[(10, 32, 0, 0)]), dg.DG_ERR_INVALID_ARG),  # source rows past total_new
    (dict(seqs=[(0, 32, 2, 100)]), dg.DG_ERR_INVALID_ARG),  # needs entries 2..4 of a 4-entry table
    (dict(seqs=[(0, -1, 0, 0)]), dg.DG_ERR_INVALID_ARG),
])
def test_kv_write_validation(change, status):
    seqs = change.pop("seqs", None)
    a = _kv(**({"seqs": seqs} if seqs else {}))
    for key, val in change.items():
        setattr(a, key, val)
    assert dg.load().dg_kv_write(ctypes.byref(a), None) == status
    assert dg.last_error()


def test_paged_table_indices_stay_in_32_bits():
    """Table indices are 32-bit in the kernels: a table range past 2^31 - 1 is refused."""
    a = _attn(seqs=[(0, 32, 2**31 - 2, 64, BIDIR)])
    a.block_size, a.block_table, a.block_table_len, a.total_kv = 64, FAKE, 2**40, 64
    assert _status(a) == dg.DG_ERR_UNSUPPORTED
    k = _kv(seqs=[(0, 32, 2**31 - 1, 10)])
    k.block_table_len = 2**40
    assert dg.load().dg_kv_write(ctypes.byref(k), None) == dg.DG_ERR_UNSUPPORTED


def test_kv_write_nothing_to_write_is_ok():
    a = _kv(seqs=[(0, 0, 0, 0)])
    assert dg.load().dg_kv_write(ctypes.byref(a), None) == dg.DG_OK


def _inject(**over):
    a = dg.make_inject_args(_T((256,), dtype="i32"), _T((4096, 256)), _T((256, 256)), _T((256, 512)),
                            _T((256, 256)), _T((256, 256)))
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("change,status", [
    (dict(M=0), dg.DG_ERR_INVALID_ARG), (dict(vocab=0), dg.DG_ERR_INVALID_ARG),
    (dict(d=200), dg.DG_ERR_UNSUPPORTED), (dict(hidden=64), dg.DG_ERR_UNSUPPORTED),
    (dict(dtype=4), dg.DG_ERR_INVALID_ARG), (dict(tokens=None), dg.DG_ERR_INVALID_ARG),
    (dict(tokens=FAKE + 2), dg.DG_ERR_INVALID_ARG), (dict(w_down=FAKE + 8), dg.DG_ERR_INVALID_ARG),
    (dict(out=None), dg.DG_ERR_INVALID_ARG),
])
def test_inject_validation(change, status):
    a = _inject(**change)
    assert dg.load().dg_selfcond_inject(ctypes.byref(a), None) == status
    assert dg.last_error()


def test_inject_workspace():
    a = _inject()
    need = dg.inject_workspace_size(a)
    # gate/up [M, 2h] and GeGLU [M, h] intermediates at least
    assert need >= 256 * 3 * 256 * 2
    assert dg.load().dg_selfcond_inject(ctypes.byref(a), None) == dg.DG_ERR_WORKSPACE
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert dg.load().dg_selfcond_inject(ctypes.byref(a), None) == dg.DG_ERR_WORKSPACE
    assert dg.inject_workspace_size(_inject(M=0)) == ctypes.c_size_t(-1).value


def _sampler(**over):
    bufs = dg.SamplerBuffers.__new__(dg.SamplerBuffers)
    for n in ("entropy", "conf", "row_max", "row_sum", "argmax", "cand", "accept", "canvas", "prev_argmax",
              "stable_count", "num_accepted", "converged", "mean_entropy"):
        setattr(bufs, n, _T((256,)))
    logits = over.pop("logits", _T((256, 4096)))
    reqs = over.pop("reqs", [(0, 256, 1, 0)])
    a = dg.make_sampler_args(logits, reqs, 4096, bufs, 64.0)
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("change", [
    dict(num_reqs=0), dict(reqs=[(0, 1025, 1, 0)]), dict(reqs=[(200, 100, 1, 0)]),
    dict(reqs=[(0, 128, 1, 0), (100, 100, 2, 0)]), dict(reqs=[(0, 256, 1, -1)]), dict(vocab=0), dict(ld=4095),
    dict(ld=4100), dict(budget=float("inf")), dict(budget=-1.0), dict(tau=float("nan")), dict(min_accept=-1),
    dict(conf_mode=2), dict(combine=3), dict(renoise=2), dict(stable_k=0), dict(step_limit=0), dict(flags=16),
    dict(flags=4 | 8), dict(flags=4 | 2), dict(flags=8 | 2),
    dict(logits=None), dict(entropy=None), dict(accept=None), dict(canvas=FAKE + 2), dict(dtype=3),
    dict(probs=FAKE, ldq=4096), dict(probs_scale=FAKE), dict(probs=FAKE, probs_scale=FAKE, ldq=4000),
    dict(probs=FAKE + 8, probs_scale=FAKE, ldq=4096), dict(step_counter=FAKE + 2),
])
def test_sampler_validation(change):
    a = _sampler(**change)
    assert dg.load().dg_sampler_step(ctypes.byref(a), None) == dg.DG_ERR_INVALID_ARG
    assert dg.last_error()


def test_sampler_workspace():
    a = _sampler()
    need = dg.sampler_workspace_size(a)
    assert need >= 256 * 1 * 16  # one 16-byte statistics record per row and chunk
    a.workspace, a.workspace_bytes = FAKE, need - 1
    assert dg.load().dg_sampler_step(ctypes.byref(a), None) == dg.DG_ERR_WORKSPACE
    init = _sampler(flags=dg.DG_INIT_CANVAS, logits=None)
    assert dg.sampler_workspace_size(init) == 0
    # the selection alone reads neither logits nor the workspace
    sel = _sampler(flags=dg.DG_SELECT_ONLY, logits=None)
    assert dg.sampler_workspace_size(sel) == 0
    stats = _sampler(flags=dg.DG_SKIP_SELECT)
    assert dg.sampler_workspace_size(stats) == need


def _selfcond(**over):
    p = over.pop("p", _T((256, 4096)))
    e = over.pop("e", _T((4096, 256)))
    a = dg.make_selfcond_args(p, e, _T((256, 256)))
    for key, val in over.items():
        setattr(a, key[6:] if key.startswith("field_") else key, val)
    return a


@pytest.mark.parametrize("change,status", [
    (dict(M=0), dg.DG_ERR_INVALID_ARG), (dict(V=0), dg.DG_ERR_INVALID_ARG), (dict(d=200), dg.DG_ERR_UNSUPPORTED),
    (dict(ldp=4000), dg.DG_ERR_INVALID_ARG), (dict(lde=100), dg.DG_ERR_INVALID_ARG),
    (dict(ldo=100), dg.DG_ERR_INVALID_ARG), (dict(field_p=None), dg.DG_ERR_INVALID_ARG),
    (dict(embed=FAKE + 8), dg.DG_ERR_INVALID_ARG), (dict(row_max=FAKE), dg.DG_ERR_INVALID_ARG),
    (dict(row_max=FAKE, row_sum=FAKE, p_scale=FAKE), dg.DG_ERR_INVALID_ARG),
    (dict(dtype=2), dg.DG_ERR_INVALID_ARG),
])
def test_selfcond_validation(change, status):
    a = _selfcond(**change)
    assert dg.load().dg_selfcond_embed(ctypes.byref(a), None) == status
    assert dg.last_error()


def test_selfcond_workspace_is_split_k_partials():
    a = _selfcond(p=_T((256, 262144)), e=_T((262144, 2048)))
    a.d = 2048
    a.ldo = 2048
    need = dg.selfcond_workspace_size(a)
    assert need > 0 and need % (256 * 2048 * 4) == 0


def test_probe_library_exports_every_declared_function():
    """libdg_probe.so (the ceiling measurement kernels) exports what include/dg_probe.h
    declares, and refuses invalid arguments before any launch."""
    from block_denoising_step_amd import probe
    with open(os.path.join(ROOT, "include", "dg_probe.h")) as f:
        names = sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(dg_probe_\w+)\s*\(", f.read(), flags=re.M)))
    assert set(names) == set(probe.EXPORTS)
    lib = probe.load()
    for n in names:
        assert hasattr(lib, n), n
    assert lib.dg_probe_read(FAKE, 100, FAKE, 4, None) == -1  # bytes not a multiple of 16
    assert lib.dg_probe_read(FAKE, 1024, FAKE, 0, None) == -1
    assert lib.dg_probe_copy(FAKE, FAKE + 512, 1024, 4, None) == -1  # overlapping ranges
    assert lib.dg_probe_mfma_bf16(None, FAKE, 4, 0, None) == -1
    assert lib.dg_probe_mfma_bf16(None, FAKE, 4, 6, None) == -1  # not a multiple of 4


def test_force_register_staged_hook_round_trips():
    lib = dg.load()
    assert lib.dg_test_force_register_staged(1) == 0
    assert lib.dg_test_force_register_staged(0) == 1
    with dg.force_register_staged():
        assert lib.dg_test_force_register_staged(1) == 1
    assert lib.dg_test_force_register_staged(0) == 0


def test_wide_min_sub_hook_round_trips():
    lib = dg.load()
    assert lib.dg_test_wide_min_sub(16) == 64
    assert lib.dg_test_wide_min_sub(0) == 16  # < 1: back to the default
    with dg.wide_min_sub(8):
        assert lib.dg_test_wide_min_sub(8) == 8
    assert lib.dg_test_wide_min_sub(64) == 64


def test_sampler_noalloc_validation_before_any_launch():
    """dg_sampler_step_noalloc validates like dg_sampler_step (its workspace fields are
    ignored) and refuses a call that needs more than its static scratch, before any HIP
    call."""
    lib = dg.load()
    for change in (dict(num_reqs=0), dict(vocab=0), dict(flags=16), dict(entropy=None)):
        a = _sampler(**change)
        assert lib.dg_sampler_step_noalloc(ctypes.byref(a), None) == dg.DG_ERR_INVALID_ARG
    bufs = dg.SamplerBuffers.__new__(dg.SamplerBuffers)
    for n in ("entropy", "conf", "row_max", "row_sum", "argmax", "cand", "accept", "canvas", "prev_argmax",
              "stable_count", "num_accepted", "converged", "mean_entropy"):
        setattr(bufs, n, _T((2048,)))
    big = dg.make_sampler_args(_T((2048, 262144)), [(0, 1024, 1, 0), (1024, 1024, 2, 0)], 262144, bufs, 64.0)
    assert dg.sampler_workspace_size(big) > dg.DG_NOALLOC_SCRATCH_BYTES
    assert lib.dg_sampler_step_noalloc(ctypes.byref(big), None) == dg.DG_ERR_WORKSPACE
    assert "DG_NOALLOC_SCRATCH_BYTES" in dg.last_error()
