"""C ABI checks that need no GPU: the library loads, exports every function
include/attn_prefill.h declares, and turns invalid or unsupported requests
into EINVAL (-2) / DECLINED (-1) before any HIP call (so no device is
needed to see them)."""
import ctypes
import os
import re

import pytest

from gqa_flash_attention_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_prefill.h")

FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def test_exports_every_declared_function(L):
    declared = _declared_functions()
    assert "attn_prefill" in declared and "attn_prefill_varlen" in declared
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(binding.EXPORTED) == declared


def _call(L, *, q=FAKE, k=FAKE, v=FAKE, out=FAKE, past=0, window=-1, sink=None, scale=0.125,
          sq=16, h_q=8, h_kv=2, d=64, s_cap=64, dtype=1, out_dtype=1):
    return L.attn_prefill(q, k, v, past, window, sink, scale, out, sq, h_q, h_kv, d, s_cap,
                          dtype, out_dtype, None)


def _varlen(L, cu, past, *, window=-1, h_q=8, h_kv=2, d=64, s_cap=64, log=None, ptr=FAKE):
    cu_a = (ctypes.c_int32 * len(cu))(*cu)
    pl_a = (ctypes.c_int32 * max(1, len(past)))(*past)
    return L.attn_prefill_varlen(ptr, ptr, ptr, cu_a, pl_a, len(past), window, None, 0.125, ptr,
                                 h_q, h_kv, d, s_cap, 1, 1, log, None)


@pytest.mark.parametrize("kw,code", [
    (dict(h_q=6, h_kv=4), binding.ATTN_EINVAL),          # h_q not a multiple of h_kv
    (dict(past=-1), binding.ATTN_EINVAL),
    (dict(past=60, sq=16, s_cap=64), binding.ATTN_EINVAL),  # past + sq > s_cap
    (dict(q=None), binding.ATTN_EINVAL),
    (dict(out=None), binding.ATTN_EINVAL),
    (dict(sq=-3), binding.ATTN_EINVAL),
    (dict(h_q=0), binding.ATTN_EINVAL),
    (dict(scale=float("nan")), binding.ATTN_EINVAL),
    (dict(d=96), binding.ATTN_DECLINED),                  # head dim not implemented
    (dict(d=512), binding.ATTN_DECLINED),                 # head dim not implemented
    (dict(dtype=3, out_dtype=3), binding.ATTN_DECLINED),  # f32 inputs
    (dict(dtype=1, out_dtype=2), binding.ATTN_DECLINED),  # f16 in, bf16 out
    (dict(q=MISALIGNED), binding.ATTN_DECLINED),
    (dict(scale=0.7), binding.ATTN_DECLINED),             # fp16: q * scale * log2 e may overflow
    (dict(scale=-0.7), binding.ATTN_DECLINED),
])
def test_rejects_before_touching_a_device(L, kw, code):
    assert _call(L, **kw) == code
    assert binding.attn_last_error() != ""


def test_empty_chunk_is_a_noop(L):
    assert _call(L, sq=0, q=None, k=None, v=None, out=None) == binding.ATTN_OK
    assert _varlen(L, [0], []) == binding.ATTN_OK
    assert _varlen(L, [0, 0, 0], [3, 5], ptr=None) == binding.ATTN_OK


@pytest.mark.parametrize("cu,past,s_cap", [
    ([1, 5], [0], 64),          # cu_seqlens must start at 0
    ([0, 8, 4], [0, 0], 64),    # decreasing
    ([0, 8, 20], [0, 50], 61),  # second sequence: 50 + 12 keys > capacity 61
    ([0, 8], [-2], 64),         # negative cached prefix
])
def test_varlen_metadata_checks(L, cu, past, s_cap):
    assert _varlen(L, cu, past, s_cap=s_cap) == binding.ATTN_EINVAL


def test_tile_log_must_be_usable(L):
    log = binding.TileLog(None, 4, 0, 0, 0)   # capacity without storage
    assert _varlen(L, [0, 8], [0], log=ctypes.byref(log)) == binding.ATTN_EINVAL


def test_configs_are_named(L):
    n = binding.attn_config_count()
    assert n >= 1
    names = [binding.attn_config_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert binding.attn_config_name(n) is None
    with pytest.raises(binding.AttnError):
        binding.attn_force_config(n)
    binding.attn_force_config(-1)


def test_tuning_stats_start_empty(L):
    binding.attn_tune_reset()
    st = binding.attn_tune_stats()
    assert st == {"sweeps": 0, "tuning_launches": 0, "cached_keys": 0}


def test_binding_refuses_bad_tensors():
    import torch
    q = torch.zeros(4, 2, 64, dtype=torch.float16)
    k = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(ValueError):
        binding.attn_prefill(q.transpose(0, 1), k, k, 0, -1, None, 0.1, q)
    with pytest.raises(ValueError):
        binding.attn_prefill(q[0], k, k, 0, -1, None, 0.1, q)


def test_split_entry_validates_before_any_gpu_call():
    L = binding.lib()
    cu = (ctypes.c_int32 * 2)(0, 64)
    past = (ctypes.c_int32 * 1)(0)
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first

    def call(n_split, ws, ws_bytes, flags=0):
        return L.attn_prefill_split(fake, fake, fake, cu, past, 1, -1, None, ctypes.c_float(0.125),
                                    fake, None, 8, 2, 64, 64, binding.ATTN_F16, binding.ATTN_F16,
                                    n_split, flags, ws, ws_bytes, None, None)

    need = binding.attn_split_workspace_bytes(64, 8, 64, 4)
    assert need == 4 * 64 * 8 * 65 * 4
    assert binding.attn_split_workspace_bytes(64, 8, 64, 1) == 0
    assert binding.attn_split_workspace_bytes(-1, 8, 64, 2) == -1
    assert call(0, fake, need) == binding.ATTN_EINVAL
    assert call(65, fake, need) == binding.ATTN_EINVAL
    assert call(4, None, need) == binding.ATTN_EINVAL
    assert call(4, fake, need - 4) == binding.ATTN_EINVAL
    assert "workspace" in binding.attn_last_error()
    assert call(4, ctypes.c_void_p(0x10004), need) == binding.ATTN_DECLINED
    assert call(1, None, 0, flags=2) == binding.ATTN_EINVAL
    assert "flags" in binding.attn_last_error()


def test_paged_entry_validates_before_any_gpu_call():
    L = binding.lib()
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first

    def call(indptr, past, sq=64, n_pool=4096, idx=fake, h_kv=2, d=64, ptr=fake):
        cu = (ctypes.c_int32 * 2)(0, sq)
        ip = None if indptr is None else (ctypes.c_int32 * len(indptr))(*indptr)
        pl = (ctypes.c_int32 * 1)(past)
        return L.attn_prefill_paged(ptr, ptr, ptr, n_pool, idx, ip, cu, pl, 1, -1, None,
                                    ctypes.c_float(0.125), ptr, None, 8, h_kv, d,
                                    binding.ATTN_F16, binding.ATTN_F16, 0, None, None)

    assert call(None, 0) == binding.ATTN_EINVAL                 # no kv_indptr
    assert call([0, 100], 0, idx=None) == binding.ATTN_EINVAL   # no kv_indices
    assert call([0, 100], 50) == binding.ATTN_EINVAL            # 100 indices for 114 keys
    assert "pool indices" in binding.attn_last_error()
    assert call([5, 3], 0) == binding.ATTN_EINVAL               # decreasing kv_indptr
    assert call([-1, 200], 0) == binding.ATTN_EINVAL            # negative start
    assert call([0, 100], 0, n_pool=0) == binding.ATTN_EINVAL
    # pool offsets are 32-bit: 2^23 rows x 2 heads x 128 x 2 bytes = 4 GiB declines
    assert call([0, 100], 0, n_pool=1 << 23, d=128) == binding.ATTN_DECLINED
    assert call([0, 100], 0, ptr=ctypes.c_void_p(0x10008)) == binding.ATTN_DECLINED


def test_noalloc_entry_checks_its_scratch_limit_before_any_gpu_call():
    L = binding.lib()
    fake = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first
    tokens = 4096
    cu = (ctypes.c_int32 * 2)(0, tokens)
    past = (ctypes.c_int32 * 1)(0)

    def call(n_split, h_q=64):
        return L.attn_prefill_split_noalloc(fake, fake, fake, cu, past, 1, -1, None,
                                            ctypes.c_float(0.125), fake, None, h_q, 8, 64, tokens,
                                            binding.ATTN_F16, binding.ATTN_F16, n_split, 0, None,
                                            None)

    assert binding.attn_split_workspace_bytes(tokens, 64, 64, 2) > binding.ATTN_NOALLOC_SCRATCH_BYTES
    assert call(2) == binding.ATTN_EINVAL
    assert "scratch" in binding.attn_last_error()
    assert call(0) == binding.ATTN_EINVAL
    assert call(2, h_q=6) == binding.ATTN_EINVAL   # h_q not a multiple of h_kv


def test_scale_limit_names_the_reason(L):
    # only requests that fail validation are made here: fake pointers never
    # reach a device
    assert _call(L, scale=0.7) == binding.ATTN_DECLINED
    assert "scale" in binding.attn_last_error()
