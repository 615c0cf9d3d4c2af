"""Python binding of libattn_prefill.so (the C ABI in include/attn_prefill.h).

Argument marshalling only: tensors become device pointers and sizes, the
current torch stream becomes the hipStream_t, and every step of the
attention runs in the library's HIP kernels.  There is no fallback: if the
library is not built, every call raises.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# ATTN_PREFILL_LIB may name another build of the same library (A/B timing).
LIB_PATH = os.environ.get("ATTN_PREFILL_LIB") or os.path.join(_HERE, "libattn_prefill.so")

ATTN_OK, ATTN_DECLINED, ATTN_EINVAL, ATTN_EHIP = 0, -1, -2, -3
ATTN_F16, ATTN_BF16, ATTN_F32 = 1, 2, 3
ATTN_FLAG_NONCAUSAL = 1
ATTN_LOG_FIELDS = 40
ATTN_LOG_MAX_WAVES = 8
ATTN_LOG_WAVES = 16
LOG_FIELDS = ("b", "h_first", "n_heads", "q_first", "q_last", "t_first", "t_last",
              "n_visited", "n_waves", "n_splits", "part", "n_parts", "rows_per_wave")

_DTYPE_CODE = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}

ATTN_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = ("attn_prefill", "attn_prefill_varlen", "attn_prefill_split",
            "attn_prefill_split_noalloc", "attn_prefill_paged",
            "attn_split_workspace_bytes", "attn_last_error", "attn_tune_stats",
            "attn_tune_reset", "attn_tuned_config", "attn_config_count", "attn_config_name",
            "attn_force_config")


class AttnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


class AttnDeclined(AttnError):
    pass


class TileLog(ctypes.Structure):
    _fields_ = [("records", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("n_records", ctypes.c_int64), ("bkv", ctypes.c_int32),
                ("q_rows", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)


def lib():
    """The loaded ctypes library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(hipcc for gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    L.attn_prefill.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, ctypes.c_float, _vp, _i32, _i32,
                               _i32, _i32, _i32, _i32, _i32, _vp]
    L.attn_prefill.restype = ctypes.c_int
    L.attn_prefill_varlen.argtypes = [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, _vp,
                                      ctypes.c_float, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                      ctypes.POINTER(TileLog), _vp]
    L.attn_prefill_varlen.restype = ctypes.c_int
    L.attn_prefill_split.argtypes = [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, _vp,
                                     ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                     _i32, _i32, _i32, _vp, ctypes.c_int64,
                                     ctypes.POINTER(TileLog), _vp]
    L.attn_prefill_split.restype = ctypes.c_int
    L.attn_prefill_split_noalloc.argtypes = [_vp, _vp, _vp, _i32p, _i32p, _i32, _i32, _vp,
                                             ctypes.c_float, _vp, _vp, _i32, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _i32, ctypes.POINTER(TileLog),
                                             _vp]
    L.attn_prefill_split_noalloc.restype = ctypes.c_int
    L.attn_prefill_paged.argtypes = [_vp, _vp, _vp, ctypes.c_int64, _vp, _i32p, _i32p, _i32p,
                                     _i32, _i32, _vp, ctypes.c_float, _vp, _vp, _i32, _i32,
                                     _i32, _i32, _i32, _i32, ctypes.POINTER(TileLog), _vp]
    L.attn_prefill_paged.restype = ctypes.c_int
    L.attn_split_workspace_bytes.argtypes = [ctypes.c_int64, _i32, _i32, _i32]
    L.attn_split_workspace_bytes.restype = ctypes.c_int64
    L.attn_last_error.argtypes = []
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_tune_stats.argtypes = [_i64p, _i64p, _i64p]
    L.attn_tune_stats.restype = ctypes.c_int
    L.attn_tune_reset.argtypes = []
    L.attn_tune_reset.restype = None
    L.attn_tuned_config.argtypes = [_i32, _i32, _i32, ctypes.c_int64, _i32, _i32, _i32, _i32]
    L.attn_tuned_config.restype = ctypes.c_int32
    L.attn_config_count.argtypes = []
    L.attn_config_count.restype = ctypes.c_int32
    L.attn_config_name.argtypes = [_i32]
    L.attn_config_name.restype = ctypes.c_char_p
    L.attn_force_config.argtypes = [_i32]
    L.attn_force_config.restype = ctypes.c_int
    _lib = L
    return L


def attn_last_error() -> str:
    return lib().attn_last_error().decode()


def _check(code):
    if code == ATTN_OK:
        return code
    msg = attn_last_error()
    if code == ATTN_DECLINED:
        raise AttnDeclined(code, msg)
    raise AttnError(code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _require(t, name, ndim):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in _DTYPE_CODE:
        raise ValueError(f"{name}: unsupported dtype {t.dtype}")


def _check_tensors(q, k, v, out, head_sink, n_slots=None, tokens=None, lse=None, extra=()):
    """Consistency of the tensors of one call, checked before the library is
    reached (the C ABI receives bare pointers and cannot check them): shapes
    and dtypes that agree with each other, and every tensor on the GPU.
    k / v are caches [batch, h_kv, s_cap, d] or pools [n_pool, h_kv, d]."""
    h_q, d = q.shape[1], q.shape[2]
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out {tuple(out.shape)} must have q's shape {tuple(q.shape)}")
    if out.dtype not in (q.dtype, torch.float32):
        raise ValueError(f"out dtype {out.dtype} must be q's ({q.dtype}) or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError(f"k / v dtypes ({k.dtype}, {v.dtype}) must equal q's ({q.dtype})")
    if tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"v {tuple(v.shape)} must have k's shape {tuple(k.shape)}")
    if k.shape[-1] != d:
        raise ValueError(f"head dim of k ({k.shape[-1]}) differs from q's ({d})")
    if n_slots is not None and k.shape[0] < n_slots:
        raise ValueError(f"the caches hold {k.shape[0]} sequence slots, {n_slots} needed")
    if tokens is not None and q.shape[0] != tokens:
        raise ValueError(f"q has {q.shape[0]} rows, cu_seqlens_q ends at {tokens}")
    if head_sink is not None:
        if head_sink.dtype != torch.float32 or not head_sink.is_contiguous():
            raise ValueError("head_sink must be a contiguous float32 tensor")
        if head_sink.numel() != h_q:
            raise ValueError(f"head_sink has {head_sink.numel()} entries, h_q = {h_q}")
    if lse is not None and (lse.dtype != torch.float32 or not lse.is_contiguous()
                            or tuple(lse.shape) != (q.shape[0], h_q)):
        raise ValueError("lse must be a contiguous float32 tensor [tokens, h_q]")
    named = [("q", q), ("k", k), ("v", v), ("out", out), ("head_sink", head_sink),
             ("lse", lse)] + list(extra)
    for name, t in named:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")


def _tile_log(tile_log):
    if tile_log is None:
        return None
    if (tile_log.dtype != torch.int32 or tile_log.dim() != 2
            or tile_log.shape[1] != ATTN_LOG_FIELDS or not tile_log.is_contiguous()):
        raise ValueError(f"tile_log must be a contiguous int32 tensor [capacity, {ATTN_LOG_FIELDS}]")
    if not tile_log.is_cuda:
        raise ValueError("tile_log must be a GPU tensor")
    return TileLog(tile_log.data_ptr(), tile_log.shape[0], 0, 0, 0)


def _seq_meta(cu_seqlens_q, past_len):
    nseq = len(past_len)
    if len(cu_seqlens_q) != nseq + 1:
        raise ValueError("cu_seqlens_q must have len(past_len) + 1 entries")
    cu = (ctypes.c_int32 * len(cu_seqlens_q))(*[int(x) for x in cu_seqlens_q])
    pl = (ctypes.c_int32 * max(1, nseq))(*[int(x) for x in past_len])
    return nseq, cu, pl, int(cu_seqlens_q[-1])


def attn_prefill(q, k_cache, v_cache, past_len, window, head_sink, scale, out, stream=None,
                 check=True):
    """One chunk after `past_len` cached keys.  q/out [sq, h_q, d];
    k_cache/v_cache [1, h_kv, s_cap, d]; head_sink float32 [h_q] or None."""
    _require(q, "q", 3)
    _require(out, "out", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    sq, h_q, d = q.shape
    _, h_kv, s_cap, _ = k_cache.shape
    _check_tensors(q, k_cache, v_cache, out, head_sink, n_slots=1)
    code = lib().attn_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(past_len), int(window),
                              _ptr(head_sink), float(scale), _ptr(out), sq, h_q, h_kv, d, s_cap,
                              _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], _stream(stream))
    return _check(code) if check else code


def attn_prefill_varlen(q, k_cache, v_cache, cu_seqlens_q, past_len, window, head_sink, scale,
                        out, tile_log=None, stream=None, check=True):
    """Ragged batch.  cu_seqlens_q / past_len are host sequences of ints.
    tile_log: None, or an int32 device tensor [capacity, 8] that receives the
    visited-tile records; then the return value is (code, n_records, bkv, q_rows)."""
    _require(q, "q", 3)
    _require(out, "out", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    _, h_q, d = q.shape
    batch, h_kv, s_cap, _ = k_cache.shape
    nseq, cu, pl, tokens = _seq_meta(cu_seqlens_q, past_len)
    log = _tile_log(tile_log)
    _check_tensors(q, k_cache, v_cache, out, head_sink, n_slots=nseq, tokens=tokens)
    code = lib().attn_prefill_varlen(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), cu, pl, nseq, int(window), _ptr(head_sink),
        float(scale), _ptr(out), h_q, h_kv, d, s_cap, _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype],
        ctypes.byref(log) if log is not None else None, _stream(stream))
    if check:
        _check(code)
    if log is not None:
        return code, log.n_records, log.bkv, log.q_rows
    return code


def attn_split_workspace_bytes(q_tokens, h_q, d, n_split):
    return lib().attn_split_workspace_bytes(int(q_tokens), int(h_q), int(d), int(n_split))


def attn_prefill_split(q, k_cache, v_cache, cu_seqlens_q, past_len, window, head_sink, scale,
                       out, lse=None, n_split=1, workspace=None, tile_log=None, stream=None,
                       check=True, causal=True):
    """attn_prefill_varlen with a log-sum-exp side output (lse: float32 [tokens, h_q] or
    None), KV splits across workgroups (workspace: a device tensor of at least
    attn_split_workspace_bytes(...) bytes when n_split > 1) and causal=False for
    non-causal attention (ATTN_FLAG_NONCAUSAL)."""
    _require(q, "q", 3)
    _require(out, "out", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    tokens, h_q, d = q.shape
    batch, h_kv, s_cap, _ = k_cache.shape
    nseq, cu, pl, cu_end = _seq_meta(cu_seqlens_q, past_len)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    log = _tile_log(tile_log)
    _check_tensors(q, k_cache, v_cache, out, head_sink, n_slots=nseq, tokens=cu_end, lse=lse,
                   extra=[("workspace", workspace)])
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = lib().attn_prefill_split(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), cu, pl, nseq, int(window), _ptr(head_sink),
        float(scale), _ptr(out), _ptr(lse), h_q, h_kv, d, s_cap, _DTYPE_CODE[q.dtype],
        _DTYPE_CODE[out.dtype], int(n_split), 0 if causal else ATTN_FLAG_NONCAUSAL,
        _ptr(workspace), int(ws_bytes),
        ctypes.byref(log) if log is not None else None, _stream(stream))
    if check:
        _check(code)
    if log is not None:
        return code, log.n_records, log.bkv, log.q_rows
    return code


def attn_prefill_split_noalloc(q, k_cache, v_cache, cu_seqlens_q, past_len, window, head_sink,
                               scale, out, lse=None, n_split=1, tile_log=None, stream=None,
                               check=True, causal=True):
    """attn_prefill_split without a workspace: the KV-split partials go to the
    library's static device scratch (ATTN_NOALLOC_SCRATCH_BYTES per GPU);
    nothing is allocated and no tuning sweep runs."""
    _require(q, "q", 3)
    _require(out, "out", 3)
    _require(k_cache, "k_cache", 4)
    _require(v_cache, "v_cache", 4)
    tokens, h_q, d = q.shape
    batch, h_kv, s_cap, _ = k_cache.shape
    nseq, cu, pl, cu_end = _seq_meta(cu_seqlens_q, past_len)
    log = _tile_log(tile_log)
    _check_tensors(q, k_cache, v_cache, out, head_sink, n_slots=nseq, tokens=cu_end, lse=lse)
    code = lib().attn_prefill_split_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), cu, pl, nseq, int(window), _ptr(head_sink),
        float(scale), _ptr(out), _ptr(lse), h_q, h_kv, d, s_cap, _DTYPE_CODE[q.dtype],
        _DTYPE_CODE[out.dtype], int(n_split), 0 if causal else ATTN_FLAG_NONCAUSAL,
        ctypes.byref(log) if log is not None else None, _stream(stream))
    if check:
        _check(code)
    if log is not None:
        return code, log.n_records, log.bkv, log.q_rows
    return code


def attn_prefill_paged(q, k_pool, v_pool, kv_indices, kv_indptr, cu_seqlens_q, past_len, window,
                       head_sink, scale, out, lse=None, tile_log=None, stream=None, check=True,
                       causal=True):
    """Ragged batch over a token pool: k_pool / v_pool [n_pool, h_kv, d];
    kv_indices an int32 device tensor of pool rows; kv_indptr, cu_seqlens_q and
    past_len host sequences of ints (key k of sequence b is pool row
    kv_indices[kv_indptr[b] + k])."""
    _require(q, "q", 3)
    _require(out, "out", 3)
    _require(k_pool, "k_pool", 3)
    _require(v_pool, "v_pool", 3)
    tokens, h_q, d = q.shape
    n_pool, h_kv, _ = k_pool.shape
    nseq, cu, pl, cu_end = _seq_meta(cu_seqlens_q, past_len)
    if len(kv_indptr) != nseq + 1:
        raise ValueError("kv_indptr must have len(past_len) + 1 entries")
    if kv_indices.dtype != torch.int32 or not kv_indices.is_contiguous():
        raise ValueError("kv_indices must be a contiguous int32 tensor")
    if nseq > 0 and kv_indices.numel() < int(kv_indptr[-1]):
        raise ValueError(f"kv_indices has {kv_indices.numel()} entries, kv_indptr ends at "
                         f"{int(kv_indptr[-1])}")
    log = _tile_log(tile_log)
    _check_tensors(q, k_pool, v_pool, out, head_sink, tokens=cu_end, lse=lse,
                   extra=[("kv_indices", kv_indices)])
    ip = (ctypes.c_int32 * len(kv_indptr))(*[int(x) for x in kv_indptr])
    code = lib().attn_prefill_paged(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), int(n_pool), _ptr(kv_indices), ip, cu, pl, nseq,
        int(window), _ptr(head_sink), float(scale), _ptr(out), _ptr(lse), h_q, h_kv, d,
        _DTYPE_CODE[q.dtype], _DTYPE_CODE[out.dtype], 0 if causal else ATTN_FLAG_NONCAUSAL,
        ctypes.byref(log) if log is not None else None, _stream(stream))
    if check:
        _check(code)
    if log is not None:
        return code, log.n_records, log.bkv, log.q_rows
    return code


def attn_tune_stats():
    s, l, k = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    lib().attn_tune_stats(ctypes.byref(s), ctypes.byref(l), ctypes.byref(k))
    return {"sweeps": s.value, "tuning_launches": l.value, "cached_keys": k.value}


def attn_tune_reset():
    lib().attn_tune_reset()


def attn_tuned_config(d, dtype, out_dtype, q_tokens, h_q, h_kv, window, batch):
    """Index of the configuration the tuning cache chose for this call key, or -1.
    dtype / out_dtype are torch dtypes."""
    return lib().attn_tuned_config(d, _DTYPE_CODE[dtype], _DTYPE_CODE[out_dtype], q_tokens, h_q,
                                   h_kv, window, batch)


def attn_config_count():
    return lib().attn_config_count()


def attn_config_name(i):
    n = lib().attn_config_name(i)
    return None if n is None else n.decode()


def attn_force_config(i):
    return _check(lib().attn_force_config(i))
