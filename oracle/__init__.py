"""ctypes wrapper for the CPU oracle (oracle/attn_oracle.c).

TEST INFRASTRUCTURE ONLY.  The oracle is the slow, plain, double-precision
correctness reference for causal grouped-query attention prefill with a
sliding window and per-head sink logits.  Only the tests, the smoke check
and the benchmark's CPU-baseline leg may import it; the GPU library and its
Python binding never do, and the two share no code.

All arrays are numpy float64 (exact copies of the fp16/bf16 inputs); layouts:
  q, out      [tokens, h_q, d]          (tokens = cu_seqlens_q[-1])
  k, v        [batch, h_kv, s_cap, d]
  sink        [h_q] or None
  lse         [tokens, h_q]             (natural log of the sum of exp over
                                         the row's kept scores; sink excluded)
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_attn_prefill_varlen.argtypes = [
        _dp, _dp, _dp, _i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32, _dp,
        ctypes.c_double, _dp, _i32]
    lib.oracle_attn_prefill_varlen.restype = ctypes.c_int
    lib.oracle_attn_prefill_varlen_lse.argtypes = [
        _dp, _dp, _dp, _i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32, _dp,
        ctypes.c_double, _dp, _dp, _i32]
    lib.oracle_attn_prefill_varlen_lse.restype = ctypes.c_int
    lib.oracle_attn_prefill_varlen_ex.argtypes = [
        _dp, _dp, _dp, _i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32, _i32, _dp,
        ctypes.c_double, _dp, _dp, _i32]
    lib.oracle_attn_prefill_varlen_ex.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [
        _dp, _dp, _dp, _i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32, _dp,
        ctypes.c_double, _i64, _i64p, _i32p, _dp, _i32]
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_rows_lse.argtypes = [
        _dp, _dp, _dp, _i32, _i32p, _i32p, _i32, _i32, _i32, _i32, _i32, _dp,
        ctypes.c_double, _i64, _i64p, _i32p, _dp, _dp, _i32]
    lib.oracle_attn_rows_lse.restype = ctypes.c_int
    lib.oracle_attn_masked.argtypes = [
        _dp, _dp, _dp, _i32, _i32, _i32, _u8p, ctypes.c_double, ctypes.c_double, _dp]
    lib.oracle_attn_masked.restype = ctypes.c_int
    lib.oracle_kept.argtypes = [_i64, _i64, _i64, _i64]
    lib.oracle_kept.restype = ctypes.c_int
    lib.oracle_tile_range.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64p, _i64p]
    lib.oracle_tile_range.restype = None
    lib.oracle_tile_has_kept.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _i64]
    lib.oracle_tile_has_kept.restype = ctypes.c_int
    lib.oracle_kept_pairs.argtypes = [_i64, _i64, _i64]
    lib.oracle_kept_pairs.restype = ctypes.c_int64
    _lib = lib
    return lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(_dp)


def _i32arr(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


def attn_prefill_varlen(q, k, v, cu_seqlens_q, past_len, window, sink, scale, threads=0,
                        return_lse=False, causal=True):
    """Full output [tokens, h_q, d] in float64 (see attn_oracle.c); with
    return_lse, also the log-sum-exp [tokens, h_q] of each row's kept scores;
    causal=False keeps every key of the sequence (above the window's floor)."""
    lib = _load()
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    tokens, h_q, d = q.shape
    batch, h_kv, s_cap, d2 = k.shape
    assert d == d2 and v.shape == k.shape
    cu, cup = _i32arr(cu_seqlens_q)
    pl, plp = _i32arr(past_len)
    assert cu.shape == (batch + 1,) and pl.shape == (batch,) and cu[-1] == tokens
    if sink is not None:
        sink, sp = _f64(sink)
    else:
        sp = None
    out = np.zeros((tokens, h_q, d), dtype=np.float64)
    lse = np.zeros((tokens, h_q), dtype=np.float64) if return_lse else None
    rc = lib.oracle_attn_prefill_varlen_ex(qp, kp, vp, batch, cup, plp, h_q, h_kv, d, s_cap,
                                           int(window), 1 if causal else 0, sp, float(scale),
                                           out.ctypes.data_as(_dp),
                                           lse.ctypes.data_as(_dp) if return_lse else None,
                                           int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_prefill_varlen rejected its arguments ({rc})")
    return (out, lse) if return_lse else out


def attn_prefill(q, k, v, past_len, window, sink, scale, threads=0, return_lse=False):
    """One sequence: q [sq, h_q, d], k/v [1, h_kv, s_cap, d] (or [h_kv, s_cap, d])."""
    k = np.asarray(k)
    v = np.asarray(v)
    if k.ndim == 3:
        k = k[None]
        v = v[None]
    sq = q.shape[0]
    return attn_prefill_varlen(q, k, v, [0, sq], [past_len], window, sink, scale, threads,
                               return_lse)


def attn_rows(q, k, v, cu_seqlens_q, past_len, window, sink, scale, row_tok, row_head,
              threads=0, return_lse=False):
    """Output rows [(row_tok[r], row_head[r])] -> array [n_rows, d] in float64
    (and, with return_lse, their log-sum-exp [n_rows])."""
    lib = _load()
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    tokens, h_q, d = q.shape
    batch, h_kv, s_cap, _ = k.shape
    cu, cup = _i32arr(cu_seqlens_q)
    pl, plp = _i32arr(past_len)
    rt = np.ascontiguousarray(row_tok, dtype=np.int64)
    rh = np.ascontiguousarray(row_head, dtype=np.int32)
    assert rt.shape == rh.shape and rt.ndim == 1
    if sink is not None:
        sink, sp = _f64(sink)
    else:
        sp = None
    out = np.zeros((rt.shape[0], d), dtype=np.float64)
    lse = np.zeros(rt.shape[0], dtype=np.float64) if return_lse else None
    rc = lib.oracle_attn_rows_lse(qp, kp, vp, batch, cup, plp, h_q, h_kv, d, s_cap, int(window),
                                  sp, float(scale), rt.shape[0], rt.ctypes.data_as(_i64p),
                                  rh.ctypes.data_as(_i32p), out.ctypes.data_as(_dp),
                                  lse.ctypes.data_as(_dp) if return_lse else None, int(threads))
    if rc != 0:
        raise ValueError(f"oracle_attn_rows rejected its arguments ({rc})")
    return (out, lse) if return_lse else out


def attn_masked(q, k, v, mask, sink, scale):
    """One head under an explicit mask: q [sq, d], k/v [skv, d], mask [sq, skv] bool.
    sink: float or None."""
    lib = _load()
    q, qp = _f64(q)
    k, kp = _f64(k)
    v, vp = _f64(v)
    sq, d = q.shape
    skv = k.shape[0]
    m = np.ascontiguousarray(mask, dtype=np.uint8)
    assert m.shape == (sq, skv)
    out = np.zeros((sq, d), dtype=np.float64)
    s = float("-inf") if sink is None else float(sink)
    rc = lib.oracle_attn_masked(qp, kp, vp, sq, skv, d, m.ctypes.data_as(_u8p), s,
                                float(scale), out.ctypes.data_as(_dp))
    if rc != 0:
        raise ValueError(f"oracle_attn_masked rejected its arguments ({rc})")
    return out


def kept(past_len, q, k, window):
    """The mask predicate: does chunk row q keep key k?"""
    return bool(_load().oracle_kept(past_len, q, k, window))


def tile_range(past_len, q_first, q_last, window, bkv):
    """(t_lo, t_hi): the KV tiles a Q tile of chunk rows [q_first, q_last] visits."""
    lo = ctypes.c_int64()
    hi = ctypes.c_int64()
    _load().oracle_tile_range(past_len, q_first, q_last, window, bkv, ctypes.byref(lo),
                              ctypes.byref(hi))
    return lo.value, hi.value


def tile_has_kept(past_len, sq, q_first, q_last, window, bkv, t):
    """Brute-force mask scan: does KV tile t hold a key some row of the Q tile keeps?"""
    return bool(_load().oracle_tile_has_kept(past_len, sq, q_first, q_last, window, bkv, t))


def kept_pairs(past_len, sq, window):
    """Number of (row, key) pairs kept by the mask for one head of one chunk."""
    return int(_load().oracle_kept_pairs(past_len, sq, window))
