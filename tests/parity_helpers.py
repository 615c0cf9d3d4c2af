"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, compare."""
import numpy as np
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth

TOL = 1e-3  # relL2 bound for fp16/bf16 inputs with fp32 accumulation


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((got - ref).ravel()) / np.linalg.norm(ref.ravel()))


def rne(ref, torch_dtype):
    """Round an oracle result to the GPU output dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(ref)).to(torch_dtype).to(torch.float64).numpy()


def to_device(inp):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return dev


def run_gpu(dev, out_dtype=None, log_capacity=0, q=None, cu=None, past=None):
    """Call attn_prefill_varlen on device inputs.  Returns (out, log, bkv, q_rows)."""
    q = dev["q"] if q is None else q
    cu = dev["cu_seqlens"] if cu is None else cu
    past = dev["past_len"] if past is None else past
    out = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=q.device)
    log = None
    if log_capacity:
        log = torch.full((log_capacity, 8), -7, dtype=torch.int32, device=q.device)
    res = binding.attn_prefill_varlen(q, dev["k_cache"], dev["v_cache"], cu, past,
                                      dev["window"], dev["sink"], dev["scale"], out, tile_log=log)
    torch.cuda.synchronize()
    if log is None:
        return out, None, None, None
    _, n, bkv, q_rows = res
    return out, log[:n].cpu().numpy(), bkv, q_rows


def oracle_full(inp):
    sink = None if inp["sink"] is None else f64(inp["sink"])
    return oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                      inp["cu_seqlens"], inp["past_len"], inp["window"], sink,
                                      inp["scale"])


def oracle_rows(inp, toks, heads, q=None, cu=None, past=None):
    sink = None if inp["sink"] is None else f64(inp["sink"])
    q = inp["q"] if q is None else q
    return oracle.attn_rows(f64(q), f64(inp["k_cache"]), f64(inp["v_cache"]),
                            inp["cu_seqlens"] if cu is None else cu,
                            inp["past_len"] if past is None else past, inp["window"], sink,
                            inp["scale"], toks, heads)


def check_tile_log(recs, bkv, q_rows, cu, past, window, h_q):
    """Every record's visited range equals the oracle's tile-floor formula
    exactly, and the records cover every (row, head) exactly once."""
    assert recs.shape[0] > 0
    tokens = cu[-1]
    cover = np.zeros((tokens, h_q), dtype=np.int64)
    for rec in recs:
        b, h0, nh, q0, q1, tf, tl, n = (int(x) for x in rec)
        assert 0 <= b < len(past)
        sq = cu[b + 1] - cu[b]
        assert 0 <= q0 <= q1 < sq and q1 - q0 + 1 <= q_rows and q0 % q_rows == 0
        lo, hi = oracle.tile_range(past[b], q0, q1, window, bkv)
        assert (tf, tl, n) == (lo, hi, hi - lo + 1), (rec, lo, hi)
        cover[cu[b] + q0:cu[b] + q1 + 1, h0:h0 + nh] += 1
    assert np.all(cover == 1)


def sample_rows(rng, tokens, h_q, n, must=()):
    toks = list(must) + list(rng.integers(0, tokens, size=n))
    heads = list(rng.integers(0, h_q, size=len(toks)))
    return np.array(toks, dtype=np.int64), np.array(heads, dtype=np.int32)


__all__ = ["TOL", "f64", "rel_l2", "rne", "to_device", "run_gpu", "oracle_full", "oracle_rows",
           "check_tile_log", "sample_rows", "synth", "binding"]
