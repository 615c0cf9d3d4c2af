"""GPU parity of the token-pool KV layout (attn_prefill_paged): keys reached
through kv_indptr / kv_indices into a pool of token rows [n_pool, h_kv, d]
(sglang pull request 34468, "Commit 1").

Each sequence's dense cache rows are scattered to random rows of a pool whose
other rows hold NaN, so a key read through a wrong index shows up.  The pool
call and the dense call run the same kernels on the same values in the same
order, so on every configuration their outputs, log-sum-exps and tile logs
must be identical bit for bit; both are also checked against the oracle.  A
window-bounded index list (only the prefix keys a window row can keep) must
give the result of the full prefix.
"""
import numpy as np
import pytest
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth
from parity_helpers import TOL, check_tile_log, f64, new_log, rel_l2, to_device

pytestmark = pytest.mark.gpu

CASES = [
    synth.Case("p_ragged_w", h_q=8, h_kv=2, d=64, sq=[70, 1, 129, 300], past=[0, 517, 900, 64],
               window=100, seed=61),
    synth.Case("p_full", h_q=8, h_kv=1, d=64, sq=[256, 33], past=[640, 0], window=-1, seed=62),
    synth.Case("p_bf16_d128", h_q=16, h_kv=2, d=128, sq=[150, 64], past=[300, 1000], window=128,
               dtype="bf16", seed=63),
    synth.Case("p_d256", h_q=4, h_kv=2, d=256, sq=[90], past=[200], window=-1, seed=64),
    # long sequences: dozens of KV tiles per Q tile, so the pool-row lists of
    # the ping-pong kernel cycle through their ring many times, and Q tiles of
    # one call span 1 .. 80 tiles (every prologue / steady / tail transition)
    synth.Case("p_long", h_q=16, h_kv=2, d=64, sq=[512, 37, 200], past=[3000, 5000, 0],
               window=-1, seed=71),
    synth.Case("p_long_w_bf16", h_q=16, h_kv=2, d=64, sq=[300], past=[6000], window=1000,
               dtype="bf16", seed=72),
]


def _each_config():
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            yield cfg
    finally:
        binding.attn_force_config(-1)


def make_pool(inp, seed, keep_from=None, extra=37):
    """Scatter every sequence's keys [lo_b, past_b + sq_b) of the dense caches
    to random pool rows (lo_b = keep_from[b] or 0); the other pool rows hold
    NaN.  Returns (k_pool, v_pool, kv_indices, kv_indptr) on the host."""
    k, v = inp["k_cache"], inp["v_cache"]
    _, h_kv, _, d = k.shape
    cu, past = inp["cu_seqlens"], inp["past_len"]
    spans = []
    for b in range(len(past)):
        lo = 0 if keep_from is None else keep_from[b]
        spans.append((lo, past[b] + cu[b + 1] - cu[b]))
    total = sum(hi - lo for lo, hi in spans)
    n_pool = total + extra
    rng = np.random.default_rng(seed)
    rows = rng.permutation(n_pool)[:total]
    k_pool = torch.full((n_pool, h_kv, d), float("nan"), dtype=k.dtype)
    v_pool = torch.full((n_pool, h_kv, d), float("nan"), dtype=v.dtype)
    indptr, at = [0], 0
    for b, (lo, hi) in enumerate(spans):
        r = torch.from_numpy(rows[at:at + hi - lo])
        k_pool[r] = k[b, :, lo:hi, :].transpose(0, 1)
        v_pool[r] = v[b, :, lo:hi, :].transpose(0, 1)
        at += hi - lo
        indptr.append(at)
    return k_pool, v_pool, torch.from_numpy(rows.astype(np.int32)), indptr


def _lse_out(dev, out_dtype):
    tokens, h_q, _ = dev["q"].shape
    out = torch.full(dev["q"].shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((tokens, h_q), float("nan"), dtype=torch.float32, device="cuda")
    log = new_log(4096, "cuda")
    return out, lse, log


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_pool_equals_dense_bitwise_and_matches_oracle(case):
    inp = synth.make(case)
    dev = to_device(inp)
    k_pool, v_pool, idx, indptr = make_pool(inp, case.seed)
    k_pool, v_pool, idx = k_pool.cuda(), v_pool.cuda(), idx.cuda()
    ref = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                     inp["cu_seqlens"], inp["past_len"], inp["window"],
                                     f64(inp["sink"]), inp["scale"])
    for cfg in _each_config():
        name = binding.attn_config_name(cfg)
        a, a_lse, a_log = _lse_out(dev, torch.float32)
        res_a = binding.attn_prefill_split(dev["q"], dev["k_cache"], dev["v_cache"],
                                           inp["cu_seqlens"], inp["past_len"], inp["window"],
                                           dev["sink"], inp["scale"], a, lse=a_lse,
                                           tile_log=a_log)
        b, b_lse, b_log = _lse_out(dev, torch.float32)
        res_b = binding.attn_prefill_paged(dev["q"], k_pool, v_pool, idx, indptr,
                                           inp["cu_seqlens"], inp["past_len"], inp["window"],
                                           dev["sink"], inp["scale"], b, lse=b_lse,
                                           tile_log=b_log)
        torch.cuda.synchronize()
        assert torch.equal(a, b), name
        assert torch.equal(a_lse, b_lse), name
        assert res_a[1:] == res_b[1:], name
        n, bkv, q_rows = res_b[1:]
        assert torch.equal(a_log[:n], b_log[:n]), name
        check_tile_log(b_log[:n].cpu().numpy(), bkv, q_rows, inp["cu_seqlens"],
                       inp["past_len"], inp["window"], case.h_q)
        assert rel_l2(f64(b), ref) <= TOL, (name, rel_l2(f64(b), ref))


def test_pool_dtype_output_and_decode_rows():
    # decode-shaped: one row per sequence, fp16 output, window 128 and none
    for window in (128, -1):
        case = synth.Case("p_decode", h_q=16, h_kv=2, d=64, sq=[1] * 6,
                          past=[0, 1, 127, 128, 700, 2047], window=window, seed=65)
        inp = synth.make(case)
        dev = to_device(inp)
        k_pool, v_pool, idx, indptr = make_pool(inp, 66)
        ref = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]),
                                         f64(inp["v_cache"]), inp["cu_seqlens"],
                                         inp["past_len"], window, f64(inp["sink"]), inp["scale"])
        for cfg in _each_config():
            out = torch.full(dev["q"].shape, float("nan"), dtype=torch.float16, device="cuda")
            binding.attn_prefill_paged(dev["q"], k_pool.cuda(), v_pool.cuda(), idx.cuda(), indptr,
                                       inp["cu_seqlens"], inp["past_len"], window, dev["sink"],
                                       inp["scale"], out)
            torch.cuda.synchronize()
            assert rel_l2(f64(out), ref) <= TOL, (binding.attn_config_name(cfg), window)


def test_window_bounded_index_list_equals_full_prefix():
    # the list keeps only the prefix keys a window row can see: past' = min(past, window - 1)
    window = 100
    case = synth.Case("p_wbound", h_q=8, h_kv=2, d=64, sq=[200, 57, 1], past=[1500, 30, 4000],
                      window=window, seed=67)
    inp = synth.make(case)
    dev = to_device(inp)
    keep_from = [p - min(p, window - 1) for p in inp["past_len"]]
    past2 = [min(p, window - 1) for p in inp["past_len"]]
    k_pool, v_pool, idx, indptr = make_pool(inp, 68, keep_from=keep_from)
    ref = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                     inp["cu_seqlens"], inp["past_len"], window,
                                     f64(inp["sink"]), inp["scale"])
    for cfg in _each_config():
        out = torch.full(dev["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
        binding.attn_prefill_paged(dev["q"], k_pool.cuda(), v_pool.cuda(), idx.cuda(), indptr,
                                   inp["cu_seqlens"], past2, window, dev["sink"], inp["scale"],
                                   out)
        torch.cuda.synchronize()
        assert torch.all(torch.isfinite(out)), binding.attn_config_name(cfg)
        assert rel_l2(f64(out), ref) <= TOL, binding.attn_config_name(cfg)


def test_noncausal_pool_call():
    case = synth.Case("p_nc", h_q=8, h_kv=2, d=64, sq=[90, 40], past=[100, 0], window=-1, seed=69)
    inp = synth.make(case)
    dev = to_device(inp)
    k_pool, v_pool, idx, indptr = make_pool(inp, 70)
    ref = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                     inp["cu_seqlens"], inp["past_len"], -1, f64(inp["sink"]),
                                     inp["scale"], causal=False)
    out = torch.full(dev["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
    binding.attn_prefill_paged(dev["q"], k_pool.cuda(), v_pool.cuda(), idx.cuda(), indptr,
                               inp["cu_seqlens"], inp["past_len"], -1, dev["sink"], inp["scale"],
                               out, causal=False)
    torch.cuda.synchronize()
    assert rel_l2(f64(out), ref) <= TOL


def _random_pool_cases(n=12, seed=3031):
    """Seeded random ragged batches for the token-pool layout: long prefixes
    (so the ping-pong kernel's LDS row ring wraps many times), empty and
    one-row sequences, windows from none to wider than the sequence, both
    dtypes, d 64 and 128."""
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (16, 2), (64, 8), (8, 1)]
    out = []
    for i in range(n):
        h_q, h_kv = heads[rng.integers(len(heads))]
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        nb = int(rng.integers(1, 4))
        sq = [int(rng.choice([0, 1, 16, 77, 130, 300])) for _ in range(nb)]
        if sum(sq) == 0:
            sq[0] = 50
        past = [int(rng.choice([0, 63, 700, 2100, 4100])) for _ in range(nb)]
        window = int(rng.choice([-1, -1, 1, 128, 1000]))
        out.append(synth.Case(f"prand{i}_{h_q}x{h_kv}_d{d}_{dtype}_w{window}", h_q=h_q, h_kv=h_kv,
                              d=d, sq=sq, past=past, window=window, dtype=dtype, seed=900 + i))
    return out


@pytest.mark.parametrize("case", _random_pool_cases(), ids=lambda c: c.name)
def test_random_pool_shapes_every_config(case):
    test_pool_equals_dense_bitwise_and_matches_oracle(case)
