"""Decode steps (one query row per sequence after a cached prefix) with a
sliding window and sinks: GPU parity against the oracle on every kernel
configuration, and the visited-tile records.

hip-ep pull request 622 ("Notes") leaves windowed decode with sinks
unverified on its decomposed path; here it is the same fused kernel with
sq = 1 per sequence: the window's floor clamps the KV loop to the last
`window` keys (plus the tile they start in)."""
import numpy as np
import pytest
import torch

from gqa_flash_attention_prefill_amd import binding, synth
from parity_helpers import TOL, check_tile_log, f64, oracle_full, rel_l2, rne, run_gpu, to_device

pytestmark = pytest.mark.gpu

PASTS = [0, 1, 63, 64, 127, 200, 511, 1000, 1023, 1500, 2047, 2900]


def _case(window, dtype="f16", d=64, h_q=16, h_kv=2, seed=60):
    return synth.Case(f"decode_w{window}_{dtype}_d{d}", h_q=h_q, h_kv=h_kv, d=d,
                      sq=[1] * len(PASTS), past=list(PASTS), window=window, dtype=dtype,
                      seed=seed)


def _each_config():
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            yield cfg
    finally:
        binding.attn_force_config(-1)


@pytest.mark.parametrize("window", [-1, 1, 128, 1000])
def test_decode_step_matches_oracle_on_every_config(window):
    case = _case(window)
    inp = synth.make(case)
    dev = to_device(inp)
    ref = oracle_full(inp)
    for cfg in _each_config():
        out, recs, bkv, q_rows = run_gpu(dev, out_dtype=torch.float32, log_capacity=4096)
        name = binding.attn_config_name(cfg)
        assert rel_l2(f64(out), ref) <= TOL, (name, rel_l2(f64(out), ref))
        check_tile_log(recs, bkv, q_rows, inp["cu_seqlens"], inp["past_len"], window, case.h_q)
        out16, _, _, _ = run_gpu(dev)
        assert rel_l2(f64(out16), rne(ref, torch.float16)) <= TOL, name


def test_decode_bf16_d128_tp4_heads():
    case = _case(128, dtype="bf16", d=128, h_q=16, h_kv=2, seed=61)
    inp = synth.make(case)
    dev = to_device(inp)
    ref = oracle_full(inp)
    for cfg in _each_config():
        out, _, _, _ = run_gpu(dev, out_dtype=torch.float32)
        assert rel_l2(f64(out), ref) <= TOL, binding.attn_config_name(cfg)


def test_windowed_decode_walks_at_most_the_window_tiles():
    # with window W the loop of a decode row visits the tiles holding keys
    # [past - W + 1, past]: at most ceil(W / bkv) + 1 tiles, whatever the prefix
    case = _case(128)
    inp = synth.make(case)
    dev = to_device(inp)
    for cfg in _each_config():
        _, recs, bkv, _ = run_gpu(dev, log_capacity=4096)
        assert recs[:, 7].max() <= -(-128 // bkv) + 1, binding.attn_config_name(cfg)
