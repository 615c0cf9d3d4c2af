"""Non-causal attention (attn_prefill_split, causal=False): GPU parity with
the oracle's non-causal mode on every configuration, with and without a
window and KV splits, and the tile ceiling (the last key's tile for every
Q tile)."""
import numpy as np
import pytest
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth
from parity_helpers import TOL, check_tile_log, f64, new_log, rel_l2, to_device

pytestmark = pytest.mark.gpu

CASES = [
    synth.Case("nc_nowin", h_q=8, h_kv=2, d=64, sq=[333], past=[700], window=-1, seed=81),
    synth.Case("nc_w100", h_q=8, h_kv=2, d=64, sq=[250], past=[300], window=100, seed=82),
    synth.Case("nc_ragged", h_q=8, h_kv=2, d=64, sq=[70, 129], past=[0, 512], window=-1, seed=83),
    synth.Case("nc_bf16_d128", h_q=16, h_kv=2, d=128, sq=[150], past=[200], window=-1,
               dtype="bf16", seed=84),
]


def _each_config():
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            yield cfg
    finally:
        binding.attn_force_config(-1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("n_split", [1, 3])
def test_noncausal_matches_oracle(case, n_split):
    inp = synth.make(case)
    dev = to_device(inp)
    sink = f64(inp["sink"])
    ref, ref_lse = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]),
                                              f64(inp["v_cache"]), inp["cu_seqlens"],
                                              inp["past_len"], case.window, sink, case.scale,
                                              return_lse=True, causal=False)
    tokens, h_q, d = inp["q"].shape
    nbytes = binding.attn_split_workspace_bytes(tokens, h_q, d, n_split)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    for cfg in _each_config():
        out = torch.full(dev["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((tokens, h_q), float("nan"), dtype=torch.float32, device="cuda")
        log = new_log(4096, "cuda")
        _, n, bkv, q_rows = binding.attn_prefill_split(
            dev["q"], dev["k_cache"], dev["v_cache"], dev["cu_seqlens"], dev["past_len"],
            case.window, dev["sink"], case.scale, out, lse=lse, n_split=n_split, workspace=ws,
            tile_log=log, causal=False)
        torch.cuda.synchronize()
        name = binding.attn_config_name(cfg)
        assert rel_l2(f64(out), ref) <= TOL, (name, rel_l2(f64(out), ref))
        assert np.abs(f64(lse) - ref_lse).max() <= 2e-3, name
        # every Q tile walks up to the last key's tile (no causal ceiling)
        check_tile_log(log[:n].cpu().numpy(), bkv, q_rows, inp["cu_seqlens"], inp["past_len"],
                       case.window, case.h_q, causal=False)


def test_noncausal_differs_from_causal():
    case = CASES[0]
    inp = synth.make(case)
    dev = to_device(inp)
    for cfg in _each_config():
        name = binding.attn_config_name(cfg)
        outs = []
        for causal in (True, False):
            out = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
            binding.attn_prefill_split(dev["q"], dev["k_cache"], dev["v_cache"],
                                       dev["cu_seqlens"], dev["past_len"], -1, dev["sink"],
                                       case.scale, out, causal=causal)
            outs.append(out)
        torch.cuda.synchronize()
        # The last row of the chunk keeps every key either way; the first row
        # keeps its causal prefix only.  The last row agrees to the parity
        # bound, not bit for bit: the lazy rescale shares one reference-max
        # decision among a wave's rows, whose kept keys differ between the
        # modes, so that row's fp16 P is rounded against different maxima.
        last = rel_l2(f64(outs[0][-1]), f64(outs[1][-1]))
        first = rel_l2(f64(outs[0][0]), f64(outs[1][0]))
        assert last <= TOL, (name, last)
        assert first > 0.1, (name, first)
