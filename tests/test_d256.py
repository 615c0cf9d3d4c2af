"""Head dim 256 (sglang pull request 34468 tests its kernel at head_dim
64/128/256): GPU parity against the oracle on every configuration, with a
window and sinks, bf16, a ragged batch, and KV splits with the log-sum-exp."""
import numpy as np
import pytest
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth
from parity_helpers import TOL, check_tile_log, f64, oracle_full, rel_l2, rne, run_gpu, to_device

pytestmark = pytest.mark.gpu

CASES = [
    synth.Case("d256_w100", h_q=8, h_kv=2, d=256, sq=[200], past=[300], window=100, seed=101),
    synth.Case("d256_bf16", h_q=8, h_kv=1, d=256, sq=[150], past=[450], window=-1, dtype="bf16",
               seed=102),
    synth.Case("d256_ragged", h_q=4, h_kv=2, d=256, sq=[33, 0, 97], past=[0, 10, 130],
               window=64, seed=103),
]


def _each_config():
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            yield cfg
    finally:
        binding.attn_force_config(-1)


@pytest.mark.parametrize("case", CASES, ids=lambda c: c.name)
def test_d256_matches_oracle_on_every_config(case):
    inp = synth.make(case)
    dev = to_device(inp)
    ref = oracle_full(inp)
    for cfg in _each_config():
        out, recs, bkv, q_rows = run_gpu(dev, out_dtype=torch.float32, log_capacity=4096)
        name = binding.attn_config_name(cfg)
        assert rel_l2(f64(out), ref) <= TOL, (name, rel_l2(f64(out), ref))
        assert bkv == 32, name
        check_tile_log(recs, bkv, q_rows, inp["cu_seqlens"], inp["past_len"], case.window,
                       case.h_q)
        outd, _, _, _ = run_gpu(dev)
        assert rel_l2(f64(outd), rne(ref, dev["q"].dtype)) <= TOL, name


def test_d256_split_with_lse():
    case = CASES[0]
    inp = synth.make(case)
    dev = to_device(inp)
    ref, ref_lse = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]),
                                              f64(inp["v_cache"]), inp["cu_seqlens"],
                                              inp["past_len"], case.window, f64(inp["sink"]),
                                              case.scale, return_lse=True)
    tokens, h_q, d = inp["q"].shape
    ws = torch.empty(binding.attn_split_workspace_bytes(tokens, h_q, d, 3), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(dev["q"].shape, dtype=torch.float32, device="cuda")
    lse = torch.empty((tokens, h_q), dtype=torch.float32, device="cuda")
    binding.attn_prefill_split(dev["q"], dev["k_cache"], dev["v_cache"], dev["cu_seqlens"],
                               dev["past_len"], case.window, dev["sink"], case.scale, out,
                               lse=lse, n_split=3, workspace=ws)
    torch.cuda.synchronize()
    assert rel_l2(f64(out), ref) <= TOL
    assert np.abs(f64(lse) - ref_lse).max() <= 2e-3
