"""The no-allocation entry point (attn_prefill_split_noalloc) against the
split entry point with a caller workspace (attn_prefill_split), through the
C ABI: on every kernel configuration, forced for both calls, the outputs and
log-sum-exps are equal bit for bit, and both match the oracle.  Two calls in
a row, the second with a smaller input, so the second reuses a scratch that
still holds the first call's partials."""
import numpy as np
import pytest
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth
from parity_helpers import TOL, check_rows, f64, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # (case, n_split): the larger call first
    (synth.Case("na_big", h_q=16, h_kv=2, d=64, sq=[512, 300], past=[3000, 700], window=-1,
                seed=61), 4),
    (synth.Case("na_small", h_q=8, h_kv=2, d=64, sq=[130], past=[900], window=100, seed=62), 3),
    (synth.Case("na_bf16_d128", h_q=16, h_kv=2, d=128, sq=[200, 64], past=[450, 30], window=128,
                dtype="bf16", seed=63), 2),
]


def _each_config():
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            yield cfg
    finally:
        binding.attn_force_config(-1)


def _outputs(q, out_dtype):
    tokens, h_q, _ = q.shape
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((tokens, h_q), float("nan"), dtype=torch.float32, device="cuda")
    return out, lse


def test_noalloc_equals_workspace_entry_on_two_calls_in_a_row():
    assert torch.cuda.is_available()
    prepared = []
    for case, n_split in CASES:
        inp = synth.make(case)
        ref, ref_lse = oracle.attn_prefill_varlen(
            f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]), inp["cu_seqlens"],
            inp["past_len"], inp["window"], f64(inp["sink"]), inp["scale"], return_lse=True)
        prepared.append((case, n_split, inp, to_device(inp), ref, ref_lse))
    for cfg in _each_config():
        name = binding.attn_config_name(cfg)
        for case, n_split, inp, dev, ref, ref_lse in prepared:
            q = dev["q"]
            tokens, h_q, d = q.shape
            nbytes = binding.attn_split_workspace_bytes(tokens, h_q, d, n_split)
            assert 0 < nbytes <= binding.ATTN_NOALLOC_SCRATCH_BYTES
            ws = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda")
            a, a_lse = _outputs(q, torch.float32)
            binding.attn_prefill_split(q, dev["k_cache"], dev["v_cache"], inp["cu_seqlens"],
                                       inp["past_len"], inp["window"], dev["sink"], inp["scale"],
                                       a, lse=a_lse, n_split=n_split, workspace=ws)
            b, b_lse = _outputs(q, torch.float32)
            binding.attn_prefill_split_noalloc(q, dev["k_cache"], dev["v_cache"],
                                               inp["cu_seqlens"], inp["past_len"], inp["window"],
                                               dev["sink"], inp["scale"], b, lse=b_lse,
                                               n_split=n_split)
            torch.cuda.synchronize()
            tag = f"{case.name}[{name}]"
            assert torch.equal(a, b), tag
            assert torch.equal(a_lse, b_lse), tag
            check_rows(f64(b), ref, tag)
            assert np.abs(f64(b_lse) - ref_lse).max() <= 2e-3, tag
            # the input dtype's output as well
            c, _ = _outputs(q, q.dtype)
            binding.attn_prefill_split_noalloc(q, dev["k_cache"], dev["v_cache"],
                                               inp["cu_seqlens"], inp["past_len"], inp["window"],
                                               dev["sink"], inp["scale"], c, n_split=n_split)
            torch.cuda.synchronize()
            assert torch.isfinite(c).all(), tag


def test_noalloc_rejects_partials_above_its_scratch():
    case = synth.Case("na_huge", h_q=64, h_kv=8, d=64, sq=[2048], past=[0], window=-1, seed=64)
    inp = synth.make(case)
    dev = to_device(inp)
    n_split = 2
    need = binding.attn_split_workspace_bytes(2048, 64, 64, n_split)
    assert need > binding.ATTN_NOALLOC_SCRATCH_BYTES
    out = torch.full(dev["q"].shape, 7.0, dtype=torch.float32, device="cuda")
    code = binding.attn_prefill_split_noalloc(dev["q"], dev["k_cache"], dev["v_cache"],
                                              inp["cu_seqlens"], inp["past_len"], -1,
                                              dev["sink"], inp["scale"], out, n_split=n_split,
                                              check=False)
    torch.cuda.synchronize()
    assert code == binding.ATTN_EINVAL
    assert "scratch" in binding.attn_last_error()
    assert torch.all(out == 7.0)
