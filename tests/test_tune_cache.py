"""Tuning cache: keyed on the call shape, not on the growing KV length.

hip-ep #622, commit "tuning key": a cache keyed on skv ran one sweep per chunk
of a chunked prefill; keyed on (d, sq, H_q, G) it runs one sweep per process,
and commit "window in v5" adds the window to the key.  A chunked prefill over
full-attention and windowed layers must therefore sweep exactly twice.
"""
import pytest
import torch

from gqa_flash_attention_prefill_amd import binding, synth

pytestmark = pytest.mark.gpu


def test_one_sweep_per_layer_type_over_a_chunked_prefill(monkeypatch):
    monkeypatch.delenv("ATTN_PREFILL_TUNE", raising=False)
    monkeypatch.delenv("ATTN_PREFILL_CONFIG", raising=False)
    binding.attn_force_config(-1)
    binding.attn_tune_reset()
    chunk, n_chunks = 512, 8
    layers = []
    for window in (-1, 128):
        case = synth.Case(f"tune_w{window}", h_q=16, h_kv=2, d=64, sq=[chunk * n_chunks],
                          past=[0], window=window, seed=31, poison_tail=False)
        inp = synth.make(case, device="cuda")
        layers.append((case, inp, torch.empty_like(inp["q"])))
    for _ in range(2):                       # the second prefill must not sweep again
        for c in range(n_chunks):
            for case, inp, out in layers:
                q = inp["q"][c * chunk:(c + 1) * chunk]
                o = out[c * chunk:(c + 1) * chunk]
                binding.attn_prefill(q, inp["k_cache"], inp["v_cache"], c * chunk, case.window,
                                     inp["sink"], case.scale, o)
    torch.cuda.synchronize()
    st = binding.attn_tune_stats()
    n_cfg = binding.attn_config_count()
    assert st["sweeps"] == 2, st
    assert st["cached_keys"] == 2, st
    # each sweep times every configuration in three passes: a warm-up, a
    # first batch of three launches, a longer batch (at most 64) when three
    # take under ~150 us, and two more passes of the same length
    assert 2 * n_cfg * 10 <= st["tuning_launches"] <= 2 * n_cfg * (1 + 3 + 3 * 64), st
    for _, _, out in layers:
        assert torch.isfinite(out).all()
    # the cache answers for exactly the two swept keys
    for window in (-1, 128):
        idx = binding.attn_tuned_config(64, torch.float16, torch.float16, chunk, 16, 2, window, 1)
        assert 0 <= idx < n_cfg
    assert binding.attn_tuned_config(64, torch.float16, torch.float16, chunk, 16, 2, 64, 1) == -1
    assert binding.attn_tuned_config(64, torch.float16, torch.float16, chunk + 1, 16, 2, -1, 1) == -1


def test_disabled_tuning_uses_default_without_sweeping(monkeypatch):
    monkeypatch.setenv("ATTN_PREFILL_TUNE", "0")
    binding.attn_tune_reset()
    case = synth.Case("notune", h_q=8, h_kv=1, d=64, sq=[256], past=[100], window=-1, seed=32)
    inp = synth.make(case, device="cuda")
    out = torch.empty_like(inp["q"])
    binding.attn_prefill(inp["q"], inp["k_cache"], inp["v_cache"], 100, -1, inp["sink"],
                         case.scale, out)
    torch.cuda.synchronize()
    assert binding.attn_tune_stats()["sweeps"] == 0
    assert torch.isfinite(out).all()
