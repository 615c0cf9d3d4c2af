"""Layouts and variants served by the existing calls.

* Window-bounded prefix layout (sglang pull request 34468, "Commit 1" body:
  its attention backend hands sliding-window layers window_kv_indptr/indices,
  so the kernel sees a prefix of min(prefix, window) tokens): a cache that
  holds only the last min(past, window) prefix keys, passed with that as
  past_len, must give the rows of the full-prefix layout, because both mask
  bounds compare a key with its own row's position and shift together.
* smooth_softmax (hip-ep pull request 622, "harness: sink cases"): read as a
  zero sink logit on every head (one extra zero logit in the denominator),
  i.e. head_sink = zeros.
"""
import numpy as np
import pytest
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth
from parity_helpers import TOL, f64, rel_l2

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("past,window", [(3000, 128), (100, 128), (999, 1), (2048, 513)])
def test_window_bounded_prefix_layout_matches_full_layout(past, window):
    sq = 300
    case = synth.Case("wb", h_q=16, h_kv=2, d=64, sq=[sq], past=[past], window=window, seed=91,
                      poison_tail=False)
    full = synth.make(case)
    ref = oracle.attn_prefill_varlen(f64(full["q"]), f64(full["k_cache"]), f64(full["v_cache"]),
                                     [0, sq], [past], window, f64(full["sink"]), case.scale)
    keep = min(past, window)
    k_w = full["k_cache"][:, :, past - keep:past + sq].contiguous().cuda()
    v_w = full["v_cache"][:, :, past - keep:past + sq].contiguous().cuda()
    q = full["q"].cuda()
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    binding.attn_prefill(q, k_w, v_w, keep, window, full["sink"].cuda(), case.scale, out)
    torch.cuda.synchronize()
    assert rel_l2(f64(out), ref) <= TOL


def test_smooth_softmax_is_a_zero_sink():
    case = synth.Case("smooth", h_q=8, h_kv=2, d=64, sq=[200], past=[300], window=-1, seed=92)
    inp = synth.make(case)
    zeros = torch.zeros(8, dtype=torch.float32)
    ref = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                     [0, 200], [300], -1, np.zeros(8), case.scale)
    out = torch.empty(inp["q"].shape, dtype=torch.float32, device="cuda")
    binding.attn_prefill(inp["q"].cuda(), inp["k_cache"].cuda(), inp["v_cache"].cuda(), 300, -1,
                         zeros.cuda(), case.scale, out)
    torch.cuda.synchronize()
    assert rel_l2(f64(out), ref) <= TOL
    # and it differs from no sink by the expected factor per row: out_smooth =
    # out_plain * l / (l + exp(-m)), i.e. never larger in magnitude
    plain = oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                       [0, 200], [300], -1, None, case.scale)
    assert np.all(np.abs(ref) <= np.abs(plain) + 1e-12)
