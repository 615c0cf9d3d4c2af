"""Pins for the oracle's non-causal mode (every key of the sequence, above
the window's floor when one is given) against torch's
scaled_dot_product_attention in float64 (library route), plus the reading
that without a window every row of a sequence then sees the same keys."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    return np.round(rng.standard_normal(shape) * 64) / 64


def _sdpa(q, k, v, past, window, sink, scale, h_kv):
    sq, h_q, d = q.shape
    skv = past + sq
    group = h_q // h_kv
    qb = torch.from_numpy(q).permute(1, 0, 2)
    kb = torch.from_numpy(k[0, :, :skv]).repeat_interleave(group, 0)
    vb = torch.from_numpy(v[0, :, :skv]).repeat_interleave(group, 0)
    keep = torch.ones(sq, skv, dtype=torch.bool)
    if window > 0:
        keep &= keep.clone().triu(diagonal=past - window + 1)
    bias = torch.zeros(h_q, sq, skv + 1, dtype=torch.float64)
    bias[:, :, :skv].masked_fill_(~keep, float("-inf"))
    bias[:, :, skv] = float("-inf") if sink is None else torch.from_numpy(sink)[:, None]
    kx = torch.cat([kb, torch.zeros(h_q, 1, d, dtype=torch.float64)], 1)
    vx = torch.cat([vb, torch.zeros(h_q, 1, d, dtype=torch.float64)], 1)
    o = torch.nn.functional.scaled_dot_product_attention(qb, kx, vx, attn_mask=bias, scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("past,window,use_sink", [(0, -1, False), (20, -1, True), (7, 5, True),
                                                   (33, 40, False)])
def test_noncausal_matches_sdpa(past, window, use_sink):
    rng = np.random.default_rng(past + 3)
    sq, h_q, h_kv, d = 25, 4, 2, 16
    q = _rand(rng, sq, h_q, d)
    k = _rand(rng, 1, h_kv, past + sq, d)
    v = _rand(rng, 1, h_kv, past + sq, d)
    sink = _rand(rng, h_q) if use_sink else None
    scale = 1 / math.sqrt(d)
    got = oracle.attn_prefill_varlen(q, k, v, [0, sq], [past], window, sink, scale, causal=False)
    ref = _sdpa(q, k, v, past, window, sink, scale, h_kv)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_noncausal_rows_see_the_whole_sequence():
    # identical query rows then give identical outputs, wherever they sit
    rng = np.random.default_rng(4)
    q = np.repeat(_rand(rng, 1, 2, 8), 10, axis=0)
    k = _rand(rng, 1, 1, 30, 8)
    v = _rand(rng, 1, 1, 30, 8)
    out = oracle.attn_prefill_varlen(q, k, v, [0, 10], [20], -1, None, 0.3, causal=False)
    assert np.array_equal(out, np.repeat(out[:1], 10, axis=0))
    causal = oracle.attn_prefill_varlen(q, k, v, [0, 10], [20], -1, None, 0.3)
    assert not np.array_equal(causal, np.repeat(causal[:1], 10, axis=0))
