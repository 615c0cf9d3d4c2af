"""Pins for the oracle's log-sum-exp side output (lse of each row's kept,
scaled scores; natural log; sink excluded), against things other than the
oracle itself:

* a library route: torch.logsumexp in float64 over the masked score matrix
  built with torch (K expanded per q head, mask from tril/triu);
* closed forms: q = 0 gives lse = ln(number of kept keys); window 1 gives the
  diagonal score itself;
* invariants: the sink does not enter the lse; chunked rows equal the rows of
  one whole-sequence prefill; the rows entry agrees with the full entry.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    return np.round(rng.standard_normal(shape) * 64) / 64


def _inputs(seed, batch, h_q, h_kv, d, sq, past):
    rng = np.random.default_rng(seed)
    cap = max(p + s for p, s in zip(past, sq))
    q = _rand(rng, sum(sq), h_q, d)
    k = _rand(rng, batch, h_kv, cap, d)
    v = _rand(rng, batch, h_kv, cap, d)
    sink = _rand(rng, h_q)
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    return q, k, v, sink, cu


def _torch_lse(q, k, cu, past, window, scale, h_kv):
    tokens, h_q, d = q.shape
    group = h_q // h_kv
    out = np.zeros((tokens, h_q))
    for b in range(len(past)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sq = s1 - s0
        if sq == 0:
            continue
        skv = past[b] + sq
        qb = torch.from_numpy(q[s0:s1]).permute(1, 0, 2)                  # [h_q, sq, d]
        kb = torch.from_numpy(k[b, :, :skv]).repeat_interleave(group, 0)  # [h_q, skv, d]
        s = torch.matmul(qb, kb.transpose(1, 2).contiguous()) * scale     # [h_q, sq, skv]
        ones = torch.ones(sq, skv, dtype=torch.bool)
        keep = ones.tril(diagonal=past[b])
        if window > 0:
            keep &= ones.triu(diagonal=past[b] - window + 1)
        s = s.masked_fill(~keep, float("-inf"))
        out[s0:s1] = torch.logsumexp(s, dim=-1).permute(1, 0).numpy()
    return out


CASES = [
    # batch, h_q, h_kv, d, sq, past, window
    (1, 4, 1, 16, [37], [0], -1),
    (1, 4, 2, 32, [40], [19], 5),
    (1, 8, 2, 16, [33], [70], 17),
    (3, 4, 2, 16, [9, 30, 17], [0, 45, 8], 12),
    (2, 2, 1, 128, [20, 12], [10, 40], 100),
]


@pytest.mark.parametrize("case", CASES)
def test_lse_matches_torch_logsumexp(case):
    batch, h_q, h_kv, d, sq, past, window = case
    q, k, v, sink, cu = _inputs(11 + d + sum(sq), batch, h_q, h_kv, d, sq, past)
    scale = 1.0 / math.sqrt(d)
    _, lse = oracle.attn_prefill_varlen(q, k, v, cu, past, window, sink, scale, return_lse=True)
    ref = _torch_lse(q, k, cu, past, window, scale, h_kv)
    np.testing.assert_allclose(lse, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [-1, 1, 7, 50])
def test_zero_queries_give_log_of_kept_count(window):
    q, k, v, sink, cu = _inputs(3, 1, 4, 2, 16, [30], [25])
    q[:] = 0.0
    _, lse = oracle.attn_prefill_varlen(q, k, v, cu, [25], window, sink, 0.25, return_lse=True)
    for row in range(30):
        pos = 25 + row
        count = pos + 1 if window <= 0 else min(pos + 1, window)
        assert lse[row].tolist() == pytest.approx([math.log(count)] * 4, abs=1e-13)


def test_window_one_lse_is_the_diagonal_score():
    q, k, v, sink, cu = _inputs(5, 1, 4, 2, 32, [21], [9])
    scale = 0.125
    _, lse = oracle.attn_prefill_varlen(q, k, v, cu, [9], 1, sink, scale, return_lse=True)
    for row in range(21):
        for h in range(4):
            s = scale * float(np.dot(q[row, h], k[0, h // 2, 9 + row]))
            assert lse[row, h] == pytest.approx(s, abs=1e-13)


def test_sink_does_not_enter_the_lse():
    q, k, v, sink, cu = _inputs(8, 1, 4, 1, 16, [19], [6])
    _, a = oracle.attn_prefill_varlen(q, k, v, cu, [6], 4, sink, 0.3, return_lse=True)
    _, b = oracle.attn_prefill_varlen(q, k, v, cu, [6], 4, None, 0.3, return_lse=True)
    assert np.array_equal(a, b)


def test_chunked_rows_lse_equal_whole_prefill():
    q, k, v, sink, cu = _inputs(9, 1, 4, 2, 16, [48], [0])
    _, whole = oracle.attn_prefill_varlen(q, k, v, cu, [0], 9, sink, 0.25, return_lse=True)
    for c0 in (0, 16, 32):
        _, part = oracle.attn_prefill_varlen(q[c0:c0 + 16], k, v, [0, 16], [c0], 9, sink, 0.25,
                                             return_lse=True)
        assert np.array_equal(part, whole[c0:c0 + 16])


def test_rows_entry_lse_equals_full_entry():
    q, k, v, sink, cu = _inputs(10, 2, 4, 2, 16, [12, 20], [3, 30])
    _, full = oracle.attn_prefill_varlen(q, k, v, cu, [3, 30], 6, sink, 0.25, return_lse=True)
    toks = np.array([0, 5, 11, 12, 20, 31])
    heads = np.array([0, 3, 1, 2, 0, 3], dtype=np.int32)
    _, rows = oracle.attn_rows(q, k, v, cu, [3, 30], 6, sink, 0.25, toks, heads, return_lse=True)
    assert np.array_equal(rows, full[toks, heads])
