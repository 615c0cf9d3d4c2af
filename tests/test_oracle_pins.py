"""Pins for the CPU oracle: checks against things other than the oracle itself.

* A library route: torch's scaled_dot_product_attention in float64 on the
  CPU, with K/V expanded per q head (repeat_interleave, the "expand" form of
  GQA) and the mask built from tril/triu; the sink is an extra key whose
  score is the sink logit (k = 0 plus an additive bias) and whose value row
  is zero.
* Closed forms: window 1 returns the query's own value row; window 1 with a
  sink scales it by 1 / (1 + exp(sink - s)); identical keys give the mean of
  the visible value rows with the sink's share taken out.
* Invariants from the pages: sink = -inf equals no sink; a window at least as
  long as the sequence equals no window; chunked rows equal the same rows of
  one whole-sequence prefill; a fully masked row is 0 and finite; shifting
  every score and the sink by one constant changes nothing.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(rng, *shape):
    # values on a coarse binary grid so inputs are exact in fp16 as well
    return np.round(rng.standard_normal(shape) * 64) / 64


def _inputs(seed, batch, h_q, h_kv, d, sq, past, s_cap=None):
    rng = np.random.default_rng(seed)
    need = max(p + s for p, s in zip(past, sq))
    cap = s_cap or need
    q = _rand(rng, sum(sq), h_q, d)
    k = _rand(rng, batch, h_kv, cap, d)
    v = _rand(rng, batch, h_kv, cap, d)
    sink = _rand(rng, h_q)
    cu = np.concatenate([[0], np.cumsum(sq)]).astype(np.int32)
    return q, k, v, sink, cu


def _sdpa_reference(q, k, v, cu, past, window, sink, scale, h_kv):
    """Library route, float64: F.scaled_dot_product_attention per sequence."""
    tokens, h_q, d = q.shape
    group = h_q // h_kv
    out = np.zeros_like(q)
    for b in range(len(past)):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        sq = s1 - s0
        if sq == 0:
            continue
        skv = past[b] + sq
        qb = torch.from_numpy(q[s0:s1]).permute(1, 0, 2)                  # [h_q, sq, d]
        kb = torch.from_numpy(k[b, :, :skv]).repeat_interleave(group, 0)  # [h_q, skv, d]
        vb = torch.from_numpy(v[b, :, :skv]).repeat_interleave(group, 0)
        ones = torch.ones(sq, skv, dtype=torch.bool)
        keep = ones.tril(diagonal=past[b])                 # key <= past + row
        if window > 0:
            keep &= ones.triu(diagonal=past[b] - window + 1)   # key >= past + row - window + 1
        bias = torch.zeros(h_q, sq, skv + 1, dtype=torch.float64)
        bias[:, :, :skv].masked_fill_(~keep, float("-inf"))
        if sink is None:
            bias[:, :, skv] = float("-inf")
        else:
            bias[:, :, skv] = torch.from_numpy(np.asarray(sink, dtype=np.float64))[:, None]
        kx = torch.cat([kb, torch.zeros(h_q, 1, d, dtype=torch.float64)], 1)
        vx = torch.cat([vb, torch.zeros(h_q, 1, d, dtype=torch.float64)], 1)
        o = torch.nn.functional.scaled_dot_product_attention(qb, kx, vx, attn_mask=bias,
                                                             scale=scale)
        out[s0:s1] = o.permute(1, 0, 2).numpy()
    return out


SDPA_CASES = [
    # batch, h_q, h_kv, d, sq, past, window, sink
    (1, 4, 1, 16, [37], [0], -1, False),
    (1, 4, 1, 16, [37], [0], -1, True),
    (1, 4, 2, 32, [40], [19], 5, True),
    (1, 8, 2, 16, [33], [70], 17, True),
    (1, 6, 3, 8, [25], [3], 1, True),
    (3, 4, 2, 16, [9, 30, 17], [0, 45, 8], 12, True),
    (3, 4, 4, 64, [16, 1, 20], [5, 0, 64], -1, True),
    (2, 2, 1, 128, [20, 12], [10, 40], 100, False),
]


@pytest.mark.parametrize("case", SDPA_CASES)
def test_matches_sdpa_library_route(case):
    batch, h_q, h_kv, d, sq, past, window, use_sink = case
    q, k, v, sink, cu = _inputs(7 + d + sum(sq), batch, h_q, h_kv, d, sq, past)
    sink = sink if use_sink else None
    scale = 1.0 / math.sqrt(d)
    got = oracle.attn_prefill_varlen(q, k, v, cu, past, window, sink, scale)
    ref = _sdpa_reference(q, k, v, cu, past, window, sink, scale, h_kv)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_window_one_is_own_value_row():
    # hip-ep #622, "harness: window cases": window = 1 reduces to each query
    # seeing only itself, so the output is exactly that key's value row.
    q, k, v, _, cu = _inputs(3, 1, 4, 2, 16, [21], [11])
    out = oracle.attn_prefill_varlen(q, k, v, cu, [11], 1, None, 0.25)
    for i in range(21):
        for h in range(4):
            assert np.array_equal(out[i, h], v[0, h // 2, 11 + i])


def test_window_one_with_sink_closed_form():
    # one kept key with score s and a sink logit: weight 1 / (1 + exp(sink - s))
    q, k, v, sink, cu = _inputs(4, 1, 4, 1, 16, [13], [6])
    scale = 0.3
    out = oracle.attn_prefill_varlen(q, k, v, cu, [6], 1, sink, scale)
    for i in range(13):
        for h in range(4):
            s = scale * float(np.dot(q[i, h], k[0, 0, 6 + i]))
            expect = v[0, 0, 6 + i] / (1.0 + math.exp(sink[h] - s))
            np.testing.assert_allclose(out[i, h], expect, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("window", [-1, 1, 3, 8, 50])
@pytest.mark.parametrize("use_sink", [False, True])
def test_identical_keys_average_visible_values(window, use_sink):
    # all keys equal => all kept scores equal to s; out = sum(v_kept) / (n + exp(sink - s))
    rng = np.random.default_rng(11)
    past, sq, d, h_q = 9, 14, 8, 2
    q = _rand(rng, sq, h_q, d)
    key = _rand(rng, d)
    k = np.broadcast_to(key, (1, 1, past + sq, d)).copy()
    v = _rand(rng, 1, 1, past + sq, d)
    sink = _rand(rng, h_q) if use_sink else None
    scale = 0.5
    out = oracle.attn_prefill_varlen(q, k, v, [0, sq], [past], window, sink, scale)
    for i in range(sq):
        pos = past + i
        lo = 0 if window <= 0 else max(0, pos - window + 1)
        n = pos - lo + 1
        for h in range(h_q):
            s = scale * float(np.dot(q[i, h], key))
            denom = n + (math.exp(sink[h] - s) if use_sink else 0.0)
            expect = v[0, 0, lo:pos + 1].sum(0) / denom
            np.testing.assert_allclose(out[i, h], expect, rtol=1e-12, atol=1e-14)


def test_sink_minus_inf_equals_no_sink_bitwise():
    q, k, v, _, cu = _inputs(5, 2, 8, 2, 32, [20, 7], [5, 33])
    none = oracle.attn_prefill_varlen(q, k, v, cu, [5, 33], 9, None, 0.2)
    neg = oracle.attn_prefill_varlen(q, k, v, cu, [5, 33], 9, np.full(8, -np.inf), 0.2)
    assert np.array_equal(none, neg)


@pytest.mark.parametrize("window", [0, 40, 41, 1000])
def test_wide_window_equals_causal_bitwise(window):
    # hip-ep #622 and sglang #34468: a window wider than the sequence must
    # reproduce full attention exactly; window <= 0 disables it.
    q, k, v, sink, cu = _inputs(6, 1, 4, 2, 16, [25], [15])
    full = oracle.attn_prefill_varlen(q, k, v, cu, [15], -1, sink, 0.25)
    win = oracle.attn_prefill_varlen(q, k, v, cu, [15], window, sink, 0.25)
    assert np.array_equal(full, win)


@pytest.mark.parametrize("window", [-1, 6, 64])
def test_chunked_rows_equal_whole_prefill_rows_bitwise(window):
    # a chunk of sq rows after past cached keys computes rows [past, past+sq)
    # of one prefill over the whole sequence
    past, sq, total = 48, 20, 80
    rng = np.random.default_rng(12)
    q_all = _rand(rng, total, 4, 16)
    k = _rand(rng, 1, 2, total, 16)
    v = _rand(rng, 1, 2, total, 16)
    sink = _rand(rng, 4)
    whole = oracle.attn_prefill_varlen(q_all, k, v, [0, total], [0], window, sink, 0.25)
    chunk = oracle.attn_prefill_varlen(q_all[past:past + sq], k, v, [0, sq], [past], window,
                                       sink, 0.25)
    assert np.array_equal(chunk, whole[past:past + sq])


def test_common_shift_of_scores_and_sink_is_invariant():
    # adding u to every key shifts every score by c = scale * <q, u>; shifting
    # the sink by the same c leaves the softmax unchanged (sink is in
    # scaled-score units, hip-ep #622 "fold sink into v5 epilogue")
    rng = np.random.default_rng(13)
    sq, d = 12, 16
    q = _rand(rng, sq, 1, d)
    k = _rand(rng, 1, 1, sq, d)
    v = _rand(rng, 1, 1, sq, d)
    u = _rand(rng, d)
    scale = 0.4
    for i in range(sq):
        row_q = q[i:i + 1]
        c = scale * float(np.dot(row_q[0, 0], u))
        sink = np.array([0.7])
        base = oracle.attn_prefill_varlen(row_q, k[:, :, :i + 1], v[:, :, :i + 1], [0, 1],
                                          [i], -1, sink, scale)
        shifted = oracle.attn_prefill_varlen(row_q, k[:, :, :i + 1] + u, v[:, :, :i + 1],
                                             [0, 1], [i], -1, sink + c, scale)
        np.testing.assert_allclose(shifted, base, rtol=1e-12, atol=1e-14)


def test_fully_masked_row_is_zero_and_finite():
    # hip-ep #622, "fold sink into v5 epilogue": a row whose max stays -inf
    # skips the sink and keeps the clamped denominator -> output 0, no NaN
    rng = np.random.default_rng(14)
    q = _rand(rng, 4, 8)
    k = _rand(rng, 6, 8)
    v = _rand(rng, 6, 8)
    mask = np.ones((4, 6), dtype=bool)
    mask[1] = False
    mask[3] = False
    for sink in (None, 2.5):
        out = oracle.attn_masked(q, k, v, mask, sink, 0.3)
        assert np.all(np.isfinite(out))
        assert np.array_equal(out[1], np.zeros(8)) and np.array_equal(out[3], np.zeros(8))
        assert np.any(out[0] != 0)


def test_masked_entry_agrees_with_prefill_entry():
    q, k, v, sink, cu = _inputs(15, 1, 1, 1, 16, [18], [7])
    win = 5
    mask = np.array([[oracle.kept(7, i, j, win) for j in range(25)] for i in range(18)])
    a = oracle.attn_masked(q[:, 0], k[0, 0, :25], v[0, 0, :25], mask, sink[0], 0.25)
    b = oracle.attn_prefill_varlen(q, k, v, cu, [7], win, sink[:1], 0.25)[:, 0]
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_rows_entry_equals_full_output_bitwise():
    q, k, v, sink, cu = _inputs(16, 3, 4, 2, 16, [10, 3, 8], [4, 0, 30], s_cap=40)
    full = oracle.attn_prefill_varlen(q, k, v, cu, [4, 0, 30], 7, sink, 0.25)
    toks = np.array([0, 9, 10, 12, 13, 20])
    heads = np.array([0, 3, 1, 2, 3, 0])
    rows = oracle.attn_rows(q, k, v, cu, [4, 0, 30], 7, sink, 0.25, toks, heads)
    assert np.array_equal(rows, full[toks, heads])


def test_keys_beyond_the_sequence_are_never_read():
    # NaN in cache positions >= past + sq must not reach the output
    q, k, v, sink, cu = _inputs(17, 2, 4, 2, 16, [6, 9], [3, 1], s_cap=24)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 9:] = np.nan
    v2[0, :, 9:] = np.nan
    k2[1, :, 10:] = np.nan
    v2[1, :, 10:] = np.nan
    a = oracle.attn_prefill_varlen(q, k, v, cu, [3, 1], -1, sink, 0.25)
    b = oracle.attn_prefill_varlen(q, k2, v2, cu, [3, 1], -1, sink, 0.25)
    assert np.array_equal(a, b)


def test_rejects_invalid_arguments():
    q, k, v, sink, cu = _inputs(18, 1, 4, 2, 16, [8], [2])
    with pytest.raises(ValueError):
        oracle.attn_prefill_varlen(q, k, v, cu, [3], -1, sink, 0.25)  # past + sq > s_cap


def test_kept_pairs_counts_the_mask():
    for past in (0, 5, 64):
        for sq in (1, 7, 40):
            for window in (-1, 1, 3, 16, 200):
                brute = sum(oracle.kept(past, i, j, window)
                            for i in range(sq) for j in range(past + sq))
                assert oracle.kept_pairs(past, sq, window) == brute
