"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the same seeded inputs, compare."""
import numpy as np
import torch

import oracle
from gqa_flash_attention_prefill_amd import binding, synth

TOL = 1e-3  # relL2 bound for fp16/bf16 inputs with fp32 accumulation
# Per-row bound: each (token, head) row's own relL2.  A row's rounding error
# (16-bit P, the pre-scaled fp16 Q, one rounding of the output) is of the
# same size as the global figure, spread over only d elements, so it stays
# within a few times TOL; a row computed from wrong keys, a wrong head or a
# wrong position is off by tens of percent.
ROW_TOL = 4e-3
# A bf16 output compared with the oracle rounded to bf16 differs only where
# the two round differently: one bf16 ulp (2^-7 of the element at most) on a
# row's largest element is a relL2 of up to 2^-7 for that row.
ROW_TOL_BF16_OUT = 2.0 ** -7


def row_tol_for(out_dtype):
    return ROW_TOL_BF16_OUT if out_dtype == torch.bfloat16 else ROW_TOL


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm((got - ref).ravel()) / np.linalg.norm(ref.ravel()))


def rne(ref, torch_dtype):
    """Round an oracle result to the GPU output dtype (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(ref)).to(torch_dtype).to(torch.float64).numpy()


def to_device(inp):
    dev = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    return dev


def new_log(capacity, device):
    """A visited-tile log buffer ([capacity, ATTN_LOG_FIELDS] int32, poisoned)."""
    return torch.full((capacity, binding.ATTN_LOG_FIELDS), -7, dtype=torch.int32, device=device)


def run_gpu(dev, out_dtype=None, log_capacity=0, q=None, cu=None, past=None):
    """Call attn_prefill_varlen on device inputs.  Returns (out, log, bkv, q_rows)."""
    q = dev["q"] if q is None else q
    cu = dev["cu_seqlens"] if cu is None else cu
    past = dev["past_len"] if past is None else past
    out = torch.full(q.shape, float("nan"), dtype=out_dtype or q.dtype, device=q.device)
    log = new_log(log_capacity, q.device) if log_capacity else None
    res = binding.attn_prefill_varlen(q, dev["k_cache"], dev["v_cache"], cu, past,
                                      dev["window"], dev["sink"], dev["scale"], out, tile_log=log)
    torch.cuda.synchronize()
    if log is None:
        return out, None, None, None
    _, n, bkv, q_rows = res
    return out, log[:n].cpu().numpy(), bkv, q_rows


def oracle_full(inp):
    sink = None if inp["sink"] is None else f64(inp["sink"])
    return oracle.attn_prefill_varlen(f64(inp["q"]), f64(inp["k_cache"]), f64(inp["v_cache"]),
                                      inp["cu_seqlens"], inp["past_len"], inp["window"], sink,
                                      inp["scale"])


def oracle_rows(inp, toks, heads, q=None, cu=None, past=None):
    sink = None if inp["sink"] is None else f64(inp["sink"])
    q = inp["q"] if q is None else q
    return oracle.attn_rows(f64(q), f64(inp["k_cache"]), f64(inp["v_cache"]),
                            inp["cu_seqlens"] if cu is None else cu,
                            inp["past_len"] if past is None else past, inp["window"], sink,
                            inp["scale"], toks, heads)


def _range(past, q_first, q_last, window, bkv, skv, causal):
    """The oracle's tile range of chunk rows [q_first, q_last]; without the
    causal bound every row keeps keys up to the sequence's last (skv - 1)."""
    lo, hi = oracle.tile_range(past, q_first, q_last, window, bkv)
    return lo, (hi if causal else (skv - 1) // bkv)


def _progression(lo, hi, base, step, offset):
    """(first, last, count) of the tiles t in [lo, hi] with (t - base) % step
    == offset, or (-1, -1, 0) if there are none."""
    if hi < lo:
        return -1, -1, 0
    first = lo + (offset - (lo - base)) % step
    last = hi - ((hi - base) - offset) % step
    if first > hi or last < lo:
        return -1, -1, 0
    return first, last, (last - first) // step + 1


def check_tile_log(recs, bkv, q_rows, cu, past, window, h_q, causal=True):
    """The visited-tile records against the oracle's tile-floor formula,
    integer for integer.  Every compared number is an observation of the
    kernel: each wave notes the tiles whose scores its softmax used, and the
    record's union is formed from those notes.  Checks:
      * each wave (32 or 64 rows, as the record says) used exactly the tiles
        of its own residue class (it takes
        every n_splits-th tile of its part of the range) that hold a key some
        row of the wave keeps (the oracle's range over the wave's rows);
      * each record's union is its part of the Q tile's range, the parts of a
        work item partition the oracle's range of the Q tile (consecutive
        parts of ceil(tiles / n_parts)), and the waves' own ranges cover it;
      * the work items cover every (row, head) exactly once."""
    assert recs.shape[0] > 0
    assert recs.shape[1] == binding.ATTN_LOG_FIELDS
    tokens = cu[-1]
    cover = np.zeros((tokens, h_q), dtype=np.int64)
    parts = {}
    W0 = binding.ATTN_LOG_WAVES
    for rec in recs:
        rec = [int(x) for x in rec]
        b, h0, nh, q0, q1, tf, tl, nv, nw, ns, part, nparts = rec[:12]
        assert 0 <= b < len(past), rec
        sq = cu[b + 1] - cu[b]
        skv = past[b] + sq
        assert 0 <= q0 <= q1 < sq and q1 - q0 + 1 <= q_rows and q0 % q_rows == 0, rec
        assert 1 <= nw <= binding.ATTN_LOG_MAX_WAVES and ns >= 1 and nw % ns == 0, rec
        rpw = rec[12]
        assert 0 <= part < nparts and rpw in (32, 64) and rec[13:16] == [0, 0, 0], rec
        lo, hi = _range(past[b], q0, q1, window, bkv, skv, causal)
        if nparts == 1:
            pl, ph = lo, hi
        else:
            per = (hi - lo + nparts) // nparts
            pl = lo + part * per
            ph = min(hi, pl + per - 1)
        want = (pl, ph, ph - pl + 1) if ph >= pl else (-1, -1, 0)
        assert (tf, tl, nv) == want, ("record union", rec[:12], want)
        n_rg = nw // ns
        union = set()
        for w in range(binding.ATTN_LOG_MAX_WAVES):
            got = tuple(rec[W0 + 3 * w:W0 + 3 * w + 3])
            if w >= nw:
                assert got == (-1, -1, 0), (rec[:12], w, got)
                continue
            rg, sp = w % n_rg, w // n_rg
            wp0 = q0 + (rg * rpw) // nh
            wp1 = min(q0 + (rg * rpw + rpw - 1) // nh, sq - 1)
            if wp0 >= sq or ph < pl:
                exp = (-1, -1, 0)
            else:
                wl, wh = _range(past[b], wp0, wp1, window, bkv, skv, causal)
                exp = _progression(max(wl, pl), min(wh, ph), pl, ns, sp)
            assert got == exp, ("wave", rec[:12], w, got, exp)
            if exp[2]:
                union.update(range(exp[0], exp[1] + 1, ns))
        assert union == set(range(pl, ph + 1)), ("waves do not cover the part", rec[:12])
        parts.setdefault((b, h0, q0), set()).add((part, nparts))
        if part == 0:
            cover[cu[b] + q0:cu[b] + q1 + 1, h0:h0 + nh] += 1
    for key, ps in parts.items():
        n = next(iter(ps))[1]
        assert ps == {(i, n) for i in range(n)}, (key, ps)
    assert np.all(cover == 1)


def row_rel_l2(got, ref):
    """relL2 of every output row (last axis), in float64."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.sqrt(((got - ref) ** 2).sum(axis=-1))
    den = np.sqrt((ref ** 2).sum(axis=-1))
    return num / np.maximum(den, 1e-300)


def check_rows(got, ref, name="", row_tol=ROW_TOL):
    """Global relL2 <= TOL, and every row's own relL2 <= row_tol."""
    err = rel_l2(got, ref)
    rows = row_rel_l2(got, ref)
    worst = float(rows.max()) if rows.size else 0.0
    print(f"{name}: relL2 {err:.3e}, worst row {worst:.3e} over {rows.size} rows", flush=True)
    assert err <= TOL, (name, err)
    assert worst <= row_tol, (name, worst, np.unravel_index(int(rows.argmax()), rows.shape))
    return err, worst


def sample_rows(rng, tokens, h_q, n, must=()):
    toks = list(must) + list(rng.integers(0, tokens, size=n))
    heads = list(rng.integers(0, h_q, size=len(toks)))
    return np.array(toks, dtype=np.int64), np.array(heads, dtype=np.int32)


__all__ = ["TOL", "ROW_TOL", "ROW_TOL_BF16_OUT", "row_tol_for", "f64", "rel_l2", "row_rel_l2", "check_rows", "rne", "to_device",
           "new_log", "run_gpu", "oracle_full", "oracle_rows", "check_tile_log", "sample_rows",
           "synth", "binding"]
