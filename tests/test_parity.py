"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bar: relL2 <= 1e-3 for the fp32 output and for the
fp16/bf16 output against the oracle rounded to that dtype; the visited-tile
records equal the tile-floor formula exactly; no NaN anywhere (cache
positions past each sequence's keys hold NaN, so a stray read shows)."""
import numpy as np
import pytest
import torch

import oracle
from parity_helpers import (TOL, binding, check_rows, check_tile_log, f64, new_log, oracle_full,
                            oracle_rows, rel_l2, rne, row_tol_for, run_gpu, sample_rows, synth,
                            to_device)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    binding.lib()
    yield


def _full_check(case, out_dtypes=("same", "f32"), log=True, every_config=False):
    """Whole output against the oracle (and the tile log against the floor
    formula); with every_config, once per kernel configuration, forced."""
    inp = synth.make(case)
    dev = to_device(inp)
    ref = oracle_full(inp)
    for cfg in (_each_config() if every_config else [None]):
        name = case.name if cfg is None else f"{case.name}[{binding.attn_config_name(cfg)}]"
        for od in out_dtypes:
            tdt = case.torch_dtype if od == "same" else torch.float32
            cap = case.tokens * case.h_q if log else 0
            out, recs, bkv, q_rows = run_gpu(dev, out_dtype=tdt, log_capacity=cap)
            got = f64(out)
            assert np.all(np.isfinite(got)), f"{name}: non-finite output"
            expect = ref if tdt == torch.float32 else rne(ref, tdt)
            check_rows(got, expect, f"{name} out={od}", row_tol=row_tol_for(tdt))
            if log:
                check_tile_log(recs, bkv, q_rows, case.cu_seqlens, case.past, case.window, case.h_q)
    return ref


def test_tiny_config():
    _full_check(synth.tiny())


MID = [
    # (name, h_q, h_kv, d, sq, past, window, dtype, sink)
    ("g4_w100_past700", 8, 2, 64, [333], [700], 100, "f16", True),
    ("g4_nowin_past700", 8, 2, 64, [333], [700], -1, "f16", True),
    ("g4_w128_past0", 8, 2, 64, [333], [0], 128, "f16", True),
    ("g4_w129", 8, 2, 64, [257], [129], 129, "f16", False),
    ("g4_w1", 8, 2, 64, [100], [37], 1, "f16", True),
    ("g4_wide", 8, 2, 64, [100], [37], 5000, "f16", True),
    ("g8_w128_past8192", 16, 2, 64, [130], [8192], 128, "f16", True),
    ("g8_d128_bf16", 16, 2, 128, [300], [450], 128, "bf16", True),
    ("g8_d128_bf16_nowin", 16, 2, 128, [300], [450], -1, "bf16", True),
    ("g8_d128_f16", 16, 2, 128, [190], [65], 100, "f16", True),
    ("g8_d64_bf16", 16, 2, 64, [190], [65], 63, "bf16", True),
    ("g1_mha", 4, 4, 64, [150], [90], 65, "f16", True),
    ("g3_odd_group", 6, 2, 64, [150], [90], 100, "f16", True),
    ("g16", 16, 1, 64, [77], [200], 33, "f16", True),
    ("g64_mqa", 64, 1, 64, [40], [100], -1, "f16", True),
    ("ragged_f16", 8, 2, 64, [1, 0, 77, 200, 5], [0, 5, 300, 64, 1000], 100, "f16", True),
    ("ragged_bf16_d128", 8, 1, 128, [129, 3, 64], [0, 700, 1], -1, "bf16", True),
    # an empty first sequence: every work item's sequence is found by the
    # search past the first table entry
    ("ragged_first_empty", 8, 2, 64, [0, 45, 0, 130], [5, 0, 7, 200], 64, "f16", True),
    # more sequences than one launch's table holds (128): the call is split
    # into launches whose tables start at sequence 128
    ("ragged_150_seqs", 8, 2, 64, [(7 * i) % 6 for i in range(150)],
     [(37 * i) % 301 for i in range(150)], 50, "f16", True),
]


@pytest.mark.parametrize("spec", MID, ids=[m[0] for m in MID])
def test_mid_cases(spec):
    name, h_q, h_kv, d, sq, past, window, dtype, sink = spec
    case = synth.Case(name, h_q=h_q, h_kv=h_kv, d=d, sq=sq, past=past, window=window,
                      dtype=dtype, sink=sink, seed=77 + sum(sq) + sum(past),
                      s_cap=max(p + s for p, s in zip(past, sq)) + 23)
    _full_check(case, every_config=True)


def _random_cases(n=24, seed=2024):
    """Seeded random call shapes: ragged batches (empty sequences included),
    windows from 1 to wider than the sequence, both dtypes, d 64 and 128, and
    group sizes that give 16-, 32- and 128-row position spans per Q tile."""
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (16, 2), (32, 4), (8, 1), (4, 4)]
    out = []
    for i in range(n):
        h_q, h_kv = heads[rng.integers(len(heads))]
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["f16", "bf16"]))
        nb = int(rng.integers(1, 5))
        sq = [int(rng.choice([0, 1, 7, 16, 33, 64, 100, 129, 257])) for _ in range(nb)]
        if sum(sq) == 0:
            sq[0] = 45
        past = [int(rng.choice([0, 3, 31, 64, 200, 513, 1400])) for _ in range(nb)]
        window = int(rng.choice([-1, 1, 17, 64, 100, 128, 160, 1000]))
        out.append((f"rand{i}_{h_q}x{h_kv}_d{d}_{dtype}_w{window}", h_q, h_kv, d, sq, past, window,
                    dtype))
    return out


@pytest.mark.parametrize("spec", _random_cases(), ids=lambda s: s[0])
def test_random_shapes_every_config(spec):
    name, h_q, h_kv, d, sq, past, window, dtype = spec
    case = synth.Case(name, h_q=h_q, h_kv=h_kv, d=d, sq=sq, past=past, window=window, dtype=dtype,
                      seed=500 + sum(sq) + sum(past), s_cap=max(p + s for p, s in zip(past, sq)) + 9)
    _full_check(case, out_dtypes=("same",), every_config=True)


def _each_config():
    """Yield every kernel configuration, forced for the calls made meanwhile
    (bitwise properties hold within one configuration; the tuner may pick
    different ones for different call shapes)."""
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            yield cfg
    finally:
        binding.attn_force_config(-1)


def test_wide_window_equals_causal_bitwise():
    # hip-ep #622 "harness: window cases": a window wider than the sequence
    # must reproduce full attention exactly
    case = synth.Case("wide", h_q=8, h_kv=2, d=64, sq=[300], past=[200], window=-1, seed=5)
    dev = to_device(synth.make(case))
    for cfg in _each_config():
        dev["window"] = -1
        a, _, _, _ = run_gpu(dev)
        dev["window"] = 500
        b, _, _, _ = run_gpu(dev)
        dev["window"] = 10 ** 6
        c, _, _, _ = run_gpu(dev)
        assert torch.equal(a, b) and torch.equal(a, c), cfg


def test_sink_minus_inf_equals_no_sink_bitwise():
    case = synth.Case("sinkinf", h_q=8, h_kv=2, d=64, sq=[200], past=[100], window=64, seed=6)
    dev = to_device(synth.make(case))
    for cfg in _each_config():
        dev["sink"] = None
        a, _, _, _ = run_gpu(dev)
        dev["sink"] = torch.full((8,), float("-inf"), dtype=torch.float32, device="cuda")
        b, _, _, _ = run_gpu(dev)
        assert torch.equal(a, b), cfg


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_window_one_returns_own_value_row(dtype):
    # hip-ep #622 "harness: window cases": window 1 -> each query sees only itself
    case = synth.Case("w1", h_q=8, h_kv=2, d=64, sq=[150], past=[40], window=1, sink=False,
                      dtype=dtype, seed=8)
    inp = synth.make(case)
    out, _, _, _ = run_gpu(to_device(inp))
    v = inp["v_cache"][0]                    # [h_kv, cap, d]
    expect = v[:, 40:190].permute(1, 0, 2).repeat_interleave(4, dim=1)
    assert torch.equal(out.cpu(), expect)


def test_chunk_rows_match_whole_prefill_rows_bitwise():
    # chunk rows at past c0 equal rows [c0, c0 + sq) of one prefill over the
    # whole sequence; bitwise under one kernel configuration (KV tiles are
    # aligned to key 0 of the sequence and Q tiles to multiples of their rows)
    case = synth.Case("chunks", h_q=8, h_kv=2, d=64, sq=[640], past=[0], window=100, seed=9,
                      poison_tail=False)
    inp = synth.make(case)
    dev = to_device(inp)
    for cfg in _each_config():
        whole, _, _, _ = run_gpu(dev, out_dtype=torch.float32)
        for c0 in (0, 128, 384):
            part, _, _, _ = run_gpu(dev, out_dtype=torch.float32,
                                    q=dev["q"][c0:c0 + 128].contiguous(), cu=[0, 128], past=[c0])
            assert torch.equal(part, whole[c0:c0 + 128]), (cfg, c0)


@pytest.mark.parametrize("residues", [(2, 3, 6, 7), (2,), (7,), (0, 1, 4, 5)])
def test_scores_rising_far_past_the_reference(residues):
    # Online softmax with a lazily raised reference max (FlashAttention-2,
    # "Algorithm"; a stale max is exact after rescaling): a wave's first
    # tiles set the reference near 0, then keys whose key index mod 8 is in
    # `residues` score about 40 (log2 units) above it.  exp2 of that against
    # the old reference overflows fp16, so the kernels must see the rise
    # wherever the key sits in the tile and raise the reference before P is
    # used; the result must stay finite and match the oracle.
    case = synth.Case("rising", h_q=8, h_kv=2, d=64, sq=[128], past=[1024], window=-1,
                      seed=31, poison_tail=False)
    inp = synth.make(case)
    q, k = inp["q"].float(), inp["k_cache"].float()
    q = 1.0 + 0.05 * q                     # every row points along (1, ..., 1)
    k = 0.05 * k                           # scores near 0 ...
    keys = torch.arange(k.shape[2])
    big = (keys >= 384) & (keys < 640) & torch.isin(keys % 8, torch.tensor(residues))
    k[:, :, big, :] += 3.5                 # ... except these: q.k/8 * log2(e) ~ 40
    inp["q"], inp["k_cache"] = q.half(), k.half()
    ref = oracle_full(inp)
    dev = to_device(inp)
    for cfg in _each_config():
        name = f"rising{residues}[{binding.attn_config_name(cfg)}]"
        out, _, _, _ = run_gpu(dev, out_dtype=torch.float32)
        got = f64(out)
        assert np.all(np.isfinite(got)), f"{name}: non-finite output"
        check_rows(got, ref, name)


def test_declined_request_leaves_output_untouched():
    q = torch.randn(16, 4, 96, device="cuda", dtype=torch.float16)
    k = torch.randn(1, 2, 16, 96, device="cuda", dtype=torch.float16)
    out = torch.full_like(q, 3.0)
    code = binding.attn_prefill(q, k, k, 0, -1, None, 0.1, out, check=False)
    torch.cuda.synchronize()
    assert code == binding.ATTN_DECLINED
    assert torch.all(out == 3.0)


# ---------------------------------------------------------------------------
# Full-size workloads, at the shapes the benchmark times.  Whole outputs where
# the oracle finishes in seconds on the host's cores (the 4096-row prefill,
# the window chunks, the deepest chunk of each 16k layer type), sampled rows
# elsewhere; every check in both the input dtype (against the oracle rounded
# to it) and fp32, with the per-row bound beside the global one, and the
# visited-tile records of the call.
# ---------------------------------------------------------------------------
def _call(inp, case, out_dtype, q=None, cu=None, past=None):
    dev = to_device(inp)
    qd = None if q is None else q.cuda()
    rows = (q if q is not None else inp["q"]).shape[0]
    return run_gpu(dev, out_dtype=out_dtype, q=qd, cu=cu, past=past,
                   log_capacity=rows * case.h_q)


def _whole_check(case, inp=None, q=None, cu=None, past=None, tag=""):
    inp = inp or synth.make(case)
    cu = inp["cu_seqlens"] if cu is None else cu
    past = inp["past_len"] if past is None else past
    sink = None if inp["sink"] is None else f64(inp["sink"])
    ref = oracle.attn_prefill_varlen(f64(inp["q"] if q is None else q), f64(inp["k_cache"]),
                                     f64(inp["v_cache"]), cu, past, inp["window"], sink,
                                     inp["scale"])
    name = case.name + tag
    for tdt in (case.torch_dtype, torch.float32):
        out, recs, bkv, q_rows = _call(inp, case, tdt, q=q, cu=cu, past=past)
        got = f64(out)
        assert np.all(np.isfinite(got)), name
        expect = ref if tdt == torch.float32 else rne(ref, tdt)
        check_rows(got, expect, f"{name} whole out={tdt}", row_tol=row_tol_for(tdt))
        check_tile_log(recs, bkv, q_rows, cu, past, case.window, case.h_q)


def _sampled_check(case, n_rows=160, seed=0, q=None, cu=None, past=None, inp=None):
    inp = inp or synth.make(case)
    cu = inp["cu_seqlens"] if cu is None else cu
    past = inp["past_len"] if past is None else past
    tokens = cu[-1]
    rng = np.random.default_rng(seed)
    must = [0, tokens - 1] + [c for c in cu[1:-1]] + [max(c - 1, 0) for c in cu[1:-1]]
    toks, heads = sample_rows(rng, tokens, case.h_q, n_rows, must=must)
    ref = oracle_rows(inp, toks, heads, q=q, cu=cu, past=past)
    for tdt in (case.torch_dtype, torch.float32):
        out, recs, bkv, q_rows = _call(inp, case, tdt, q=q, cu=cu, past=past)
        assert torch.isfinite(out).all(), case.name
        got = f64(out)[toks, heads]
        expect = ref if tdt == torch.float32 else rne(ref, tdt)
        check_rows(got, expect, f"{case.name} {len(toks)} sampled rows out={tdt}",
                   row_tol=row_tol_for(tdt))
        check_tile_log(recs, bkv, q_rows, cu, past, case.window, case.h_q)


def test_full_attention_sq4096():
    _whole_check(synth.full_sq4096())


@pytest.mark.parametrize("past", [0, 512, 8192])
def test_sliding_window_chunk512(past):
    _whole_check(synth.swa_chunk(past))


def test_ragged_batch_bf16_d128():
    _sampled_check(synth.ragged_bf16(), n_rows=4096)


@pytest.mark.parametrize("layer", [0, 1])
def test_chunked_16k_layer_deepest_chunk(layer):
    # the last chunk (512 rows after 15872 cached keys), whole output
    case = synth.chunked16k_layer(layer)
    inp = synth.make(case)
    C = synth.CHUNKED16K_CHUNK
    c = synth.CHUNKED16K_TOKENS // C - 1
    q = inp["q"][c * C:(c + 1) * C].contiguous()
    _whole_check(case, inp=inp, q=q, cu=[0, C], past=[c * C], tag=f"_chunk{c}")


@pytest.mark.parametrize("layer", [0, 1])
def test_chunked_16k_layer_sampled_chunks(layer):
    case = synth.chunked16k_layer(layer)
    inp = synth.make(case)
    C = synth.CHUNKED16K_CHUNK
    for c in (0, 1, 15):
        q = inp["q"][c * C:(c + 1) * C].contiguous()
        _sampled_check(case, n_rows=256, seed=c, q=q, cu=[0, C], past=[c * C], inp=inp)


def test_first_call_sweep_with_poisoned_cache_tail():
    # The first call of a new tuning key times every configuration (on the
    # caller's cache, up to its capacity) before the real launch; positions
    # past the valid keys hold NaN here, and the call still returns the
    # oracle's result with nothing non-finite.
    binding.attn_tune_reset()
    case = synth.Case("sweep_poison", h_q=16, h_kv=2, d=64, sq=[384], past=[200], window=-1,
                      seed=91, s_cap=3000)
    inp = synth.make(case)
    assert torch.isnan(inp["k_cache"][0, :, 584:]).all()
    ref = oracle_full(inp)
    out, recs, bkv, q_rows = run_gpu(to_device(inp), out_dtype=torch.float32,
                                     log_capacity=case.tokens * case.h_q)
    assert binding.attn_tune_stats()["sweeps"] == 1
    assert torch.isfinite(out).all()
    check_rows(f64(out), ref, case.name)
    check_tile_log(recs, bkv, q_rows, case.cu_seqlens, case.past, case.window, case.h_q)


def _forced(name):
    """Force the configuration called `name` for the calls made meanwhile."""
    idx = [binding.attn_config_name(i) for i in range(binding.attn_config_count())].index(name)
    binding.attn_force_config(idx)


def test_streaming_window_full_size():
    # The streaming window configuration at the benchmark's window shapes: the
    # ragged bf16 d 128 batch (sampled rows, long runs of Q tiles per
    # workgroup over the block ring) and the 512-row window chunks at past 0
    # and 8192 (whole outputs); it runs these calls itself (bkv 32).
    try:
        _forced("swin_r128_kv32")
        _sampled_check(synth.ragged_bf16(), n_rows=4096, seed=3)
        for past in (0, 8192):
            _whole_check(synth.swa_chunk(past), tag=f"_swin_past{past}")
        inp = synth.make(synth.ragged_bf16())
        _, _, bkv, _ = _call(inp, synth.ragged_bf16(), torch.float32)
        assert bkv == 32
    finally:
        binding.attn_force_config(-1)


def test_streaming_config_falls_back_where_it_does_not_run():
    # Forced onto calls it does not run -- full attention, a window too wide
    # for its block ring, KV splits -- the streaming window configuration
    # gives way to the default one: the oracle's results, and the default's
    # 64-key tiles in the tile log.
    try:
        _forced("swin_r128_kv32")
        for window in (-1, 5000):
            case = synth.Case(f"fallback_w{window}", h_q=16, h_kv=2, d=64, sq=[200], past=[300],
                              window=window, seed=41)
            inp = synth.make(case)
            out, recs, bkv, q_rows = run_gpu(to_device(inp), out_dtype=torch.float32,
                                             log_capacity=case.tokens * case.h_q)
            check_rows(f64(out), oracle_full(inp), case.name)
            assert bkv == 64, case.name
            check_tile_log(recs, bkv, q_rows, case.cu_seqlens, case.past, case.window, case.h_q)
        case = synth.Case("fallback_split", h_q=16, h_kv=2, d=64, sq=[200], past=[300], window=128,
                          seed=42)
        inp = synth.make(case)
        dev = to_device(inp)
        out = torch.full(dev["q"].shape, float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(binding.attn_split_workspace_bytes(case.tokens, case.h_q, case.d, 2),
                         dtype=torch.uint8, device="cuda")
        log = new_log(2 * case.tokens * case.h_q, "cuda")
        _, n, bkv, q_rows = binding.attn_prefill_split(
            dev["q"], dev["k_cache"], dev["v_cache"], inp["cu_seqlens"], inp["past_len"],
            case.window, dev["sink"], inp["scale"], out, n_split=2, workspace=ws, tile_log=log)
        torch.cuda.synchronize()
        check_rows(f64(out), oracle_full(inp), case.name)
        assert bkv == 64 and n > 0
    finally:
        binding.attn_force_config(-1)


@pytest.mark.parametrize("dtype,window", [("f16", -1), ("bf16", 4096)])
def test_long_context_128k_keys(dtype, window):
    # A 256-row chunk after 130,816 cached keys (131,072 in all): thousands of
    # KV tiles per Q tile (the ping-pong kernel's steady loop, the lazy
    # rescale and fp32 accumulation over 128k keys), whole outputs against the
    # oracle and tile logs, on every configuration.
    case = synth.Case(f"ctx128k_{dtype}_w{window}", h_q=8, h_kv=1, d=64, sq=[256], past=[130816],
                      window=window, dtype=dtype, seed=51)
    _full_check(case, every_config=True)
