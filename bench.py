"""Benchmark: fused causal GQA flash-attention prefill on one MI355X.

Workload (one step): a 16k-token prefill of gpt-oss attention geometry run
as 32 chunks of 512 tokens over a growing KV cache (chunk c at past_len
512c), through 24 layers that alternate full attention and a 128-key
sliding window (12 of each), H_q = 64, H_kv = 8, d = 64, fp16, per-head
sinks.  Every layer owns its own q / cache / out buffers (so no layer finds
another's KV in cache), all resident in HBM before timing starts.  Calls run
chunk-major (chunk c through all 24 layers, then chunk c + 1), as a model's
chunked prefill does.

Reported: useful TFLOP/s over the whole step (useful = 4 * d * H_q per kept
(query, key) pair; masked work in visited tiles does not count) from the host
clock around K back-to-back steps; the full-attention layers' TFLOP/s and
fraction of the MI355X dense fp16/bf16 MFMA peak, and microseconds per layer
call, from passes that run one step's calls of one layer type alone (in step
order, back to back) between one HIP event pair on the launch stream; per-call
times from HIP events recorded around every launch in E further steps (each
pair adds about 2 us of queue work to its call); median / min / p90 of the
per-step times, of the passes, of the per-layer times (12 layers x E samples
per layer type) and of the first and last chunk's calls; the cold first call
of each layer type (its tuning sweep included).  Beside it: the CPU oracle's throughput on a bounded row sample of
the same workload, and one whole call of the oracle single-threaded.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--event-steps E]
       python bench.py --ab OTHER_BUILD.so   (interleaved A/B/A of two builds)
"""
import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS_F16 = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "prefill attention useful TFLOP/s & % bf16 MFMA peak; us/layer-call at 16k"

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "full_attention_16k_traffic.txt")
# the device code a recorded HBM-traffic figure belongs to (host-side changes
# such as the tuner's do not change a kernel's traffic)
KERNEL_SOURCES = [os.path.join(ROOT, "gqa_flash_attention_prefill_amd", "csrc", f)
                  for f in ("attn_kernel.hip", "attn_internal.h")]
COPY_BYTES = 1 << 30   # the calibration copy reads and writes 1 GiB

H_Q, H_KV, D, WINDOW = 64, 8, 64, 128
LAYERS, CHUNK, TOKENS = 24, 512, 16384
N_CHUNKS = TOKENS // CHUNK


def kept_pairs(past, sq, window):
    """Kept (query, key) pairs of one head for a chunk of sq rows after past keys."""
    pos = past + np.arange(sq, dtype=np.int64)
    lo = np.zeros_like(pos) if window <= 0 else np.maximum(0, pos - window + 1)
    return int((pos - lo + 1).sum())


def useful_flops(past, sq, window):
    return 4.0 * D * H_Q * kept_pairs(past, sq, window)


def algorithmic_bytes(past, sq, window, elem=2):
    """Q read + O write + K and V over the keys the chunk's rows keep (union)."""
    lo = 0 if window <= 0 else max(0, past - window + 1)
    keys = past + sq - lo
    return elem * (2 * sq * H_Q * D + 2 * keys * H_KV * D)


def layer_window(layer):
    return WINDOW if layer % 2 == 1 else -1


def make_layers(torch, dev):
    """Per-layer device buffers, drawn with the seeded generator recipe of
    gqa_flash_attention_prefill_amd.synth (N(0,1) in fp32 rounded to fp16)."""
    from gqa_flash_attention_prefill_amd import synth
    layers = []
    for layer in range(LAYERS):
        case = synth.chunked16k_layer(layer)
        inp = synth.make(case, device=dev)
        out = torch.empty_like(inp["q"])
        layers.append((case, inp, out))
    return layers


def cpu_baseline(torch, layers_cpu, budget_s=12.0):
    """Time the oracle (as it stands) on a row sample of the workload: rows
    drawn uniformly over the 16k positions and all 64 heads of one full and
    one window layer (a chunk row equals the same row of one whole-sequence
    prefill, so the oracle runs on the whole-sequence view).  The sample size
    is calibrated to about `budget_s` seconds of oracle time."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        threads = min(threads, int(os.environ["OMP_NUM_THREADS"]))
    rng = np.random.default_rng(1234)
    prepared = []
    for case, inp in layers_cpu:
        prepared.append((case, {
            "q": inp["q"].double().numpy(), "k": inp["k_cache"].double().numpy(),
            "v": inp["v_cache"].double().numpy(), "sink": inp["sink"].double().numpy()}))

    def run(n_rows):
        flops, secs = 0.0, 0.0
        for case, a in prepared:
            toks = rng.integers(0, TOKENS, size=n_rows)
            heads = rng.integers(0, H_Q, size=n_rows).astype(np.int32)
            lo = np.zeros_like(toks) if case.window <= 0 else np.maximum(0, toks - case.window + 1)
            flops += 4.0 * D * float((toks - lo + 1).sum())
            t0 = time.perf_counter()
            oracle.attn_rows(a["q"], a["k"], a["v"], [0, TOKENS], [0], case.window, a["sink"],
                             case.scale, toks, heads, threads=threads)
            secs += time.perf_counter() - t0
        return flops, secs

    f, s = run(64)
    n = int(np.clip(64 * budget_s / max(s, 1e-3), 64, 200000))
    f, s = run(n)

    # one whole call of the workload, single-threaded: chunk 0 of a window
    # layer (512 rows, no prefix, window 128)
    case, a = prepared[1]
    t0 = time.perf_counter()
    oracle.attn_prefill_varlen(a["q"][:CHUNK], a["k"], a["v"], [0, CHUNK], [0], case.window,
                               a["sink"], case.scale, threads=1)
    one_ms = (time.perf_counter() - t0) * 1e3
    return {"value": f / s / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} rows x 2 layers (1 full, 1 window-128) drawn uniformly over the "
                      f"16k positions and 64 heads, fp64 oracle, {s:.1f} s",
            "seconds": round(s, 2), "cpu_model": cpu_model(),
            "single_thread_call": {"call": "window-128 layer, chunk 0 (512 rows, past 0)",
                                   "threads": 1, "ms": round(one_ms, 1)}}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def dist(xs, nd=3):
    """median / min / p90 / mean of a sample (and its size)."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), nd), "min": round(float(a.min()), nd),
            "p90": round(float(np.percentile(a, 90)), nd), "mean": round(float(a.mean()), nd),
            "n": int(a.size)}


def _load_lib(path):
    """A library build's attn_prefill / attn_prefill_varlen through ctypes
    (for A/B timing)."""
    L = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    i32p = ctypes.POINTER(ctypes.c_int32)
    L.attn_prefill.argtypes = [vp, vp, vp, i32, i32, vp, ctypes.c_float, vp, i32, i32, i32, i32,
                               i32, i32, i32, vp]
    L.attn_prefill.restype = ctypes.c_int
    L.attn_prefill_varlen.argtypes = [vp, vp, vp, i32p, i32p, i32, i32, vp, ctypes.c_float, vp,
                                      i32, i32, i32, i32, i32, i32, vp, vp]
    L.attn_prefill_varlen.restype = ctypes.c_int
    return L


def ragged_calls(torch, binding, reps=8):
    """`reps` calls of the ragged bf16 d 128 batch (8 sequences, 16 q / 2 KV
    heads, window 128, bf16 out) as attn_prefill_varlen argument tuples."""
    from gqa_flash_attention_prefill_amd import synth
    rc = synth.ragged_bf16()
    rc = synth.Case(rc.name, h_q=rc.h_q, h_kv=rc.h_kv, d=rc.d, sq=list(rc.sq), past=list(rc.past),
                    window=rc.window, dtype=rc.dtype, seed=rc.seed, poison_tail=False)
    inp = synth.make(rc, device="cuda:0")
    out = torch.empty_like(inp["q"])
    batch, h_kv, s_cap, d = inp["k_cache"].shape
    cu, past = inp["cu_seqlens"], inp["past_len"]
    keep = (inp, out)
    a = (ctypes.c_void_p(inp["q"].data_ptr()), ctypes.c_void_p(inp["k_cache"].data_ptr()),
         ctypes.c_void_p(inp["v_cache"].data_ptr()), (ctypes.c_int32 * len(cu))(*cu),
         (ctypes.c_int32 * len(past))(*past), len(past), rc.window,
         ctypes.c_void_p(inp["sink"].data_ptr()), ctypes.c_float(rc.scale),
         ctypes.c_void_p(out.data_ptr()), rc.h_q, h_kv, d, s_cap, binding.ATTN_BF16,
         binding.ATTN_BF16, None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return [("attn_prefill_varlen", keep, a)] * reps


def ab_compare(torch, binding, lib_b, rounds, layers_calls):
    """Interleaved A/B of two builds of the library on the whole 16k step:
    per round A, B, then A again (the same-variant control), each one step of
    768 calls between an event pair on the launch stream.  A is the in-tree
    build, B the given one (both tune their own configurations first)."""
    A, B = binding.lib(), _load_lib(lib_b)
    stream = torch.cuda.current_stream()

    def step(L):
        for fn, _, a in layers_calls:
            f = getattr(L, fn) if isinstance(fn, str) else L.attn_prefill
            if f(*a) != 0:
                raise RuntimeError("attention call failed in the A/B run")

    for L in (A, B):
        step(L)
        step(L)
    torch.cuda.synchronize()
    res = {"a": [], "b": [], "a_control": []}
    for _ in range(rounds):
        for key, L in (("a", A), ("b", B), ("a_control", A)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step(L)
            e1.record(stream)
            torch.cuda.synchronize()
            res[key].append(e0.elapsed_time(e1))
    a, b, c = (np.array(res[k]) for k in ("a", "b", "a_control"))
    return {"mode": "interleaved A/B/A (A = in-tree build, B = " + os.path.basename(lib_b) + ")",
            "rounds": rounds, "ms_per_step": {"a": dist(a), "b": dist(b), "a_control": dist(c)},
            "b_over_a_median": round(float(np.median(b / a)), 4),
            "control_over_a_median": round(float(np.median(c / a)), 4)}


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def recorded_traffic():
    """HBM bytes per full-attention launch from the committed counter summary,
    or None if it is missing or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibration(torch):
    """A plain device copy of known size, read cold: 1 GiB is written, a
    second 1 GiB buffer is written to push it out of the caches, then the
    first is copied (1 GiB read + 1 GiB written).  Its FETCH_SIZE /
    WRITE_SIZE readings scale the attention kernel's counters to bytes."""
    x = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    evict = torch.full((COPY_BYTES // 4,), 2.0, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    y.copy_(x)
    torch.cuda.synchronize()
    del x, y, evict


def _classify(name):
    if "attn_swin_kernel" in name:   # window calls only
        return "attn_window"
    if "attn_fwd_kernel" in name or "attn_pp_kernel" in name:
        return "attn_window" if ", true," in name else "attn_full"
    if "copy" in name.lower() or "elementwise" in name.lower():
        return "copy"
    return None


def summarize_trace(path):
    """Average kernel durations from a rocprofv3 --kernel-trace --stats CSV:
    for each call kind, the instantiation with the most calls (the tuned one;
    the others ran only in the tuning sweep)."""
    out = {}
    for r in csv.DictReader(open(path)):
        kind = _classify(r["Name"])
        if kind not in ("attn_full", "attn_window"):
            continue
        cur = {"calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
               "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
               "kernel": r["Name"]}
        if kind not in out or cur["calls"] > out[kind]["calls"]:
            out[kind] = cur
    return out


def summarize_counters(fetch_dir, write_dir):
    """Per-launch FETCH_SIZE / WRITE_SIZE (KiB) of the full-attention calls and
    of the calibration copy, and the copy-derived scale factors."""
    def collect(d, counter):
        per = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                kind = _classify(r["Kernel_Name"])
                if kind is None:
                    continue
                key = (kind, r["Kernel_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        # per kind, keep the instantiation with the most dispatches (the tuned one)
        by_name = {}
        for (kind, name, _), v in per.items():
            by_name.setdefault((kind, name), []).append(v)
        agg = {}
        for (kind, name), vals in by_name.items():
            if kind == "copy":   # the calibration copy is the largest copy dispatch
                agg["copy"] = [max(agg.get("copy", [0.0]) + vals)]
            elif kind not in agg or len(vals) > len(agg[kind]):
                agg[kind] = vals
        return agg
    fetch, write = collect(fetch_dir, "FETCH_SIZE"), collect(write_dir, "WRITE_SIZE")
    copy_f = max(fetch.get("copy", [0.0]))   # the 1 GiB copy is the largest copy dispatch
    copy_w = max(write.get("copy", [0.0]))
    kib = COPY_BYTES / 1024.0
    f_scale = kib / copy_f if copy_f else None
    w_scale = kib / copy_w if copy_w else None
    fa = fetch.get("attn_full", [])
    wa = write.get("attn_full", [])
    res = {"copy_fetch_kib": copy_f, "copy_write_kib": copy_w, "fetch_scale": f_scale,
           "write_scale": w_scale,
           "attn_full_launches": len(fa),
           "attn_full_fetch_kib_raw": sum(fa) / len(fa) if fa else None,
           "attn_full_write_kib_raw": sum(wa) / len(wa) if wa else None}
    if fa and wa and f_scale and w_scale:
        res["fetch_bytes_per_launch"] = res["attn_full_fetch_kib_raw"] * f_scale * 1024
        res["write_bytes_per_launch"] = res["attn_full_write_kib_raw"] * w_scale * 1024
    return res


def summarize_pmc(d):
    """Mean over dispatches of each counter (summed over its instances) for the
    attention kernels of a rocprofv3 --pmc run."""
    per = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if _classify(r["Kernel_Name"]) not in ("attn_full", "attn_window"):
                continue
            key = (r["Kernel_Name"], r["Dispatch_Id"], r["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    out = {}
    for (name, _, counter), v in per.items():
        out.setdefault(name, {}).setdefault(counter, []).append(v)
    return {name: {c: {"mean": sum(v) / len(v), "dispatches": len(v)} for c, v in cs.items()}
            for name, cs in out.items()}


def one_call(torch, binding, chunk):
    """Three untimed launches of one full-attention call shape (chunk `chunk`
    of the 16k prefill: 512 rows after 512 * chunk cached keys) on layer 0's
    buffers, for hardware-counter passes on that shape alone."""
    from gqa_flash_attention_prefill_amd import synth
    torch.cuda.set_device(0)
    case = synth.chunked16k_layer(0)
    inp = synth.make(case, device="cuda:0")
    out = torch.empty_like(inp["q"])
    q = inp["q"][chunk * CHUNK:(chunk + 1) * CHUNK]
    o = out[chunk * CHUNK:(chunk + 1) * CHUNK]
    for _ in range(3):
        binding.attn_prefill(q, inp["k_cache"], inp["v_cache"], chunk * CHUNK, case.window,
                             inp["sink"], case.scale, o)
    torch.cuda.synchronize()
    print(f"[bench] one_call chunk {chunk}: 3 launches of the full-attention call", flush=True)


CANDIDATE_LAUNCHES = 3


def candidate_calls(torch, binding):
    """The call shapes of the per-configuration counter table: the deepest
    full-attention chunk of the 16k prefill (512 rows after 15872 keys), a
    window-128 chunk at mid depth (512 rows after 8192 keys), both fp16 with
    sinks, and the ragged bf16 d 128 batch of 8 sequences (window 128, bf16
    out).  Returns [(label, callable)]."""
    from gqa_flash_attention_prefill_amd import synth
    out = []
    for layer, chunk, label in ((0, N_CHUNKS - 1, "full_chunk31"), (1, 16, "window128_chunk16")):
        case = synth.chunked16k_layer(layer)
        inp = synth.make(case, device="cuda:0")
        o = torch.empty_like(inp["q"])
        q = inp["q"][chunk * CHUNK:(chunk + 1) * CHUNK]
        oc = o[chunk * CHUNK:(chunk + 1) * CHUNK]

        def call(inp=inp, q=q, oc=oc, chunk=chunk, case=case):
            binding.attn_prefill(q, inp["k_cache"], inp["v_cache"], chunk * CHUNK, case.window,
                                 inp["sink"], case.scale, oc)
        out.append((label, call))
    rc = synth.ragged_bf16()
    rc = synth.Case(rc.name, h_q=rc.h_q, h_kv=rc.h_kv, d=rc.d, sq=list(rc.sq), past=list(rc.past),
                    window=rc.window, dtype=rc.dtype, seed=rc.seed, poison_tail=False)
    rinp = synth.make(rc, device="cuda:0")
    rout = torch.empty_like(rinp["q"])

    def ragged():
        binding.attn_prefill_varlen(rinp["q"], rinp["k_cache"], rinp["v_cache"],
                                    rinp["cu_seqlens"], rinp["past_len"], rinp["window"],
                                    rinp["sink"], rc.scale, rout)
    out.append(("ragged8_bf16_d128", ragged))
    return out


def run_candidates(torch, binding):
    """Every kernel configuration, forced, on each candidate call shape:
    CANDIDATE_LAUNCHES launches per (configuration, call), in a fixed order
    (configurations outer), then the 1 GiB calibration copy.  Under a
    profiler the attention dispatches come in groups of CANDIDATE_LAUNCHES in
    the printed order."""
    torch.cuda.set_device(0)
    calls = candidate_calls(torch, binding)
    order = []
    try:
        for cfg in range(binding.attn_config_count()):
            binding.attn_force_config(cfg)
            for label, fn in calls:
                for _ in range(CANDIDATE_LAUNCHES):
                    fn()
                torch.cuda.synchronize()
                order.append([binding.attn_config_name(cfg), label])
    finally:
        binding.attn_force_config(-1)
    copy_calibration(torch)
    print(json.dumps({"candidate_order": order, "launches": CANDIDATE_LAUNCHES}), flush=True)


def summarize_candidates(order_file, trace_csv, pmc_dirs):
    """Per (configuration, call): mean kernel duration over the launches after
    the first (kernel trace) and the mean of every counter of the PMC passes
    over the same dispatches; HBM bytes from FETCH_SIZE / WRITE_SIZE scaled by
    the calibration copy's readings of the same counters."""
    order = None
    for line in open(order_file):
        line = line.strip()
        if line.startswith("{") and "candidate_order" in line:
            order = json.loads(line)
    assert order is not None, "no candidate_order line"
    n = order["launches"]
    groups = order["candidate_order"]

    def attn_rows(rows, key_name, key_id):
        att = [r for r in rows if _classify(r[key_name]) in ("attn_full", "attn_window")]
        ids = sorted({int(r[key_id]) for r in att})
        return att, ids

    trace = list(csv.DictReader(open(trace_csv)))
    att, ids = attn_rows(trace, "Kernel_Name", "Dispatch_Id")
    assert len(ids) == n * len(groups), (len(ids), n, len(groups))
    dur = {int(r["Dispatch_Id"]): (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
           for r in att}
    names = {int(r["Dispatch_Id"]): r["Kernel_Name"] for r in att}
    table = []
    for gi, (cfg, label) in enumerate(groups):
        gid = ids[gi * n:(gi + 1) * n][1:]
        table.append({"config": cfg, "call": label,
                      "kernel": names[gid[0]].split("(")[0].replace(
                          "attn::(anonymous namespace)::", ""),
                      "us": round(float(np.mean([dur[i] for i in gid])), 2), "counters": {}})
    copy_vals = {}
    for d in pmc_dirs:
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(f)))
        per = {}
        copies = {}
        for r in rows:
            key = (int(r["Dispatch_Id"]), r["Counter_Name"])
            if _classify(r["Kernel_Name"]) == "copy":
                copies[key] = copies.get(key, 0.0) + float(r["Counter_Value"])
            elif _classify(r["Kernel_Name"]) in ("attn_full", "attn_window"):
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        pids = sorted({k[0] for k in per})
        assert len(pids) == n * len(groups), (d, len(pids))
        counters = sorted({k[1] for k in per})
        for (cid, cname), v in copies.items():
            copy_vals[cname] = max(copy_vals.get(cname, 0.0), v)
        for gi in range(len(groups)):
            gid = pids[gi * n:(gi + 1) * n][1:]
            for cname in counters:
                table[gi]["counters"][cname] = float(np.mean([per[(i, cname)] for i in gid]))
    kib = COPY_BYTES / 1024.0
    for row in table:
        c = row["counters"]
        if "FETCH_SIZE" in c and copy_vals.get("FETCH_SIZE"):
            row["hbm_read_mb"] = round(c["FETCH_SIZE"] * kib / copy_vals["FETCH_SIZE"] * 1024 / 1e6, 2)
        if "WRITE_SIZE" in c and copy_vals.get("WRITE_SIZE"):
            row["hbm_write_mb"] = round(c["WRITE_SIZE"] * kib / copy_vals["WRITE_SIZE"] * 1024 / 1e6, 2)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and "GRBM_GUI_ACTIVE" in c:
            # 256 CUs x 4 SIMDs over the XCDs' active cycles (8 XCDs)
            row["mfma_busy"] = round(c["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                     (1024 * c["GRBM_GUI_ACTIVE"] / 8), 4)
            row["clock_ghz"] = round(c["GRBM_GUI_ACTIVE"] / 8 / (row["us"] * 1e3), 3)
        if "SQ_INSTS_VALU" in c and c.get("SQ_INSTS_MFMA"):
            row["valu_per_mfma"] = round(c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"], 2)
        if "TCC_HIT" in c and "TCC_MISS" in c:
            row["l2_hit"] = round(c["TCC_HIT"] / max(1.0, c["TCC_HIT"] + c["TCC_MISS"]), 4)
    return {"copy_calibration": copy_vals, "rows": table}


def _time_calls(torch, binding, args, reps=20):
    """Mean us per call of `reps` back-to-back attn_prefill_split calls with
    pre-marshalled arguments, between one event pair on the launch stream
    (per-call events would add their own queue work to calls this short)."""
    L = binding.lib()
    for _ in range(3):
        rc = L.attn_prefill_split(*args)
        if rc != 0:
            raise RuntimeError(binding.attn_last_error())
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        L.attn_prefill_split(*args)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / reps


def _split_args(torch, binding, inp, case, cu, past, window, out, n_split, ws):
    import ctypes
    cu_a = (ctypes.c_int32 * len(cu))(*cu)
    past_a = (ctypes.c_int32 * len(past))(*past)
    code = {torch.float16: binding.ATTN_F16, torch.bfloat16: binding.ATTN_BF16}
    batch, h_kv, s_cap, d = inp["k_cache"].shape
    return (ctypes.c_void_p(inp["q"].data_ptr()), ctypes.c_void_p(inp["k_cache"].data_ptr()),
            ctypes.c_void_p(inp["v_cache"].data_ptr()), cu_a, past_a, len(past), window,
            ctypes.c_void_p(inp["sink"].data_ptr()), ctypes.c_float(case.scale),
            ctypes.c_void_p(out.data_ptr()), None, inp["q"].shape[1], h_kv, d, s_cap,
            code[inp["q"].dtype], code[out.dtype], n_split, 0, ctypes.c_void_p(ws.data_ptr()),
            ws.numel(), None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def split_demo(torch, binding):
    """KV splits across workgroups on calls with few Q tiles: one 512-row chunk
    after a 15872-key prefix at a tensor-parallel rank's heads (16 q / 2 KV,
    full attention, sinks), d 64 fp16 and d 128 bf16.  Without splits such a
    call has 64 Q-tile workgroups for 256 CUs.  Mean of 20 back-to-back calls
    per point (see _time_calls); the tuning sweep runs before timing."""
    import numpy as np
    from gqa_flash_attention_prefill_amd import synth
    res = []
    for d, dtype in ((64, "f16"), (128, "bf16")):
        case = synth.Case(f"tp4_d{d}", h_q=16, h_kv=2, d=d, sq=[512], past=[15872], window=-1,
                          dtype=dtype, seed=77, poison_tail=False)
        inp = synth.make(case, device="cuda")
        out = torch.empty_like(inp["q"])
        fl = useful_flops(15872, 512, -1) * 16 / H_Q * d / D
        row = {"d": d, "dtype": dtype}
        for n in (1, 2, 4, 8):
            nbytes = binding.attn_split_workspace_bytes(512, 16, d, n)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
            args = _split_args(torch, binding, inp, case, [0, 512], [15872], -1, out, n, ws)
            us = _time_calls(torch, binding, args)
            row[f"n_split_{n}"] = {"us": round(us, 2), "tflops": round(fl / us / 1e6, 1)}
        res.append(row)
    return {"workload": "one 512-row chunk, 15872-key prefix, 16 q / 2 KV heads (TP4 rank), "
                        "full attention, sinks", "results": res}


def decode_demo(torch, binding):
    """One decode step (one query row per sequence) of a 64-sequence batch,
    every sequence after a 16383-key prefix, H_q 64 / H_kv 8, d 64, fp16,
    sinks: window 128 and full attention (also with KV splits).  HBM-bound:
    GB/s of algorithmic bytes (q + out + each sequence's kept K/V keys once)
    against 8 TB/s.  Mean of 20 back-to-back calls (see _time_calls)."""
    import numpy as np
    from gqa_flash_attention_prefill_amd import synth
    B, past = 64, 16383
    case = synth.Case("decode64", h_q=H_Q, h_kv=H_KV, d=D, sq=[1] * B, past=[past] * B,
                      window=-1, seed=78, poison_tail=False)
    inp = synth.make(case, device="cuda")
    out = torch.empty_like(inp["q"])
    cu = list(range(B + 1))
    res = {}
    for label, window, n_split in (("window128", WINDOW, 1), ("full", -1, 1),
                                   ("full_split2", -1, 2), ("full_split4", -1, 4)):
        nbytes = binding.attn_split_workspace_bytes(B, H_Q, D, n_split)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        keys = past + 1 if window <= 0 else min(window, past + 1)
        algo = 2 * (2 * B * H_Q * D + 2 * B * keys * H_KV * D)
        args = _split_args(torch, binding, inp, case, cu, [past] * B, window, out, n_split, ws)
        us = _time_calls(torch, binding, args)
        res[label] = {"us": round(us, 2), "hbm_gbs": round(algo / us / 1e3, 1),
                      "frac_of_8tbs": round(algo / us / 1e3 / 8000.0, 4)}
    return {"workload": "decode step: 64 sequences x 1 row after 16383 cached keys, H_q 64 / "
                        "H_kv 8, d 64, fp16, sinks", "results": res}


def paged_demo(torch, binding):
    """The token-pool layout against dense caches on the same keys: every
    key row moved to a random row of a pool [n_pool, H_kv, d] (no two
    consecutive keys adjacent), addressed through kv_indices.  Two calls:
    the deepest full-attention chunk of the 16k prefill (512 rows after 15872
    keys) and a 64-sequence decode step (one row after 16383 keys each),
    H_q 64 / H_kv 8, d 64, fp16, sinks.  Mean of 20 back-to-back calls each;
    the dense split entry with an lse output runs the same kernel variant as
    the pool call, the plain dense call the variant without the options."""
    from gqa_flash_attention_prefill_amd import synth
    L = binding.lib()
    res = []
    for label, nseq, past, sq in (("chunk31_full", 1, 15872, 512), ("decode64_full", 64, 16383, 1)):
        case = synth.Case(label, h_q=H_Q, h_kv=H_KV, d=D, sq=[sq] * nseq, past=[past] * nseq,
                          window=-1, seed=79, poison_tail=False)
        inp = synth.make(case, device="cuda")
        tokens = sq * nseq
        skv = past + sq
        out = torch.empty_like(inp["q"])
        lse = torch.empty((tokens, H_Q), dtype=torch.float32, device="cuda")
        g = torch.Generator(device="cpu").manual_seed(80)
        n_pool = nseq * skv
        rows = torch.randperm(n_pool, generator=g).to(torch.int32)
        k_pool = torch.empty((n_pool, H_KV, D), dtype=torch.float16, device="cuda")
        v_pool = torch.empty_like(k_pool)
        rows_d = rows.to("cuda")
        for b in range(nseq):
            r = rows_d[b * skv:(b + 1) * skv].long()
            k_pool[r] = inp["k_cache"][b, :, :skv, :].transpose(0, 1)
            v_pool[r] = inp["v_cache"][b, :, :skv, :].transpose(0, 1)
        cu = (ctypes.c_int32 * (nseq + 1))(*[sq * i for i in range(nseq + 1)])
        pl = (ctypes.c_int32 * nseq)(*([past] * nseq))
        ip = (ctypes.c_int32 * (nseq + 1))(*[skv * i for i in range(nseq + 1)])
        st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        f16 = binding.ATTN_F16
        s_cap = inp["k_cache"].shape[2]
        vp = lambda t: ctypes.c_void_p(t.data_ptr())
        dense = (vp(inp["q"]), vp(inp["k_cache"]), vp(inp["v_cache"]), cu, pl, nseq, -1,
                 vp(inp["sink"]), ctypes.c_float(case.scale), vp(out), H_Q, H_KV, D, s_cap, f16,
                 f16, None, st)
        dense_lse = (vp(inp["q"]), vp(inp["k_cache"]), vp(inp["v_cache"]), cu, pl, nseq, -1,
                     vp(inp["sink"]), ctypes.c_float(case.scale), vp(out), vp(lse), H_Q, H_KV, D,
                     s_cap, f16, f16, 1, 0, None, 0, None, st)
        pool = (vp(inp["q"]), vp(k_pool), vp(v_pool), n_pool, vp(rows_d), ip, cu, pl, nseq, -1,
                vp(inp["sink"]), ctypes.c_float(case.scale), vp(out), vp(lse), H_Q, H_KV, D, f16,
                f16, 0, None, st)
        row = {"call": label}
        for name, fn, a in (("dense", L.attn_prefill_varlen, dense),
                            ("dense_lse", L.attn_prefill_split, dense_lse),
                            ("pool_lse", L.attn_prefill_paged, pool)):
            for _ in range(3):
                if fn(*a) != 0:
                    raise RuntimeError(binding.attn_last_error())
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                fn(*a)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / 20
            fl = 4.0 * D * H_Q * nseq * sum(past + i + 1 for i in range(sq))
            row[name] = {"us": round(us, 2), "tflops": round(fl / us / 1e6, 1)}
        res.append(row)
    return {"workload": "token pool (keys scattered to random pool rows) vs dense caches, "
                        "H_q 64 / H_kv 8, d 64, fp16, sinks, full attention", "results": res}


def configs_demo(torch, binding):
    """The other workloads of this path, each timed as one call (the tuning
    sweep first, then the mean of 50 back-to-back calls between one event
    pair): the tiny case, a gpt-oss-20b full-attention layer (4096 rows, no
    prefix), the window-128 chunk of 512 rows at past 0 / 512 / 8192 (full
    prefix in the cache), and the ragged bf16 d 128 batch of 8 sequences with
    fp32 and bf16 outputs.  Useful TFLOP/s counts kept pairs only; GB/s is
    algorithmic bytes (q + out + each sequence's kept-key union of K and V,
    read once) per call time."""
    from gqa_flash_attention_prefill_amd import synth
    L = binding.lib()
    cases = [(synth.tiny(), None), (synth.full_sq4096(), None), (synth.swa_chunk(0), None),
             (synth.swa_chunk(512), None), (synth.swa_chunk(8192), None),
             (synth.ragged_bf16(), torch.float32), (synth.ragged_bf16(), None)]
    res = []
    for case, out_dtype in cases:
        c2 = synth.Case(case.name, h_q=case.h_q, h_kv=case.h_kv, d=case.d, sq=list(case.sq),
                        past=list(case.past), window=case.window, dtype=case.dtype,
                        seed=case.seed, poison_tail=False)
        inp = synth.make(c2, device="cuda")
        q = inp["q"]
        out = torch.empty(q.shape, dtype=out_dtype or q.dtype, device="cuda")
        cu, past, w = inp["cu_seqlens"], inp["past_len"], inp["window"]
        batch, h_kv, s_cap, d = inp["k_cache"].shape
        code = {torch.float16: binding.ATTN_F16, torch.bfloat16: binding.ATTN_BF16,
                torch.float32: binding.ATTN_F32}
        args = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(inp["k_cache"].data_ptr()),
                ctypes.c_void_p(inp["v_cache"].data_ptr()),
                (ctypes.c_int32 * len(cu))(*cu), (ctypes.c_int32 * len(past))(*past), len(past),
                w, ctypes.c_void_p(inp["sink"].data_ptr()), ctypes.c_float(c2.scale),
                ctypes.c_void_p(out.data_ptr()), c2.h_q, h_kv, d, s_cap, code[q.dtype],
                code[out.dtype], None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        for _ in range(3):
            if L.attn_prefill_varlen(*args) != 0:
                raise RuntimeError(binding.attn_last_error())
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            L.attn_prefill_varlen(*args)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 50
        pairs, keys = 0, 0
        for b in range(len(past)):
            sq = cu[b + 1] - cu[b]
            pos = past[b] + np.arange(sq, dtype=np.int64)
            lo = np.zeros_like(pos) if w <= 0 else np.maximum(0, pos - w + 1)
            pairs += int((pos - lo + 1).sum())
            keys += past[b] + sq - (0 if w <= 0 else max(0, past[b] - w + 1))
        fl = 4.0 * d * c2.h_q * pairs
        tokens = cu[-1]
        nbytes = (tokens * c2.h_q * d * (q.element_size() + out.element_size())
                  + 2 * keys * h_kv * d * q.element_size())
        idx = binding.attn_tuned_config(d, q.dtype, out.dtype, tokens, c2.h_q, h_kv, w, len(past))
        res.append({"workload": case.name + ("" if out_dtype is None else "_fp32out"),
                    "us": round(us, 2), "useful_tflops": round(fl / us / 1e6, 2),
                    "frac_peak": round(fl / us / 1e6 / PEAK_TFLOPS_F16, 4),
                    "algorithmic_gbs": round(nbytes / us / 1e3, 1),
                    "frac_hbm": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                    "config": binding.attn_config_name(idx) if idx >= 0 else None})
    return {"workload": "the other workloads of this path, one call each", "results": res}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--event-steps", type=int, default=5,
                    help="steps after the timed ones with an event pair around every call "
                         "(per-call distributions)")
    ap.add_argument("--ab", default=None, metavar="LIB_B",
                    help="interleaved A/B/A timing of the in-tree library against another build")
    ap.add_argument("--ab-rounds", type=int, default=10)
    ap.add_argument("--ab-kind", choices=("all", "full", "window", "ragged"), default="all",
                    help="A/B over every call of the step, only one layer type's calls, or "
                         "8 calls of the ragged bf16 d 128 batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-demo", action="store_true",
                    help="time a 64-sequence decode step (prints its own JSON line)")
    ap.add_argument("--split-demo", action="store_true",
                    help="time KV splits on a few-Q-tile call (prints its own JSON line)")
    ap.add_argument("--paged-demo", action="store_true",
                    help="time the token-pool layout against dense caches (prints its own JSON line)")
    ap.add_argument("--configs-demo", action="store_true",
                    help="time the tiny, 4096-row, window-chunk and ragged bf16 workloads "
                         "(prints its own JSON line)")
    ap.add_argument("--detail", default=None, help="write per-chunk timings (JSON) here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run the 1 GiB cold copy used to scale HBM counters")
    ap.add_argument("--summarize-trace", default=None, metavar="KERNEL_STATS_CSV")
    ap.add_argument("--summarize-counters", nargs=2, default=None,
                    metavar=("FETCH_SIZE_DIR", "WRITE_SIZE_DIR"))
    ap.add_argument("--one-call", type=int, default=None, metavar="CHUNK",
                    help="only run the full-attention call of chunk CHUNK (3 times, untimed), "
                         "for hardware-counter passes on one launch shape")
    ap.add_argument("--candidates", action="store_true",
                    help="every configuration, forced, on the counter-table call shapes "
                         "(for rocprofv3 passes; prints the dispatch order)")
    ap.add_argument("--summarize-candidates", nargs="+", default=None,
                    metavar="ARG", help="ORDER_LOG KERNEL_TRACE_CSV PMC_DIR... -> the "
                                        "per-configuration table (JSON)")
    ap.add_argument("--summarize-pmc", default=None, metavar="PMC_DIR",
                    help="per-dispatch averages of every counter of the attention kernels")
    args = ap.parse_args()
    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return
    if args.summarize_candidates:
        a = args.summarize_candidates
        print(json.dumps(summarize_candidates(a[0], a[1], a[2:]), indent=1))
        return
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(args.summarize_pmc), indent=1))
        return
    if args.summarize_counters:
        res = summarize_counters(*args.summarize_counters)
        res["kernel_source_sha256"] = kernel_source_hash()
        print(json.dumps(res, indent=1))
        return
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only; a multi-GPU figure is not produced "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from gqa_flash_attention_prefill_amd import binding
    L = binding.lib()
    if args.one_call is not None:
        one_call(torch, binding, args.one_call)
        return
    if args.candidates:
        run_candidates(torch, binding)
        return
    if args.split_demo or args.decode_demo or args.paged_demo or args.configs_demo:
        torch.cuda.set_device(0)
        demo = (split_demo if args.split_demo else decode_demo if args.decode_demo
                else paged_demo if args.paged_demo else configs_demo)
        print(json.dumps(demo(torch, binding)), flush=True)
        return
    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    layers = make_layers(torch, dev)
    torch.cuda.synchronize()

    # marshal every call's arguments once (pointers + sizes), C ABI calls below
    calls = []  # (layer, chunk, args)
    for c in range(N_CHUNKS):
        for layer, (case, inp, out) in enumerate(layers):
            q = inp["q"][c * CHUNK:(c + 1) * CHUNK]
            o = out[c * CHUNK:(c + 1) * CHUNK]
            cargs = (ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(inp["k_cache"].data_ptr()),
                    ctypes.c_void_p(inp["v_cache"].data_ptr()), c * CHUNK, case.window,
                    ctypes.c_void_p(inp["sink"].data_ptr()), ctypes.c_float(case.scale),
                    ctypes.c_void_p(o.data_ptr()), CHUNK, H_Q, H_KV, D, TOKENS,
                    binding.ATTN_F16, binding.ATTN_F16, sptr)
            calls.append((layer, c, cargs))
    flops = {(layer, c): useful_flops(c * CHUNK, CHUNK, layer_window(layer))
             for layer in range(LAYERS) for c in range(N_CHUNKS)}
    step_flops = sum(flops.values())

    def one_step(events=None):
        for i, (layer, c, a) in enumerate(calls):
            if events is not None:
                events[i][0].record(stream)
            rc = L.attn_prefill(*a)
            if rc != 0:
                raise RuntimeError(f"attn_prefill failed: {binding.attn_last_error()} ({rc})")
            if events is not None:
                events[i][1].record(stream)

    # the first call of each layer type, cold: its tuning sweep runs inside it
    first = {}
    for i, (layer, c, _) in enumerate(calls):
        first.setdefault("full" if layer_window(layer) <= 0 else "window", i)
    cold_ms = {}
    for kind in ("full", "window"):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        rc = L.attn_prefill(*calls[first[kind]][2])
        torch.cuda.synchronize()
        cold_ms[kind] = round((time.perf_counter() - t0) * 1e3, 2)
        if rc != 0:
            raise RuntimeError(f"attn_prefill failed: {binding.attn_last_error()} ({rc})")
    sweeps = binding.attn_tune_stats()

    if args.ab:
        if args.ab_kind == "ragged":
            sel = ragged_calls(torch, binding)
        else:
            keep = {"all": lambda w: True, "full": lambda w: w <= 0, "window": lambda w: w > 0}
            sel = [cl for cl in calls if keep[args.ab_kind](layer_window(cl[0]))]
        res = ab_compare(torch, binding, args.ab, args.ab_rounds, sel)
        res["calls"] = f"{args.ab_kind} ({len(sel)} calls per step)"
        print(json.dumps(res), flush=True)
        return

    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    tuned = {}
    for kind, w in (("full", -1), ("window", WINDOW)):
        idx = binding.attn_tuned_config(D, torch.float16, torch.float16, CHUNK, H_Q, H_KV, w, 1)
        tuned[kind] = binding.attn_config_name(idx) if idx >= 0 else None
    print(f"[bench] warmup done; tuning: {sweeps}; chosen: {tuned}", file=sys.stderr, flush=True)

    # Timed region: K steps of back-to-back launches, one event pair per step
    # on the launch stream (per-step times) and the host clock around all.
    step_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_ev[s][0].record(stream)
        one_step()
        step_ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1000.0 * wall / args.steps
    step_ms = [a.elapsed_time(b) for a, b in step_ev]
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms per step", file=sys.stderr,
          flush=True)

    # Event pass: E more steps with an event pair around every call (an
    # event pair per call adds queue work, so these steps stay outside the
    # whole-job figure); per-call kernel times for the breakdown, the
    # distributions and the roofline.
    E = max(1, args.event_steps)
    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)]
           for _ in calls] for _ in range(E)]
    torch.cuda.synchronize()
    for e in range(E):
        one_step(ev[e])
    torch.cuda.synchronize()
    dur = np.array([[a.elapsed_time(b) for a, b in ev[e]] for e in range(E)])  # ms
    mean_call = dur.mean(axis=0)
    full_idx = [i for i, (layer, c, _) in enumerate(calls) if layer_window(layer) <= 0]
    win_idx = [i for i, (layer, c, _) in enumerate(calls) if layer_window(layer) > 0]
    full_flops = sum(flops[(calls[i][0], calls[i][1])] for i in full_idx)
    win_flops = sum(flops[(calls[i][0], calls[i][1])] for i in win_idx)
    # sums of the per-call event-pair times (each pair adds queue work to its call)
    full_ms_pairs = mean_call[full_idx].sum()
    win_ms_pairs = mean_call[win_idx].sum()

    # Kind passes: one step's full-attention calls alone, in step order and back
    # to back between a single event pair on the launch stream (likewise the
    # window calls): each kernel's average launch duration without the per-call
    # event pairs, which add about 2 us to every call.  The roofline and the
    # per-kind rates come from these; per-chunk distributions from the pairs.
    def kind_pass(idx):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in idx:
            rc = L.attn_prefill(*calls[i][2])
            if rc != 0:
                raise RuntimeError(f"attn_prefill failed: {binding.attn_last_error()} ({rc})")
        b.record(stream)
        return a, b
    KP = max(5, E)
    passes = {"full": [], "window": []}
    torch.cuda.synchronize()
    for _ in range(KP):
        passes["full"].append(kind_pass(full_idx))
        passes["window"].append(kind_pass(win_idx))
    torch.cuda.synchronize()
    pass_ms = {k: [a.elapsed_time(b) for a, b in v] for k, v in passes.items()}
    full_ms = float(np.median(pass_ms["full"]))
    win_ms = float(np.median(pass_ms["window"]))
    full_tflops = full_flops / (full_ms * 1e-3) / 1e12
    win_bytes = sum(algorithmic_bytes(calls[i][1] * CHUNK, CHUNK, WINDOW) for i in win_idx)
    value = step_flops / (ms_per_step * 1e-3) / 1e12

    per_chunk_full = [float(np.mean([mean_call[i] for i in full_idx if calls[i][1] == c])) * 1e3
                      for c in range(N_CHUNKS)]
    per_chunk_win = [float(np.mean([mean_call[i] for i in win_idx if calls[i][1] == c])) * 1e3
                     for c in range(N_CHUNKS)]

    def layer_ms(idx):
        """ms per layer (its 32 chunk calls), one sample per layer and event step."""
        by_layer = {}
        for i in idx:
            by_layer.setdefault(calls[i][0], []).append(i)
        return [float(dur[e, ids].sum()) for e in range(E) for ids in by_layer.values()]

    def chunk_us(idx, chunk):
        return [float(dur[e, i]) * 1e3 for e in range(E) for i in idx if calls[i][1] == chunk]

    full_layer = layer_ms(full_idx)
    distributions = {
        "step_ms": dist(step_ms),
        "full_pass_ms": dist(pass_ms["full"]),
        "window_pass_ms": dist(pass_ms["window"]),
        "full_layer_ms": dist(full_layer),
        "full_pass_frac_peak": dist([full_flops / (x * 1e-3) / 1e12 / PEAK_TFLOPS_F16
                                     for x in pass_ms["full"]], 4),
        "window_layer_ms": dist(layer_ms(win_idx)),
        "full_call_us_chunk31": dist(chunk_us(full_idx, N_CHUNKS - 1), 2),
        "full_call_us_chunk0": dist(chunk_us(full_idx, 0), 2),
        "window_call_us_chunk31": dist(chunk_us(win_idx, N_CHUNKS - 1), 2),
        "window_call_us_chunk0": dist(chunk_us(win_idx, 0), 2),
    }

    if args.copy_calibration:
        copy_calibration(torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu_layers = []
        for layer in (0, 1):
            case, inp, _ = layers[layer]
            cpu_layers.append((case, {k: (v.cpu() if isinstance(v, torch.Tensor) else v)
                                      for k, v in inp.items()}))
        cpu = cpu_baseline(torch, cpu_layers)
        gpu_us = distributions["window_call_us_chunk0"]["median"]
        cpu["single_thread_call"]["gpu_us_median"] = gpu_us
        cpu["single_thread_call"]["ratio"] = round(
            cpu["single_thread_call"]["ms"] * 1e3 / gpu_us, 1)

    traffic = recorded_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "16k chunked prefill: 32 chunks of 512 (past_len 0..15872), 24 layers "
                        "alternating full attention and window 128, H_q=64, H_kv=8, d=64, fp16, "
                        "per-head sinks",
            "calls_per_step": len(calls),
            "full_attn_tflops": round(full_tflops, 2),
            "full_attn_frac_peak": round(full_tflops / PEAK_TFLOPS_F16, 4),
            "full_attn_us_per_call": round(1e3 * full_ms / len(full_idx), 2),
            "full_attn_ms_per_layer": round(full_ms / (len(full_idx) / N_CHUNKS), 3),
            "window_us_per_call": round(1e3 * win_ms / len(win_idx), 2),
            "window_hbm_gbs": round(win_bytes / (win_ms * 1e-3) / 1e9, 1),
            "kind_passes": KP,
            "per_call_event_pairs": {
                "full_us": round(1e3 * full_ms_pairs / len(full_idx), 2),
                "window_us": round(1e3 * win_ms_pairs / len(win_idx), 2),
                "full_frac_peak": round(full_flops / (full_ms_pairs * 1e-3) / 1e12
                                        / PEAK_TFLOPS_F16, 4)},
            "us_per_layer_call": round(1e3 * (full_ms + win_ms) / len(calls), 2),
            "attn_ms_per_16k_prefill": round(full_ms + win_ms, 3),
            "frac_peak_whole_step": round(value / PEAK_TFLOPS_F16, 4),
            "kernel_config": tuned,
            "distributions": distributions,
            "event_steps": E,
            "cold_first_call_ms": {**cold_ms, "tuning_sweeps": sweeps["sweeps"],
                                   "tuning_launches": sweeps["tuning_launches"]},
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(full_tflops, 2),
            "peak": PEAK_TFLOPS_F16,
            "unit": "TFLOP/s",
            "frac": round(full_tflops / PEAK_TFLOPS_F16, 4),
            "traffic": traffic,
            "traffic_source": ("recorded, not measured in this run: rocprofv3 FETCH_SIZE + "
                               "WRITE_SIZE per full-attention launch from "
                               "profiles/full_attention_16k_traffic.txt, taken on this kernel "
                               "source (its hash matches)") if traffic is not None else
                              "null: no counter record matches this kernel source",
            "kernel": "full-attention calls (window <= 0)",
            "launch_us": round(1e3 * full_ms / len(full_idx), 2),
            "duration_source": (f"median of {KP} passes of one step's {len(full_idx)} "
                                "full-attention calls, in step order and back to back, between "
                                "one HIP event pair on the launch stream"),
        },
        "cpu_baseline": cpu,
    }
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"full_us_per_chunk": per_chunk_full, "window_us_per_chunk": per_chunk_win,
                       "result": result}, f, indent=1)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
