// C ABI of the gfx950 attention-prefill library: argument checks, declines,
// the host-side work plan, the tuning cache and the launches.
//
// Conventions follow hip-ep pull request 622 ("perf(gqa): support sliding
// windows in the fused flash prefill kernel"): an unsupported request is
// declined with -1 before anything is launched, so a caller can fall back
// instead of getting a wrong result; the tuning cache is keyed on the shape
// of the call rather than on the growing KV length (commit "tuning key"),
// with the window in the key (commit "window in v5"), and tuning launches
// leave the sink out (commit "fold sink into v5 epilogue").
//
// Batch metadata (chunk lengths, cached-prefix lengths) stays on the host and
// travels to the kernel in its arguments: no device allocation, no
// host-to-device copy and no device-to-host read happen on this path.

#include "attn_prefill.h"
#include "attn_internal.h"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <numeric>
#include <string>
#include <tuple>
#include <vector>

static_assert(attn::kLogFields == ATTN_LOG_FIELDS && attn::kLogMaxWaves == ATTN_LOG_MAX_WAVES,
              "tile-log layout of the kernels and of the ABI");
static_assert(attn::kNoallocScratchBytes == ATTN_NOALLOC_SCRATCH_BYTES,
              "the no-allocation entry point's scratch size");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  if (getenv("ATTN_PREFILL_DEBUG")) fprintf(stderr, "[attn_prefill] %s (%d)\n", buf, code);
  return code;
}

// ---- device check: gfx950 only ---------------------------------------------
std::mutex g_dev_mu;
std::map<int, bool> g_dev_ok;

int check_device(int* dev_out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  *dev_out = dev;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  auto it = g_dev_ok.find(dev);
  if (it == g_dev_ok.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(ATTN_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = g_dev_ok.emplace(dev, ok).first;
  }
  if (!it->second) return fail(ATTN_DECLINED, "device %d is not gfx950", dev);
  return ATTN_OK;
}

// ---- tuning cache --------------------------------------------------------------
using TuneKey = std::tuple<int, int, int, int64_t, int, int, int, int, int, int>;
std::mutex g_tune_mu;
std::map<TuneKey, int> g_tune;
int64_t g_sweeps = 0, g_tune_launches = 0;
std::atomic<int> g_forced{-1};

int env_forced_config() {
  const char* s = getenv("ATTN_PREFILL_CONFIG");
  if (!s || !*s) return -1;
  for (int i = 0; i < attn::config_count(); ++i)
    if (strcmp(attn::config(i).name, s) == 0) return i;
  return -1;
}

bool tuning_enabled() {
  const char* s = getenv("ATTN_PREFILL_TUNE");
  return !(s && strcmp(s, "0") == 0);
}

// ---- work plan -------------------------------------------------------------
struct Call {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* sink;
  const int32_t* cu;
  const int32_t* past;
  int32_t batch, window, h_q, h_kv, d, s_cap, dtype, out_dtype;
  float scale;
  attn_tile_log* log;
  hipStream_t stream;
  // log-sum-exp output and KV splits (attn_prefill_split); defaults: none, 1
  float* lse = nullptr;
  int32_t n_split = 1;
  int32_t flags = 0;
  void* workspace = nullptr;
  int64_t workspace_bytes = 0;
  // token-pool layout (attn_prefill_paged): k / v are pools [n_pool, h_kv, d]
  const int32_t* kv_idx = nullptr;     // device: pool row of each key
  const int32_t* kv_indptr = nullptr;  // host [batch + 1]: sequence b's entries in kv_idx
  int64_t n_pool = 0;
  // attn_prefill_split_noalloc: the split workspace is the library's static
  // device scratch, and no tuning sweep runs (a sweep synchronises)
  bool noalloc = false;
};

constexpr int32_t kMaxSplit = 64;

// Workspace of a split call: partial outputs [n_split, tokens, h_q, d] fp32,
// then partial log-sum-exps [n_split, tokens, h_q] fp32.
int64_t split_workspace_bytes(int64_t tokens, int64_t h_q, int64_t d, int64_t n_split) {
  return n_split <= 1 ? 0 : n_split * tokens * h_q * (d + 1) * (int64_t)sizeof(float);
}

int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

// Whether configuration `cfg_index` runs call `c` (KernelConfig::applies).
bool applies(const Call& c, int cfg_index) {
  const int hpack = gcd_int(c.h_q / c.h_kv, 32);
  const int q_rows = attn::config(cfg_index).rows / hpack;
  const bool split_or_noncausal = c.n_split > 1 || (c.flags & ATTN_FLAG_NONCAUSAL) != 0;
  return attn::config_applies(cfg_index, c.d, c.window > 0 ? c.window : 0, q_rows,
                              split_or_noncausal);
}

// Launch every sequence of `c` with configuration `cfg`.  When `log_base` is
// non-null, records go there (the caller checked the capacity) and the number
// written is returned in *n_records.
int run_config(const Call& c, int cfg_index, bool with_sink, int32_t* log_base,
               int64_t* n_records) {
  const attn::KernelConfig& cfg = attn::config(cfg_index);
  const int group = c.h_q / c.h_kv;
  const int hpack = gcd_int(group, 32);
  const int q_rows = cfg.rows / hpack;
  attn::LaunchFn fn = cfg.fn[attn::d_index(c.d)][c.dtype == ATTN_BF16][c.out_dtype == ATTN_F32];
  if (fn == nullptr || !applies(c, cfg_index))
    return fail(ATTN_EINVAL, "configuration %s does not run this call", cfg.name);

  attn::Params p;
  memset(&p, 0, sizeof(p));
  p.q = c.q;
  p.k = c.k;
  p.v = c.v;
  p.out = c.out;
  p.sink = with_sink ? c.sink : nullptr;
  p.h_q = c.h_q;
  p.h_kv = c.h_kv;
  p.group = group;
  p.hpack = hpack;
  p.n_hgroups = group / hpack;
  p.q_rows = q_rows;
  p.s_cap = c.s_cap;
  p.window = c.window > 0 ? c.window : 0;
  p.scale_log2 = c.scale * 1.4426950408889634f;
  const int64_t tokens = c.cu[c.batch] - c.cu[0];
  p.n_split = c.n_split;
  p.ws_tokens = (int32_t)tokens;
  p.causal = (c.flags & ATTN_FLAG_NONCAUSAL) ? 0 : 1;
  if (c.kv_idx) {
    p.kv_idx = c.kv_idx;
    p.kv_row_bytes = (uint32_t)((int64_t)c.h_kv * c.d * 2);
    p.n_pool = (uint32_t)c.n_pool;
  }
  if (c.n_split > 1) {
    p.ws_o = static_cast<float*>(c.workspace);
    p.ws_lse = p.ws_o + (int64_t)c.n_split * tokens * c.h_q * c.d;
  } else {
    p.lse = c.lse;
  }

  int64_t written = 0;
  for (int32_t b0 = 0; b0 < c.batch; b0 += attn::kMaxSeq) {
    const int32_t nb = std::min<int32_t>(attn::kMaxSeq, c.batch - b0);
    attn::SeqTable& st = p.seq;
    st.n_seq = nb;
    st.cu_tiles[0] = 0;
    st.cu_q[0] = c.cu[b0];
    for (int i = 0; i < nb; ++i) {
      const int32_t sq = c.cu[b0 + i + 1] - c.cu[b0 + i];
      st.cu_tiles[i + 1] = st.cu_tiles[i] + (sq + q_rows - 1) / q_rows;
      st.cu_q[i + 1] = c.cu[b0 + i + 1];
      st.past[i] = c.past[b0 + i];
      st.slot[i] = b0 + i;
      st.kv_start[i] = c.kv_indptr ? c.kv_indptr[b0 + i] : 0;
    }
    st.n_tiles = st.cu_tiles[nb];
    const int64_t n_items = (int64_t)st.cu_tiles[nb] * c.h_kv * p.n_hgroups;
    if (n_items == 0) continue;
    if (n_items > 0x7fffffff) return fail(ATTN_EINVAL, "too many work items (%lld)",
                                          (long long)n_items);
    p.log = log_base ? log_base + written * ATTN_LOG_FIELDS : nullptr;
    hipError_t e = fn(p, (int)n_items, c.stream);
    if (e != hipSuccess) return fail(ATTN_EHIP, "kernel launch: %s", hipGetErrorString(e));
    written += n_items * c.n_split;
  }
  if (c.n_split > 1) {
    attn::MergeParams mp;
    mp.ws_o = p.ws_o;
    mp.ws_lse = p.ws_lse;
    mp.sink = with_sink ? c.sink : nullptr;
    mp.out = c.out;
    mp.lse = c.lse;
    mp.tokens = (int32_t)tokens;
    mp.h_q = c.h_q;
    mp.d = c.d;
    mp.n_split = c.n_split;
    hipError_t e = attn::launch_merge(mp, c.out_dtype == ATTN_F32, c.out_dtype == ATTN_BF16,
                                      c.stream);
    if (e != hipSuccess) return fail(ATTN_EHIP, "merge launch: %s", hipGetErrorString(e));
  }
  if (n_records) *n_records = written;
  return ATTN_OK;
}

int64_t plan_items(const Call& c, int cfg_index) {
  const int group = c.h_q / c.h_kv;
  const int hpack = gcd_int(group, 32);
  const int q_rows = attn::config(cfg_index).rows / hpack;
  int64_t tiles = 0;
  for (int32_t b = 0; b < c.batch; ++b) tiles += (c.cu[b + 1] - c.cu[b] + q_rows - 1) / q_rows;
  return tiles * c.h_kv * (group / hpack) * c.n_split;
}

// The key leaves out the KV depth, so its one sweep stands for every depth
// the key will see (for a chunked prefill: the first, shallowest chunk would
// be a poor sample).  The sweep therefore times each sequence at depth
// max(past, min(s_cap, kSweepDepth) - sq): deeper keys of the caller's own
// cache (rows past the valid prefix are in bounds; what they hold only
// reaches the sweep's discarded output).
constexpr int32_t kSweepDepth = 16384;

// One synchronous sweep: time each configuration on the caller's buffers and
// stream (the output is overwritten by the real launch that follows).
int sweep(const Call& c_in, int* best_out) {
  std::vector<int32_t> deep(c_in.batch > 0 ? c_in.batch : 1);
  for (int32_t b = 0; b < c_in.batch; ++b) {
    const int32_t sq = c_in.cu[b + 1] - c_in.cu[b];
    // a token-pool call's index lists end at its own keys: no deeper sample
    deep[b] = c_in.kv_idx ? c_in.past[b]
                          : std::max(c_in.past[b], std::min(c_in.s_cap, kSweepDepth) - sq);
  }
  Call c = c_in;
  c.past = deep.data();
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess)
    return fail(ATTN_EHIP, "hipEventCreate failed");
  // Three passes over the configurations (interleaved, so that a drift of
  // the clock hits all of them alike); in each, a configuration is launched
  // back to back until at least kMinBatchUs of work is timed, and it is
  // ranked by the median of its three per-call times.  Short calls (window
  // chunks, decode rows) then get tens of repetitions per pass, and one slow
  // or fast outlier pass does not decide the choice.
  constexpr float kMinBatchUs = 150.f;
  constexpr int kPasses = 3;
  const int n_cfg = attn::config_count();
  std::vector<float> pass_us(n_cfg * kPasses, INFINITY);
  std::vector<int> reps(n_cfg, 3);
  int64_t launches = 0;
  int rc = ATTN_OK;
  auto timed = [&](int i, int n, float* us) {
    if (hipEventRecord(e0, c.stream) != hipSuccess) return fail(ATTN_EHIP, "event");
    for (int r = 0; r < n; ++r, ++launches) {
      int rr = run_config(c, i, false, nullptr, nullptr);
      if (rr) return rr;
    }
    if (hipEventRecord(e1, c.stream) != hipSuccess) return fail(ATTN_EHIP, "event");
    if (hipEventSynchronize(e1) != hipSuccess) return fail(ATTN_EHIP, "sweep sync");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return fail(ATTN_EHIP, "event");
    *us = 1000.f * ms / n;
    return (int)ATTN_OK;
  };
  for (int pass = 0; pass < kPasses && rc == ATTN_OK; ++pass) {
    for (int i = 0; i < n_cfg && rc == ATTN_OK; ++i) {
      if (!applies(c, i)) continue;  // never chosen (its times stay infinite)
      float us = 0.f;
      if (pass == 0) {
        rc = run_config(c, i, false, nullptr, nullptr);  // warm-up
        ++launches;
        if (rc) break;
        rc = timed(i, reps[i], &us);
        if (rc) break;
        if (us * reps[i] < kMinBatchUs) {
          reps[i] = std::min(64, (int)std::ceil(kMinBatchUs / std::max(us, 0.5f)));
          rc = timed(i, reps[i], &us);
          if (rc) break;
        }
      } else {
        rc = timed(i, reps[i], &us);
        if (rc) break;
      }
      pass_us[i * kPasses + pass] = us;
      if (getenv("ATTN_PREFILL_TUNE_DEBUG"))
        fprintf(stderr, "[attn_prefill tune] %-20s pass %d %9.3f us (%d reps)\n",
                attn::config(i).name, pass, us, reps[i]);
    }
  }
  auto median = [&](int i) {
    float v[kPasses];
    for (int k = 0; k < kPasses; ++k) v[k] = pass_us[i * kPasses + k];
    std::sort(v, v + kPasses);
    return v[kPasses / 2];
  };
  int best = attn::default_config(c.d, c.dtype, c.window);
  for (int i = 0; i < n_cfg; ++i)
    if (median(i) < median(best)) best = i;
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  g_tune_launches += launches;
  *best_out = best;
  return rc;
}

int choose_config(const Call& c, int* cfg) {
  const int forced = g_forced.load();
  if (forced >= 0) { *cfg = forced; return ATTN_OK; }
  const int env = env_forced_config();
  if (env >= 0) { *cfg = env; return ATTN_OK; }
  if (!tuning_enabled()) {
    *cfg = attn::default_config(c.d, c.dtype, c.window);
    return ATTN_OK;
  }
  const int64_t tokens = c.cu[c.batch] - c.cu[0];
  TuneKey key{c.d, c.dtype, c.out_dtype, tokens, c.h_q, c.h_q / c.h_kv,
              c.window > 0 ? c.window : 0, c.batch, c.n_split,
              c.flags | (c.kv_idx ? 0x100 : 0)};  // token-pool calls tune separately
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto it = g_tune.find(key);
  if (it != g_tune.end()) { *cfg = it->second; return ATTN_OK; }
  if (c.noalloc) {
    // never sweeps: the key's earlier choice (above), else the default
    *cfg = attn::default_config(c.d, c.dtype, c.window);
    return ATTN_OK;
  }
  int best = 0;
  int rc = sweep(c, &best);
  if (rc) return rc;
  ++g_sweeps;
  g_tune.emplace(key, best);
  if (getenv("ATTN_PREFILL_TUNE_DEBUG"))
    fprintf(stderr, "[attn_prefill tune] chose %s\n", attn::config(best).name);
  *cfg = best;
  return ATTN_OK;
}

int validate(const Call& c) {
  if (c.batch < 0) return fail(ATTN_EINVAL, "batch < 0");
  if (c.batch > 0 && (!c.cu || !c.past)) return fail(ATTN_EINVAL, "null batch metadata");
  if (c.h_q <= 0 || c.h_kv <= 0 || c.d <= 0 || c.s_cap < 0)
    return fail(ATTN_EINVAL, "non-positive size");
  if (c.h_q % c.h_kv != 0) return fail(ATTN_EINVAL, "h_q %% h_kv != 0");
  if (c.batch > 0) {
    if (c.cu[0] != 0) return fail(ATTN_EINVAL, "cu_seqlens_q[0] != 0");
    for (int32_t b = 0; b < c.batch; ++b) {
      const int64_t sq = (int64_t)c.cu[b + 1] - c.cu[b];
      if (sq < 0) return fail(ATTN_EINVAL, "cu_seqlens_q decreases at %d", b);
      if (c.past[b] < 0) return fail(ATTN_EINVAL, "past_len[%d] < 0", b);
      if (c.kv_indptr) {
        const int64_t n = (int64_t)c.kv_indptr[b + 1] - c.kv_indptr[b];
        if (c.kv_indptr[b] < 0 || n < 0)
          return fail(ATTN_EINVAL, "kv_indptr negative or decreasing at %d", b);
        if ((int64_t)c.past[b] + sq > n)
          return fail(ATTN_EINVAL, "sequence %d has %lld pool indices for %lld keys", b,
                      (long long)n, (long long)c.past[b] + sq);
      } else if ((int64_t)c.past[b] + sq > c.s_cap) {
        return fail(ATTN_EINVAL, "past_len + sq > s_cap for sequence %d", b);
      }
    }
  }
  const int64_t tokens = c.batch > 0 ? c.cu[c.batch] : 0;
  if (tokens > 0 && (!c.q || !c.k || !c.v || !c.out))
    return fail(ATTN_EINVAL, "null tensor pointer");
  if (c.scale != c.scale || std::isinf(c.scale)) return fail(ATTN_EINVAL, "scale not finite");
  if (c.kv_indptr || c.kv_idx) {
    if (c.batch > 0 && !c.kv_indptr) return fail(ATTN_EINVAL, "null kv_indptr");
    if (tokens > 0 && !c.kv_idx) return fail(ATTN_EINVAL, "null kv_indices");
    if (c.n_pool < 1) return fail(ATTN_EINVAL, "n_pool < 1");
  }
  if (c.log) {
    if (c.log->capacity < 0 || (c.log->capacity > 0 && !c.log->records))
      return fail(ATTN_EINVAL, "bad tile log");
  }
  if (c.flags & ~ATTN_FLAG_NONCAUSAL) return fail(ATTN_EINVAL, "unknown flags 0x%x", c.flags);
  if (c.n_split < 1 || c.n_split > kMaxSplit)
    return fail(ATTN_EINVAL, "n_split %d outside 1..%d", c.n_split, kMaxSplit);
  if (c.noalloc && tokens > 0) {
    const int64_t need = split_workspace_bytes(tokens, c.h_q, c.d, c.n_split);
    if (need > attn::kNoallocScratchBytes)
      return fail(ATTN_EINVAL,
                  "split partials need %lld bytes, above the %lld-byte scratch of the "
                  "no-allocation entry point (use attn_prefill_split with a workspace)",
                  (long long)need, (long long)attn::kNoallocScratchBytes);
  } else if (c.n_split > 1 && tokens > 0) {
    const int64_t need = split_workspace_bytes(tokens, c.h_q, c.d, c.n_split);
    if (!c.workspace || c.workspace_bytes < need)
      return fail(ATTN_EINVAL, "split workspace holds %lld bytes, %lld needed",
                  (long long)c.workspace_bytes, (long long)need);
  }
  // declines: valid requests this library does not implement
  if (c.d != 64 && c.d != 128 && c.d != 256)
    return fail(ATTN_DECLINED, "d=%d not supported (64, 128, 256)", c.d);
  if (c.dtype != ATTN_F16 && c.dtype != ATTN_BF16)
    return fail(ATTN_DECLINED, "input dtype %d not supported", c.dtype);
  if (c.out_dtype != c.dtype && c.out_dtype != ATTN_F32)
    return fail(ATTN_DECLINED, "out dtype %d not supported for input dtype %d", c.out_dtype,
                c.dtype);
  // fp16 q is pre-scaled by scale * log2 e in fp16; |q| <= 65504, so the
  // product stays finite exactly when |scale| * log2 e <= 1
  if (c.dtype == ATTN_F16 && std::fabs((double)c.scale) * 1.4426950408889634 > 1.0)
    return fail(ATTN_DECLINED,
                "fp16 inputs with |scale| > ln 2 (%g): the pre-scaled fp16 q could overflow",
                (double)c.scale);
  if (tokens > 0) {
    auto mis = [](const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) != 0; };
    if (mis(c.q) || mis(c.k) || mis(c.v) || mis(c.out))
      return fail(ATTN_DECLINED, "tensor pointers must be 16-byte aligned");
    if (c.n_split > 1 && mis(c.workspace))
      return fail(ATTN_DECLINED, "the split workspace must be 16-byte aligned");
    // pool byte offsets travel as 32-bit load offsets
    if (c.kv_idx && c.n_pool * c.h_kv * c.d * 2 > (int64_t)0xffffffffu)
      return fail(ATTN_DECLINED, "token pool above 4 GiB per tensor not supported");
  }
  return ATTN_OK;
}

int run(const Call& c_in) {
  g_last_error.clear();
  int rc = validate(c_in);
  if (rc) return rc;
  const int64_t tokens = c_in.batch > 0 ? c_in.cu[c_in.batch] : 0;
  if (tokens == 0) {
    if (c_in.log) { c_in.log->n_records = 0; }
    return ATTN_OK;
  }
  int dev = 0;
  rc = check_device(&dev);
  if (rc) return rc;
  Call c = c_in;
  if (c.noalloc && c.n_split > 1) {
    // the static scratch of this device (its address, looked up once)
    hipError_t e = attn::noalloc_scratch(&c.workspace);
    if (e != hipSuccess) return fail(ATTN_EHIP, "scratch address: %s", hipGetErrorString(e));
    c.workspace_bytes = attn::kNoallocScratchBytes;
  }
  int cfg = 0;
  rc = choose_config(c, &cfg);
  if (rc) return rc;
  // a configuration forced onto a call it does not run: the default instead
  if (!applies(c, cfg)) cfg = attn::default_config(c.d, c.dtype, c.window);
  int32_t* log_base = nullptr;
  if (c.log) {
    const int64_t need = plan_items(c, cfg);
    if (need > c.log->capacity)
      return fail(ATTN_EINVAL, "tile log holds %lld records, %lld needed",
                  (long long)c.log->capacity, (long long)need);
    log_base = c.log->records;
    c.log->bkv = attn::config(cfg).bkv[attn::d_index(c.d)];
    const int hpack = gcd_int(c.h_q / c.h_kv, 32);
    c.log->q_rows = attn::config(cfg).rows / hpack;
  }
  int64_t n = 0;
  rc = run_config(c, cfg, true, log_base, &n);
  if (rc) return rc;
  if (c.log) c.log->n_records = n;
  if (getenv("ATTN_PREFILL_DEBUG"))
    fprintf(stderr, "[attn_prefill] config %s, %lld work items\n", attn::config(cfg).name,
            (long long)plan_items(c, cfg));
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_prefill(const void* q, const void* k_cache, const void* v_cache, int32_t past_len,
                 int32_t window, const float* head_sink, float scale, void* out, int32_t sq,
                 int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap, int32_t dtype,
                 int32_t out_dtype, void* stream) {
  try {
    if (sq < 0) return fail(ATTN_EINVAL, "sq < 0");
    const int32_t cu[2] = {0, sq};
    const int32_t past[1] = {past_len};
    Call c{q, k_cache, v_cache, out, head_sink, cu, past, 1, window, h_q, h_kv, d, s_cap,
           dtype, out_dtype, scale, nullptr, reinterpret_cast<hipStream_t>(stream)};
    return run(c);
  } catch (...) {
    return fail(ATTN_EHIP, "internal error");
  }
}

int attn_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* cu_seqlens_q, const int32_t* past_len, int32_t batch,
                        int32_t window, const float* head_sink, float scale, void* out,
                        int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap, int32_t dtype,
                        int32_t out_dtype, attn_tile_log* tile_log, void* stream) {
  try {
    Call c{q, k_cache, v_cache, out, head_sink, cu_seqlens_q, past_len, batch, window, h_q,
           h_kv, d, s_cap, dtype, out_dtype, scale, tile_log,
           reinterpret_cast<hipStream_t>(stream)};
    return run(c);
  } catch (...) {
    return fail(ATTN_EHIP, "internal error");
  }
}

int attn_prefill_split(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cu_seqlens_q, const int32_t* past_len, int32_t batch,
                       int32_t window, const float* head_sink, float scale, void* out,
                       float* lse, int32_t h_q, int32_t h_kv, int32_t d, int32_t s_cap,
                       int32_t dtype, int32_t out_dtype, int32_t n_split, int32_t flags,
                       void* workspace, int64_t workspace_bytes, attn_tile_log* tile_log,
                       void* stream) {
  try {
    Call c{q, k_cache, v_cache, out, head_sink, cu_seqlens_q, past_len, batch, window, h_q,
           h_kv, d, s_cap, dtype, out_dtype, scale, tile_log,
           reinterpret_cast<hipStream_t>(stream)};
    c.lse = lse;
    c.n_split = n_split;
    c.flags = flags;
    c.workspace = workspace;
    c.workspace_bytes = workspace_bytes;
    return run(c);
  } catch (...) {
    return fail(ATTN_EHIP, "internal error");
  }
}

int attn_prefill_split_noalloc(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens_q, const int32_t* past_len,
                               int32_t batch, int32_t window, const float* head_sink, float scale,
                               void* out, float* lse, int32_t h_q, int32_t h_kv, int32_t d,
                               int32_t s_cap, int32_t dtype, int32_t out_dtype, int32_t n_split,
                               int32_t flags, attn_tile_log* tile_log, void* stream) {
  try {
    Call c{q, k_cache, v_cache, out, head_sink, cu_seqlens_q, past_len, batch, window, h_q,
           h_kv, d, s_cap, dtype, out_dtype, scale, tile_log,
           reinterpret_cast<hipStream_t>(stream)};
    c.lse = lse;
    c.n_split = n_split;
    c.flags = flags;
    c.noalloc = true;
    return run(c);
  } catch (...) {
    return fail(ATTN_EHIP, "internal error");
  }
}

int attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool, int64_t n_pool,
                       const int32_t* kv_indices, const int32_t* kv_indptr,
                       const int32_t* cu_seqlens_q, const int32_t* past_len, int32_t batch,
                       int32_t window, const float* head_sink, float scale, void* out,
                       float* lse, int32_t h_q, int32_t h_kv, int32_t d, int32_t dtype,
                       int32_t out_dtype, int32_t flags, attn_tile_log* tile_log,
                       void* stream) {
  try {
    Call c{q, k_pool, v_pool, out, head_sink, cu_seqlens_q, past_len, batch, window, h_q,
           h_kv, d, 0, dtype, out_dtype, scale, tile_log, reinterpret_cast<hipStream_t>(stream)};
    c.lse = lse;
    c.flags = flags;
    c.kv_idx = kv_indices;
    c.kv_indptr = kv_indptr;
    c.n_pool = n_pool;
    // null index arrays would make this a dense call with s_cap 0: name them
    if (batch > 0 && (!kv_indptr || !kv_indices)) return fail(ATTN_EINVAL, "null kv_indptr / kv_indices");
    return run(c);
  } catch (...) {
    return fail(ATTN_EHIP, "internal error");
  }
}

int64_t attn_split_workspace_bytes(int64_t q_tokens, int32_t h_q, int32_t d, int32_t n_split) {
  if (q_tokens < 0 || h_q <= 0 || d <= 0 || n_split < 1) return -1;
  return split_workspace_bytes(q_tokens, h_q, d, n_split);
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_tune_stats(int64_t* sweeps, int64_t* tuning_launches, int64_t* cached_keys) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  if (sweeps) *sweeps = g_sweeps;
  if (tuning_launches) *tuning_launches = g_tune_launches;
  if (cached_keys) *cached_keys = (int64_t)g_tune.size();
  return ATTN_OK;
}

void attn_tune_reset(void) {
  std::lock_guard<std::mutex> lk(g_tune_mu);
  g_tune.clear();
  g_sweeps = 0;
  g_tune_launches = 0;
}

int32_t attn_tuned_config(int32_t d, int32_t dtype, int32_t out_dtype, int64_t q_tokens,
                          int32_t h_q, int32_t h_kv, int32_t window, int32_t batch) {
  if (h_kv <= 0) return -1;
  const TuneKey key{d, dtype, out_dtype, q_tokens, h_q, h_q / h_kv, window > 0 ? window : 0,
                    batch, 1, 0};  // the key of unsplit causal calls
  std::lock_guard<std::mutex> lk(g_tune_mu);
  auto it = g_tune.find(key);
  return it == g_tune.end() ? -1 : it->second;
}

int32_t attn_config_count(void) { return attn::config_count(); }

const char* attn_config_name(int32_t i) {
  if (i < 0 || i >= attn::config_count()) return nullptr;
  return attn::config(i).name;
}

int attn_force_config(int32_t i) {
  if (i < -1 || i >= attn::config_count()) return fail(ATTN_EINVAL, "no configuration %d", i);
  g_forced.store(i);
  return ATTN_OK;
}

}  // extern "C"
