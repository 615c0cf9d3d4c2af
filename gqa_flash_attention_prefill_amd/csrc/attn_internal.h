// Internal interface between the C ABI layer (attn_api.cpp) and the gfx950
// kernels (attn_kernel.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Sequences per launch.  Their metadata travels in the kernel arguments
// (no device copy), so a larger batch is split into several launches.
constexpr int kMaxSeq = 128;

// Visited-tile record: int32 fields per record, waves reported per record
// (the layout is attn_tile_log's, in attn_prefill.h).
constexpr int kLogFields = 40;
constexpr int kLogMaxWaves = 8;

struct SeqTable {
  int32_t n_seq;
  int32_t n_tiles;                // cu_tiles[n_seq], also read without indexing
  int32_t cu_tiles[kMaxSeq + 1];  // cumulative Q-tile counts
  int32_t cu_q[kMaxSeq + 1];      // cumulative chunk lengths (rows of q/out)
  int32_t past[kMaxSeq];          // cached keys before each chunk
  int32_t slot[kMaxSeq];          // cache slot (index into the batch dimension)
  int32_t kv_start[kMaxSeq];      // token-pool layout: first entry of each sequence in kv_idx
};

struct Params {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* sink;   // [h_q] or nullptr
  int32_t* log;        // visited-tile records for this launch, or nullptr
  int32_t h_q, h_kv, group;
  int32_t hpack;       // q heads of one KV group packed into a Q tile
  int32_t n_hgroups;   // group / hpack
  int32_t q_rows;      // chunk rows per Q tile (= tile rows / hpack)
  int32_t s_cap;
  int32_t window;
  float scale_log2;    // scale * log2(e)
  // Optional outputs and KV splits across workgroups (blockIdx.y):
  float* lse;          // [tokens, h_q] log-sum-exp of kept scores (natural log, no sink), or nullptr
  float* ws_o;         // n_split > 1: partial outputs [n_split, ws_tokens, h_q, d] (fp32)
  float* ws_lse;       // n_split > 1: partial log-sum-exp [n_split, ws_tokens, h_q] (log2 units)
  int32_t n_split;     // 1: the kernel writes `out`; > 1: it writes partials for attn merge
  int32_t ws_tokens;   // q rows of the whole call (workspace stride)
  int32_t causal;      // 0: non-causal (split/lse kernel variant only)
  // Token-pool layout (split/lse kernel variant only): k and v are pools
  // [n_pool, h_kv, d]; key k of sequence b is pool row kv_idx[kv_start[b] + k].
  const int32_t* kv_idx;  // nullptr: dense caches [batch, h_kv, s_cap, d]
  uint32_t kv_row_bytes;  // bytes between consecutive pool rows (h_kv * d * 2)
  uint32_t n_pool;        // pool rows (indices are clamped below it)
  int32_t swin_run;       // streaming window kernel: Q tiles per workgroup run (its launcher sets it)
  SeqTable seq;
};

// Combine n_split partial results (and the sink) into out / lse.
struct MergeParams {
  const float* ws_o;
  const float* ws_lse;
  const float* sink;   // [h_q] or nullptr
  void* out;
  float* lse;          // or nullptr
  int32_t tokens, h_q, d, n_split;
};
hipError_t launch_merge(const MergeParams& mp, int out_dtype_is_f32, int out_is_bf16,
                        hipStream_t stream);

enum DType { kF16 = 1, kBF16 = 2, kF32 = 3 };

using LaunchFn = hipError_t (*)(const Params&, int n_items, hipStream_t);
// Whether a configuration runs a call: d, window (<= 0: none), chunk rows per
// Q tile, and whether the call asks for KV splits, non-causal attention
// (n_split > 1 or causal == 0).
using AppliesFn = bool (*)(int d, int window, int q_rows, bool split_or_noncausal);

struct KernelConfig {
  const char* name;
  int bkv[3];     // keys per KV tile, [d_index(d)]
  int rows;       // Q-tile rows (q positions x packed heads)
  // indexed [d_index(d)][dtype == bf16][out is f32]
  LaunchFn fn[3][2][2];
  AppliesFn applies;  // nullptr: every call
};

// 0: d 64, 1: d 128, 2: d 256
inline int d_index(int d) { return d == 64 ? 0 : (d == 128 ? 1 : 2); }

// Device scratch of attn_prefill_split_noalloc: a file-scope device array of
// this many bytes (one copy per GPU, held until the process ends).  Returns
// its device address on the current device (looked up once per device).
constexpr int64_t kNoallocScratchBytes = (int64_t)32 << 20;
hipError_t noalloc_scratch(void** ptr);

int config_count();
const KernelConfig& config(int i);
// config(i).applies to the call (a configuration that does not is never
// swept, and a call forced onto it runs default_config instead)
bool config_applies(int i, int d, int window, int q_rows, bool split_or_noncausal);
int default_config(int d, int dtype, int window);

}  // namespace attn
