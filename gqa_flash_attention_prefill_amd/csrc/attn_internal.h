// Internal interface between the C ABI layer (attn_api.cpp) and the gfx950
// kernels (attn_kernel.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Sequences per launch.  Their metadata travels in the kernel arguments
// (no device copy), so a larger batch is split into several launches.
constexpr int kMaxSeq = 128;

struct SeqTable {
  int32_t n_seq;
  int32_t cu_tiles[kMaxSeq + 1];  // cumulative Q-tile counts
  int32_t cu_q[kMaxSeq + 1];      // cumulative chunk lengths (rows of q/out)
  int32_t past[kMaxSeq];          // cached keys before each chunk
  int32_t slot[kMaxSeq];          // cache slot (index into the batch dimension)
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
  SeqTable seq;
};

enum DType { kF16 = 1, kBF16 = 2, kF32 = 3 };

using LaunchFn = hipError_t (*)(const Params&, int n_items, hipStream_t);

struct KernelConfig {
  const char* name;
  int bkv[2];     // keys per KV tile, [d == 128]
  int rows;       // Q-tile rows (q positions x packed heads)
  // indexed [d == 128][dtype == bf16][out is f32]
  LaunchFn fn[2][2][2];
};

int config_count();
const KernelConfig& config(int i);
int default_config(int d, int dtype, int window);

}  // namespace attn
