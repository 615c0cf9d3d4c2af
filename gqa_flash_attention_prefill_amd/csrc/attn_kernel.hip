// Fused causal grouped-query flash-attention prefill for gfx950 (CDNA 4).
//
// What is computed (hip-ep pull request 622, "perf(gqa): support sliding
// windows in the fused flash prefill kernel"; sgl-project/sglang pull request
// 34468): for each chunk row at absolute position past + q, softmax over the
// kept keys k <= past + q and, with a window, k >= past + q - window + 1,
// with an optional per-head sink logit added to the denominator only.
//
// Work decomposition.  One workgroup = one Q tile = NW waves x 32 rows.  The
// rows of a tile are (chunk position, q head) pairs: `hpack` q heads of one
// KV group share each position, so one K/V tile staged in LDS serves every
// head of the group ("no-expand" GQA: KV heads are never replicated).
//
// Per KV tile (BKV keys):
//   * K and V move from HBM straight into an LDS ring (global_load_lds
//     direct loads, 16 bytes per lane, both row-major and XOR-swizzled in
//     16-byte chunks) several tiles ahead of their use; a barrier per stage
//     hands a landed tile to every wave;
//   * S^T = K . Q^T on v_mfma_f32_32x32x16_{f16,bf16}: with K as the A operand
//     and the wave's Q (held in registers for the whole loop) as B, each
//     lane's accumulator holds ONE query row (lane % 32) and 16 keys, so the
//     row max is an in-lane reduction plus one exchange with lane ^ 32 and
//     the rescale of the output accumulator is lane-local;
//   * mask only on boundary tiles; online softmax in exp2 space (fp16 Q is
//     pre-scaled by scale * log2 e and the running max enters as the MFMA's
//     accumulator input; bf16 applies both in one FMA); the reference max
//     is raised lazily (only when a row's tile max exceeds it by 2^8), which
//     skips most accumulator rescales; a row that has seen no key and whose
//     tile is fully masked keeps m = -inf and is guarded ("window in v5":
//     exp2(-inf - -inf) would be NaN);
//   * O^T += V^T . P^T on the same MFMA: P is converted to 16-bit in
//     registers and used directly as the B operand; V^T comes from the
//     row-major V tile through the gfx950 transposing LDS read
//     ds_read_b64_tr_b16.  For bf16 inputs P is split into hi + lo bf16
//     parts and both are accumulated, since one bf16 rounding of P alone
//     costs ~1e-3 relative error.
//   * Two waves per row group (KV splits) take alternate tiles, so each
//     SIMD holds two independent waves; their partial (m, l, O) are merged
//     through LDS before the epilogue.  Three kernels share all of the
//     above: attn_fwd_kernel, where each wave software-pipelines the matrix
//     work of one tile with the vector work of the previous one;
//     attn_pp_kernel (d 64), where the two waves of a SIMD alternate whole
//     matrix and vector phases between workgroup barriers; and
//     attn_swin_kernel (window calls of long chunks), where one workgroup
//     walks a run of consecutive Q tiles whose windows share an LDS ring of
//     32-key blocks.
//
// KV loop bounds ("window in v5"; sglang 34468 "bound the stage-1 prefix
// loop"): the loop starts at the tile holding the lowest key the Q tile's
// FIRST row keeps (lower bounds are non-decreasing within a tile) and ends
// at the tile holding the LAST row's own key; the per-row mask trims the
// rest.  Waves skip tiles outside their own rows' range.
//
// Epilogue ("fold sink into v5 epilogue"): l += exp2(sink * log2 e - m) when
// m != -inf; out = acc / max(l, FLT_MIN).

#include "attn_internal.h"

#include <float.h>

#include <mutex>
#include <type_traits>

namespace attn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct F16 {
  static constexpr bool kSplitP = false;
  static constexpr uint32_t kOnePair = 0x3c003c00u;  // two fp16 1.0
  // Q is pre-scaled by scale * log2(e) (one extra fp16 rounding of q, ~1e-4
  // relative in p, the size of P's own rounding) so that S^T arrives in exp2
  // units and the running max can enter through the MFMA accumulator input.
  static constexpr bool kPrescaleQ = true;
  __device__ static f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // round to nearest even (v_cvt_pk_f16_f32)
  __device__ static uint32_t pack(float x, float y) {
    f16x2 h = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
  __device__ static float lo_part(float, uint32_t, int) { return 0.f; }
  // l + (both fp16 halves of `packed`), accumulated in fp32 (v_dot2c_f32_f16)
  __device__ static float rowsum(uint32_t packed, float l) {
    const f16x2 one = {(_Float16)1.f, (_Float16)1.f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), one, l, false);
  }
};

struct BF16 {
  static constexpr bool kSplitP = true;
  static constexpr uint32_t kOnePair = 0x3f803f80u;  // two bf16 1.0
  static constexpr bool kPrescaleQ = false;  // a bf16 rounding of q*c would cost ~1e-3
  __device__ static f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // round to nearest even (v_cvt_pk_bf16_f32)
  __device__ static uint32_t pack(float x, float y) {
    bf16x2 h = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, h);
  }
  // x - (the bf16 value in half `which` of `packed`)
  __device__ static float lo_part(float x, uint32_t packed, int which) {
    uint32_t bits = which ? (packed & 0xffff0000u) : (packed << 16);
    return x - __builtin_bit_cast(float, bits);
  }
  __device__ static float rowsum(uint32_t, float l) { return l; }
};

template <typename TI>
__device__ inline u32x4 load16(const void* base, int64_t elem_offset) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(base) + elem_offset);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16-byte-chunk XOR swizzles of the K and V tiles in LDS (both row-major,
// one key per row), chosen so that the fragment reads below are free of bank
// conflicts on the 64-bank (256 B per clock) LDS:
//  K: S^T reads 16 bytes per lane, lanes 0..15 on 16 consecutive keys of one
//     chunk column; a pass serves 16 lanes = 256 bytes, so the 16 keys must
//     land on 16 distinct 16-byte bank groups.  At d = 64 a key row is half
//     the bank width: keys 2i and 2i + 1 sit in opposite halves, and
//     chunk ^ ((key >> 1) & 7) spreads each half's 8 keys over its 8 groups.
//     At d = 128 a row spans all banks: chunk ^ (key & 15).
//  V: transposed reads (ds_read_b64_tr_b16) take 4 keys x 32 bytes per
//     16-lane group and 8 keys per instruction; chunk ^ ((key & 3) << 1) at
//     d = 64 and chunk ^ ((key & 3) << 2) at d = 128 give every key of an
//     instruction its own banks.
template <int D>
__device__ inline int k_chunk(int key, int c) {
  return D == 64 ? c ^ ((key >> 1) & 7) : c ^ (key & 15);   // d 256: rows span two bank widths
}
template <int D>
__device__ inline int v_chunk(int key, int c) {
  return D == 64 ? c ^ ((key & 3) << 1) : c ^ ((key & 3) << 2);
}

// Lane layout used with v_mfma_f32_32x32x16 (A: 32 rows x 16 k, B: 16 k x 32
// cols, C: 32 x 32):  A/B lane l holds row/col l % 32 and k = 8 (l / 32) + 0..7;
// C lane l holds column l % 32 and rows 8 (i / 4) + 4 (l / 32) + (i % 4), i < 16.
//
// S^T = K . Q^T puts query (l % 32) in every lane's 16 accumulators, over keys
// 8 (i / 4) + 4 h + (i % 4) of a 32-key block (h = l / 32).  P = exp2(...) of
// those 16 values, converted to 16 bits, is directly the B operand (P^T) of
// two PV steps: step j2 covers keys 16 j2 + {4h .. 4h+3, 8+4h .. 8+4h+3}, in
// the order of accumulators 8 j2 .. 8 j2 + 7.  The matching A operand (V^T)
// needs, in lane (d, h), V[key][d] for those 8 keys: two ds_read_b64_tr_b16
// loads of 4 keys each.  That instruction hands lane i of each 16-lane group
// element (i % 4) of the 8-byte pieces addressed by lanes 4k + i / 4 (k < 4),
// so lane j of the group addresses V[key0 + j / 4][d0 + 4 (j % 4) .. + 3] and
// lane i receives V[key0 + k][d0 + i], k = 0..3.
template <int D>
__device__ inline u32x4 v_frag(const u32x4* vt, int g16, int db, int lane) {
  constexpr int DCH = D / 8;
  const int j = lane & 15, grp = lane >> 4;
  const int h = grp >> 1;
  const int d = db * 32 + (grp & 1) * 16 + 4 * (j & 3);
  const int key_a = g16 * 16 + 4 * h + (j >> 2);
  const int key_b = key_a + 8;
  const uint16_t* base = reinterpret_cast<const uint16_t*>(vt);
  const uint16_t* pa = base + (key_a * DCH + v_chunk<D>(key_a, d >> 3)) * 8 + (d & 7);
  const uint16_t* pb = base + (key_b * DCH + v_chunk<D>(key_b, d >> 3)) * 8 + (d & 7);
  const s16x4 ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pa);
  const s16x4 rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)pb);
  const u32x2 a2 = __builtin_bit_cast(u32x2, ra), b2 = __builtin_bit_cast(u32x2, rb);
  return u32x4{a2[0], a2[1], b2[0], b2[1]};
}

__device__ inline float other_half(float x) { return __shfl_xor(x, 32); }

// max(x, x of lane ^ 32) through v_permlane32_swap (a VALU lane swap between
// the two 32-lane halves; no LDS round trip).  With both operands holding x,
// the swap leaves the low half's values in one register and the high half's
// in the other, in every lane.  The s_nop covers the VALU-write ->
// permlane-read hazard of the operands.
__device__ inline float pair_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return __builtin_elementwise_maximum(a, b);
}

// One 16-byte-per-lane direct global -> LDS load (global_load_lds_dwordx4):
// lane i reads sbase + voff and its 16 bytes land at LDS byte address
// lds_addr + 16 i.  Issued through inline assembly so that the compiler does
// not treat it as an LDS store that every later LDS read must wait for (the
// loads fill a ring slot that no wave reads until the stage barrier; the
// kernel waits for them with explicit s_waitcnt vmcnt before that barrier).
__device__ inline void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  // the base is wave-uniform by construction; readfirstlane makes that
  // visible where the compiler cannot prove it, so it lands in SGPRs
  // (the builtin returns int: widen through uint32_t, never sign-extend)
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  sbase = reinterpret_cast<const void*>((hi << 32) | lo);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

// The same with 4 bytes per lane (global_load_lds_dword): lane i's word
// lands at lds_addr + 4 i.
__device__ inline void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  const uint64_t a = reinterpret_cast<uint64_t>(sbase);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  sbase = reinterpret_cast<const void*>((hi << 32) | lo);
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(sbase)
               : "memory", "m0");
}

__device__ inline uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt immediate (gfx9 encoding) waiting until at most n vector-memory
// operations of this wave are outstanding; LDS/export counters unconstrained.
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | (15 << 8) | (7 << 4) | (n & 15); }
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Helpers that take the kernel arguments (Params) by reference, and the
// kernels' lambdas (which capture them by reference), are always inlined: a
// call that is not needs the arguments' address, and the compiler then
// copies the whole 2.5 KB argument block into per-lane scratch at kernel
// entry (it did so for the d 128 and d 256 instantiations).
//
// One workgroup's work item: KV head g, head group hg and Q tile of sequence
// bi (items run heaviest Q tile first).  The first sequence's table entries
// are read together with the scalars the item depends on, so a one-sequence
// call decodes its item in one round trip to the kernel arguments; later
// sequences are found by binary search over the cumulative tile counts.
struct WorkItem {
  int g, hg, bi, sq, past, slot, q0, kv_start;
  int64_t tok0;
};
template <bool XTRA, bool BATCH>
__device__ __attribute__((always_inline)) WorkItem decode_item(const Params& p, int item) {
  int n_seq = p.seq.n_seq, n_tiles = p.seq.n_tiles;
  int h_kv = p.h_kv, n_hg = p.n_hgroups, q_rows = p.q_rows;
  int cu0 = p.seq.cu_q[0], cu1 = p.seq.cu_q[1], tile0 = 0;
  WorkItem w;
  w.past = p.seq.past[0];
  w.slot = p.seq.slot[0];
  w.kv_start = p.seq.kv_start[0];
  // BATCH: every kernel argument the kernel reads before its first global
  // loads, consumed here at once, so the scalar loads issue as one batch with
  // one wait (left to itself the scheduler issues them in several batches,
  // each waited for at its first use) and later reads reuse the values.  The
  // item's decode takes its operands from the statement, so it cannot be
  // scheduled between the loads.  (Some d = 128 instantiations fail to
  // compile with these scalar-register operands, so d 128 and d 256 decode
  // without it.)
  if constexpr (BATCH) {
    asm volatile(""
                 : "+s"(n_seq), "+s"(n_tiles), "+s"(h_kv), "+s"(n_hg), "+s"(q_rows)
                 : "s"(p.scale_log2), "s"(cu0), "s"(cu1), "s"(w.past), "s"(w.slot), "s"(p.h_q),
                   "s"(p.group), "s"(p.hpack), "s"(p.s_cap), "s"(p.window), "s"(p.q), "s"(p.k),
                   "s"(p.v), "s"(p.sink));
    if constexpr (XTRA)
      asm volatile("" ::"s"(w.kv_start), "s"(p.causal), "s"(p.n_split), "s"(p.kv_idx),
                   "s"(p.kv_row_bytes), "s"(p.n_pool));
  }
  w.g = item % h_kv;
  const int r0 = item / h_kv;
  w.hg = r0 % n_hg;
  const int tix = n_tiles - 1 - r0 / n_hg;
  w.bi = 0;
  if (n_seq > 1) {
    int lo = 0, hi = n_seq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (p.seq.cu_tiles[mid] <= tix) lo = mid; else hi = mid - 1;
    }
    w.bi = lo;
    if (lo > 0) {
      cu0 = p.seq.cu_q[lo];
      cu1 = p.seq.cu_q[lo + 1];
      tile0 = p.seq.cu_tiles[lo];
      w.past = p.seq.past[lo];
      w.slot = p.seq.slot[lo];
      w.kv_start = p.seq.kv_start[lo];
    }
  }
  w.sq = cu1 - cu0;
  w.tok0 = cu0;
  w.q0 = (tix - tile0) * q_rows;
  return w;
}

// Stand-in sink logit for calls without sinks (exp2 of -inf adds nothing).
__device__ const float g_no_sink = -__builtin_inff();
typedef __attribute__((address_space(1))) const float global_f32;
// The row's sink logit, read through a global (not flat) load: a flat load
// would also count against the LDS/scalar-memory counter, so the next wait on
// that counter would stall on it.
__device__ inline float load_sink(const float* sink, int head) {
  const float* ptr = sink != nullptr ? sink + head : &g_no_sink;
  return *(const global_f32*)ptr;
}

// Q fragments as the MFMAs take them: zero for rows past the chunk; fp16 Q
// pre-scaled by scale * log2 e (one fp16 rounding), so that S comes out of
// the MFMA in exp2 units; bf16 Q as loaded.  The fp16 product is finite for
// every fp16 q (|q| <= 65504) as long as |scale| * log2 e <= 1; the host
// declines fp16 calls with a larger scale.
template <typename TI, int KSTEPS>
__device__ inline void prepare_q(u32x4* qf, float c, bool valid) {
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    if constexpr (TI::kPrescaleQ) {
      const f16x8 h8 = __builtin_bit_cast(f16x8, qf[kk]);
      f16x8 o8;
#pragma unroll
      for (int e = 0; e < 8; ++e) o8[e] = (_Float16)((float)h8[e] * c);
      qf[kk] = __builtin_bit_cast(u32x4, o8);
    }
    if (!valid) qf[kk] = u32x4{0, 0, 0, 0};
  }
}

// Final epilogue of one row (each lane holds half of the row's output
// columns).  XTRA: compiled with the log-sum-exp output and the split
// partials (the plain instantiations carry neither).  m_run: the row's reference max in log2 units of the scaled
// scores; l_kept: its full sum of P over the kept keys (both lane halves);
// sink: the head's sink logit, or -inf without sinks.
//   n_split == 1: out = acc / (l_kept + exp2(sink - m)), converted to the
//     output type; with p.lse, the row's log-sum-exp (natural log, sink
//     excluded) = (m + log2 l_kept) ln 2.
//   n_split > 1: the workgroup's partial result for the merge kernel:
//     acc / l_kept in fp32 and m + log2 l_kept (log2 units), or 0 and -inf
//     when this part of the KV range kept no key of the row.
template <int D, bool XTRA, typename TI, typename TO>
__device__ __attribute__((always_inline)) void finish_row(const Params& p, const f32x16* acc,
                                                          float m_run, float l_kept,
                                  float sink, int64_t tok, int head, int half) {
  constexpr int DB = D / 32;
  const float kNegInf = -__builtin_inff();
  const int64_t row = tok * p.h_q + head;
  const bool any = m_run != kNegInf;
  if (XTRA && p.n_split > 1) {
    const int64_t prow = (int64_t)blockIdx.y * p.ws_tokens * p.h_q + row;
    const float inv = any ? 1.f / l_kept : 0.f;
    float* o = p.ws_o + prow * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + half * 4;
        *reinterpret_cast<f32x4*>(o + d0) =
            f32x4{acc[db][i4 * 4 + 0] * inv, acc[db][i4 * 4 + 1] * inv,
                  acc[db][i4 * 4 + 2] * inv, acc[db][i4 * 4 + 3] * inv};
      }
    if (half == 0) p.ws_lse[prow] = any ? m_run + __builtin_amdgcn_logf(l_kept) : kNegInf;
    return;
  }
  float l_tot = l_kept;
  if (any) l_tot += __builtin_amdgcn_exp2f(sink * kLog2e - m_run);  // exp2(-inf) = 0: no sink
  const float inv = 1.f / fmaxf(l_tot, FLT_MIN);
  const int64_t ooff = row * D;
  if constexpr (sizeof(TO) == 4) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + half * 4;
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.out) + ooff + d0) =
            f32x4{acc[db][i4 * 4 + 0] * inv, acc[db][i4 * 4 + 1] * inv,
                  acc[db][i4 * 4 + 2] * inv, acc[db][i4 * 4 + 3] * inv};
      }
  } else {
    // In each 16-value run of d (db, k) the low lanes hold values 0-3 and
    // 8-11, the high lanes (same row) 4-7 and 12-15.  One v_permlane32_swap
    // per register gives the low lanes 8-15 and the high lanes 0-7, so each
    // lane stores 16 contiguous bytes: half as many store instructions, each
    // writing 32 contiguous bytes of every row it touches.
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int i0 = 8 * k, i1 = 8 * k + 4;
        const uint32_t w0a = TI::pack(acc[db][i0 + 0] * inv, acc[db][i0 + 1] * inv);
        const uint32_t w0b = TI::pack(acc[db][i0 + 2] * inv, acc[db][i0 + 3] * inv);
        const uint32_t w1a = TI::pack(acc[db][i1 + 0] * inv, acc[db][i1 + 1] * inv);
        const uint32_t w1b = TI::pack(acc[db][i1 + 2] * inv, acc[db][i1 + 3] * inv);
        // swap(x, y): x's high lanes <-> y's low lanes
        const auto sa = __builtin_amdgcn_permlane32_swap(w1a, w0a, false, false);
        const auto sb = __builtin_amdgcn_permlane32_swap(w1b, w0b, false, false);
        const int d0 = db * 32 + 16 * k + (half ? 0 : 8);
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(p.out) + ooff + d0) =
            u32x4{sa[0], sb[0], sa[1], sb[1]};
      }
  }
  if (XTRA && p.lse != nullptr && half == 0)
    p.lse[row] = any ? (m_run + __builtin_amdgcn_logf(l_kept)) * kLn2 : kNegInf;
}

// One visited-tile record (layout: attn_tile_log in attn_prefill.h) from
// the (first, last, count) triples of the NW = R * S waves that served one
// work item, wl[3 w .. 3 w + 2]: per wave its own three numbers, and for the
// work item the union of the waves' tiles.  Wave w serves row group w % R
// and takes every S-th tile of the range from its offset w / R, so the waves
// of one offset visit runs of one residue class: their union is counted by
// merging the R runs (sorted by first tile), two runs joining when the gap
// between them is at most S.  Row group r covers Q-tile rows
// [r ROWS_PER_WAVE, (r + 1) ROWS_PER_WAVE).
template <int R, int S, int ROWS_PER_WAVE = 32>
__device__ __attribute__((always_inline)) void store_tile_record(
    int32_t* rec, const int* wl, int slot, int h_first, int hpack, int q0, int q_last,
    int part, int n_parts) {
  constexpr int NW = R * S;
  static_assert(NW <= kLogMaxWaves, "record holds every wave");
  int t_first = 0x7fffffff, t_last = -1, n_visited = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    int a[R], b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int w = s * R + r;
      const bool any = wl[3 * w + 2] > 0;
      a[r] = any ? wl[3 * w + 0] : 0x7fffffff;
      b[r] = any ? wl[3 * w + 1] : -1;
    }
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int k = 0; k + 1 < R - i; ++k)
        if (a[k] > a[k + 1]) {
          const int ta = a[k], tb = b[k];
          a[k] = a[k + 1];
          b[k] = b[k + 1];
          a[k + 1] = ta;
          b[k + 1] = tb;
        }
    int lo = a[0], hi = b[0];
#pragma unroll
    for (int r = 1; r < R; ++r) {
      if (b[r] < 0) continue;  // empty (sorted last)
      if (a[r] <= hi + S) {
        hi = max(hi, b[r]);
      } else {
        n_visited += (hi - lo) / S + 1;
        lo = a[r];
        hi = b[r];
      }
    }
    if (hi >= 0) {
      n_visited += (hi - lo) / S + 1;
      t_first = min(t_first, a[0]);
      t_last = max(t_last, hi);
    }
  }
  rec[0] = slot;
  rec[1] = h_first;
  rec[2] = hpack;
  rec[3] = q0;
  rec[4] = q_last;
  rec[5] = n_visited > 0 ? t_first : -1;
  rec[6] = n_visited > 0 ? t_last : -1;
  rec[7] = n_visited;
  rec[8] = NW;
  rec[9] = S;
  rec[10] = part;
  rec[11] = n_parts;
#pragma unroll
  for (int i = 13; i < 16; ++i) rec[i] = 0;
  rec[12] = ROWS_PER_WAVE;
#pragma unroll
  for (int w = 0; w < kLogMaxWaves; ++w) {
    rec[16 + 3 * w + 0] = w < NW ? wl[3 * w + 0] : -1;
    rec[16 + 3 * w + 1] = w < NW ? wl[3 * w + 1] : -1;
    rec[16 + 3 * w + 2] = w < NW ? wl[3 * w + 2] : 0;
  }
}

// Visited-tile record of one workgroup: each wave reports the first and last
// tile whose scores it used and how many; the waves meet in LDS and thread 0
// writes the record (store_tile_record).
template <int R, int S, int ROWS_PER_WAVE = 32>
__device__ __attribute__((always_inline)) void write_tile_log(const Params& p, void* lds_raw,
                                                              int wave, int v_first, int v_last,
                               int v_count, int slot, int h_first, int q0, int q_last) {
  int* wl = reinterpret_cast<int*>(lds_raw);
  __syncthreads();  // every LDS read of the epilogue has finished
  if ((threadIdx.x & 63) == 0) {
    wl[3 * wave + 0] = v_first;
    wl[3 * wave + 1] = v_last;
    wl[3 * wave + 2] = v_count;
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int32_t* rec = p.log + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kLogFields;
  store_tile_record<R, S, ROWS_PER_WAVE>(rec, wl, slot, h_first, p.hpack, q0, q_last,
                                         blockIdx.y, gridDim.y);
}

// This workgroup's part of the Q tile's KV tiles [t_lo, t_hi] when the range
// is cut into p.n_split contiguous parts (blockIdx.y); may come out empty.
__device__ __attribute__((always_inline)) void split_range(const Params& p, int* t_lo, int* t_hi) {
  if (p.n_split <= 1) return;
  const int per = (*t_hi - *t_lo + p.n_split) / p.n_split;  // ceil(tiles / n_split)
  const int lo = *t_lo + (int)blockIdx.y * per;
  *t_hi = min(*t_hi, lo + per - 1);
  *t_lo = lo;
}

// Workgroup = R row groups x S KV splits of one wave each.  Row group rg owns
// 32 Q-tile rows; split sp takes every S-th KV tile of the workgroup's range,
// so the S waves of a row group (two per SIMD) work on different tiles at
// once and are merged through LDS at the end.  K/V of the S tiles of one
// stage sit in one LDS slot of a 3- or 4-slot ring: while stage j is
// consumed, stage j + 1 is resident and stage j + 2 (and j + 3) is loaded by
// direct global -> LDS loads, with one barrier per stage.
//
// Each wave runs its tiles as a two-phase software pipeline:
//   phase A  MFMA: S_{i+1} = K_{i+1} . Q^T      VALU: P_i = exp2(S_i), 16-bit
//                                                    pack, row sums
//   phase B  MFMA: O^T += V_i^T . P_i^T          VALU: mask S_{i+1} (boundary
//                                                    tiles), its max, the
//                                                    rescale test
// so matrix and vector work of neighbouring tiles overlap inside the wave.
template <int D, int BKV, int R, int S_REQ, int NSLOT, bool WIN, bool XTRA, typename TI,
          typename TO>
// At least two waves per SIMD for d <= 128 (registers capped at 256 per
// wave): the small-tile configurations serve latency-bound calls (window
// chunks, decode rows, short ragged sequences), where a second resident wave
// hides more of each load than the registers it gives up would buy.  At
// d = 256 the accumulators alone need one wave per SIMD.
__global__ __launch_bounds__(R * (D >= 128 ? 1 : S_REQ) * 64, (D <= 128 ? 2 : 1)) void attn_fwd_kernel(Params p) {
  // stages of two 64-key d=128 tiles would not fit in LDS: d >= 128 uses one
  // split (and d = 256 32-key tiles, chosen by its launcher)
  constexpr int S = (D >= 128) ? 1 : S_REQ;
  constexpr int NW = R * S;
  constexpr int NT = NW * 64;
  static_assert(NSLOT == 3 || NSLOT == 4, "LDS ring of 3 or 4 stages");
  constexpr int DCH = D / 8;                // 16-byte chunks per K/V row
  constexpr int TILE_CH = BKV * DCH;        // chunks of one K (or V) tile
  constexpr int STAGE_CH = 2 * S * TILE_CH; // K and V of S tiles
  constexpr int KSTEPS = D / 16;            // MFMA k-steps of Q.K^T
  constexpr int NB = BKV / 32;              // 32-key blocks per KV tile
  constexpr int NG = BKV / 16;              // 16-key PV steps per KV tile
  constexpr int DB = D / 32;                // 32-wide d blocks of the output
  constexpr float kRescale = 8.f;           // lazy-rescale threshold (log2 units)
  static_assert(BKV % 32 == 0 && (D == 64 || D == 128 || D == 256), "tile shape");
  static_assert(S == 1 || S == 2, "1 or 2 KV splits");

  // Separate K and V rings of KD = NSLOT - 1 slots (S tiles each): the K of
  // stage s is read one step before its V (as the next tile's scores), so
  // each tensor is loaded exactly one step before its first reader and
  // neither ring needs a third slot.
  constexpr int KD = NSLOT - 1;
  constexpr int RING_CH = KD * S * TILE_CH;  // one tensor's ring
  __shared__ u32x4 lds[2 * RING_CH];         // K ring, then V ring

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep every
  // quantity derived from it in scalar registers and branch on it with SALU
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % R;
  const int sp = wave / R;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work item: (KV head, head group, Q tile), heaviest Q tiles first ----
  const WorkItem wi = decode_item<XTRA, D == 64>(p, blockIdx.x);
  const int g = wi.g, hg = wi.hg, bi = wi.bi;
  const int sq = wi.sq, past = wi.past, slot = wi.slot;
  const int64_t tok0 = wi.tok0;
  const int q0 = wi.q0;
  const int q_last = min(q0 + p.q_rows, sq) - 1;
  const int skv = past + sq;
  const int window = WIN ? p.window : 0;  // compile-time 0 for full attention

  // KV tiles of the whole Q tile: floor from the first row, ceiling from the last
  const int lo_key = window > 0 ? max(0, past + q0 - window + 1) : 0;
  int t_lo = lo_key / BKV;
  // non-causal (split/lse variant only): every row keeps every key of its
  // sequence above the window floor, so the ceiling is the last key's tile
  const bool causal = !XTRA || p.causal;
  int t_hi = (causal ? past + q_last : skv - 1) / BKV;
  if constexpr (XTRA) split_range(p, &t_lo, &t_hi);
  const int n_stages = max(0, (t_hi - t_lo + S) / S);

  // ---- this lane's row ----
  const int row = rg * 32 + col;
  const int pos = q0 + row / p.hpack;
  const int head = g * p.group + hg * p.hpack + row % p.hpack;
  const bool valid = pos < sq;
  const int row_hi = causal ? past + pos : skv - 1;           // last kept key
  const int row_lo = window > 0 ? past + pos - window + 1 : 0;  // first kept key

  // ---- this row group's rows: skip tiles none of them keeps ----
  const int wp0 = q0 + (rg * 32) / p.hpack;
  const int wp1 = min(q0 + (rg * 32 + 31) / p.hpack, sq - 1);
  const bool wave_live = wp0 < sq;
  const int w_lo = window > 0 ? max(0, past + wp0 - window + 1) / BKV : 0;
  const int w_hi = (causal ? past + wp1 : skv - 1) / BKV;
  const int w_full_lo = window > 0 ? past + wp1 - window + 1 : 0;  // max row lower bound
  const int w_full_hi = causal ? past + wp0 : skv - 1;              // min row upper bound

  const float c = p.scale_log2;
  const float kNegInf = -__builtin_inff();

  // ---- Q^T fragments (B operand), held for the whole KV loop; loaded
  // here without a branch (rows past the chunk read its last row), then
  // zeroed where invalid and pre-scaled once the first K/V loads are also in
  // flight, so that the two round trips overlap ----
  u32x4 qf[KSTEPS];
  {
    const int64_t qoff = ((tok0 + (valid ? pos : sq - 1)) * p.h_q + head) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = load16<TI>(p.q, qoff + kk * 16);
  }
  // the row's sink, read now (no branch, no use before the epilogue) so
  // that its latency hides behind the KV loop
  const float sink = load_sink(p.sink, head);

  // Token-pool layout (split/lse variant only): key k of this sequence is
  // pool row kv_list[k], rows h_kv * d elements apart; otherwise the dense
  // cache of this sequence's slot and KV head.
  const bool paged = XTRA && p.kv_idx != nullptr;
  const int32_t* kv_list = paged ? p.kv_idx + wi.kv_start : nullptr;
  const int64_t kv_base =
      paged ? (int64_t)g * D : ((int64_t)slot * p.h_kv + g) * (int64_t)p.s_cap * D;
  const uint16_t* kptr = reinterpret_cast<const uint16_t*>(p.k) + kv_base;
  const uint16_t* vptr = reinterpret_cast<const uint16_t*>(p.v) + kv_base;

  // ---- direct global -> LDS loads, one step's worth per call ----
  // A step moves 2S tile-tensors ((split, K|V)) of TILE_CH 16-byte chunks --
  // the K tiles of one stage and the V tiles of the stage before it -- as
  // 1-KB global_load_lds_dwordx4 loads (lane i's 16 bytes land at the load's
  // LDS base + 16 i); wave w issues loads w * LD_PER_WAVE + i.
  // Lane l of a load fills chunk 64 * block + l of its tile-tensor: key
  // (64 * block + l) / DCH, physical chunk l % DCH, so it fetches logical
  // chunk physical ^ swizzle(key).  Rows at or past skv are read from row
  // skv - 1 (finite data whose scores the causal mask removes, p = 0).
  constexpr int LD_PER_WAVE = STAGE_CH / 64 / NW;
  static_assert(STAGE_CH % (64 * NW) == 0 && TILE_CH % 64 == 0, "direct loads tile the stage");
  // with a 4-slot ring the waits let one step's loads stay in flight, which
  // needs every wave's loads of a step to be of one tensor (K or V)
  static_assert(NSLOT == 3 || (TILE_CH / 64) % LD_PER_WAVE == 0, "one tensor per wave");
  // this lane's key and byte offset inside its tile for each of the wave's
  // loads (the same every stage)
  int ld_key[LD_PER_WAVE];
  uint32_t ld_off[LD_PER_WAVE];
#pragma unroll
  for (int i = 0; i < LD_PER_WAVE; ++i) {
    const int qi = wave * LD_PER_WAVE + i;
    const int tt = qi / (TILE_CH / 64);
    const int chunk = (qi % (TILE_CH / 64)) * 64 + lane;
    const int key = chunk / DCH;
    const int pch = chunk % DCH;
    const int ch = (tt & 1) ? v_chunk<D>(key, pch) : k_chunk<D>(key, pch);
    ld_key[i] = key;
    ld_off[i] = (uint32_t)(key * D + ch * 8) * 2u;
  }
  // A split whose tile lies past t_hi in the last stage gets tile t_hi
  // instead: every slot a wave reads then holds finite cache data, which
  // matters because a wave without a tile still multiplies P = 0 by V.
  const uint32_t lds_addr = lds_byte_addr(lds);
  // Each step loads this wave's pieces of a stage's K / V tile-tensors:
  // K pieces of stage kst, V pieces of stage vst (a negative stage: none).
  auto piece_is_v = [&](int i) __attribute__((always_inline)) { return (((wave * LD_PER_WAVE + i) / (TILE_CH / 64)) & 1) != 0; };
  auto piece_stage = [&](int i, int kst, int vst) __attribute__((always_inline)) { return piece_is_v(i) ? vst : kst; };
  // Token-pool layout: the pool row of each of this lane's keys in the next
  // loads, read one step ahead so that the index latency hides behind the
  // step before it (keys past the sequence read row skv - 1).
  uint32_t prow[LD_PER_WAVE];
  auto piece_key = [&](int i, int stage) __attribute__((always_inline)) {
    const int tt = (wave * LD_PER_WAVE + i) / (TILE_CH / 64);
    const int t = min(t_lo + max(stage, 0) * S + (tt >> 1), t_hi);
    return min(t * BKV + ld_key[i], skv - 1);
  };
  auto fetch_rows = [&](int kst, int vst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i)
      prow[i] = (uint32_t)kv_list[piece_key(i, piece_stage(i, kst, vst))];
  };
  auto load_kv = [&](int kst, int vst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LD_PER_WAVE; ++i) {
      const int qi = wave * LD_PER_WAVE + i;
      const int tt = qi / (TILE_CH / 64);      // tile-tensor: 2 * split + (0 K, 1 V)
      const int blk = qi % (TILE_CH / 64);
      const int stage = (tt & 1) ? vst : kst;
      if (stage < 0) continue;
      const uint32_t lds_dst =
          lds_addr + (uint32_t)((tt & 1) * RING_CH + (stage % KD) * S * TILE_CH +
                                (tt >> 1) * TILE_CH + blk * 64) * 16u;
      if (paged) {
        // pool row (clamped into the pool) + this lane's chunk of the row
        const uint32_t r = min(prow[i], p.n_pool - 1u);
        lds_dma16((tt & 1) ? vptr : kptr,
                  r * p.kv_row_bytes + ld_off[i] - (uint32_t)ld_key[i] * (D * 2), lds_dst);
        continue;
      }
      const int t = min(t_lo + stage * S + (tt >> 1), t_hi);
      const char* tile = reinterpret_cast<const char*>((tt & 1) ? vptr : kptr) +
                         (int64_t)t * (BKV * D * 2);
      uint32_t voff = ld_off[i];
      if (t * BKV + BKV > skv) {
        // the tile that crosses the end of the sequence: clamp rows to skv - 1
        const int row = min(ld_key[i], skv - 1 - t * BKV);
        voff -= (uint32_t)(ld_key[i] - row) * (D * 2);
      }
      lds_dma16(tile, voff, lds_dst);
    }
  };
  // does this wave issue any piece for (kst, vst)?  (its pieces are of one
  // tensor whenever the answer decides a wait)
  auto issues = [&](int kst, int vst) __attribute__((always_inline)) { return piece_is_v(0) ? vst >= 0 : kst >= 0; };
  // wait until every load but this step's newest ones has landed in LDS
  // (`newest`: whether this wave issued loads in this step)
  auto wait_older = [&](bool newest) __attribute__((always_inline)) {
    if (NSLOT == 4 && newest)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LD_PER_WAVE));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };

  // Running state per row (this lane's query).  m_run is the reference max
  // of the scaled scores in log2 units: exact when first set, afterwards
  // raised only when a tile's max exceeds it by more than kRescale, so
  // p = exp2(s - m_run) <= 2^kRescale always fits 16 bits.
  float m_run = kNegInf;
  float l_run = 0.f;      // this lane's partial denominator (relative to m_run)
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_use = 0.f;      // m_run, or 0 while m_run = -inf
  f32x16 negm = f32x16{}; // splat(-m_use): MFMA accumulator input (prescaled-Q path)

  // tile this wave handles at stage j (if any)
  auto wave_tile = [&](int j, int* t) __attribute__((always_inline)) {
    *t = t_lo + j * S + sp;
    return wave_live && j < n_stages && *t <= t_hi && *t >= w_lo && *t <= w_hi;
  };

  // S^T of tile t from stage slot `st`, in exp2 units relative to m_use, masked
  auto scores = [&](const u32x4* kt, int t, f32x16* sc) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int kr = nb * 32 + col;
      if constexpr (TI::kPrescaleQ)
        sc[nb] = TI::mma(kt[kr * DCH + k_chunk<D>(kr, half)], qf[0], negm);
      else
        sc[nb] = TI::mma(kt[kr * DCH + k_chunk<D>(kr, half)], qf[0], f32x16{});
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk)
        sc[nb] = TI::mma(kt[kr * DCH + k_chunk<D>(kr, 2 * kk + half)], qf[kk], sc[nb]);
    }
  };
  // bf16 path: scores to exp2 units relative to m_use (fp16 path: already)
  auto to_exp2_units = [&](f32x16* sc) __attribute__((always_inline)) {
    if constexpr (!TI::kPrescaleQ) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[nb][i] = __builtin_fmaf(sc[nb][i], c, -m_use);
    }
  };
  // row max of a tile (v_maximum3_f32 tree; IEEE maximum needs no NaN
  // canonicalisation), combined over the two lane halves
  auto row_max = [&](const f32x16* sc) __attribute__((always_inline)) {
    float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; i += 2)
        m4[(i >> 1) & 3] = vmax(m4[(i >> 1) & 3], vmax(sc[nb][i], sc[nb][i + 1]));
    return pair_max(vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3])));
  };
  // is tile t free of masked (row, key) pairs for every row of this wave?
  auto interior = [&](int t) __attribute__((always_inline)) {
    const int kbase = t * BKV;
    return (kbase + BKV - 1 <= w_full_hi) && (kbase >= w_full_lo);
  };
  auto apply_mask = [&](int t, f32x16* sc) __attribute__((always_inline)) {
    const int kbase = t * BKV;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + nb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        if (key > row_hi || key < row_lo) sc[nb][i] = kNegInf;
      }
  };
  // masked, exp2-unit scores and their row max
  auto prepare = [&](int t, f32x16* sc) __attribute__((always_inline)) {
    to_exp2_units(sc);
    if (!interior(t)) apply_mask(t, sc);
    return row_max(sc);
  };
  auto set_neg_inf = [&](f32x16* sc) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[nb][i] = kNegInf;
  };
  // raise the reference max if the tile needs it (wave-uniform branch);
  // acc must not have pending PV work of an older tile when this runs
  auto rebase = [&](float mx, f32x16* sc) __attribute__((always_inline)) {
    const bool need = (mx > kRescale) || (m_run == kNegInf && mx != kNegInf);
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mx_abs = mx + m_use;  // -inf stays -inf
      const float m_new = fmaxf(m_run, mx_abs);
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_run = m_new;
      const float m_use_new = (m_new == kNegInf) ? 0.f : m_new;
      const float shift = m_use - m_use_new;
      m_use = m_use_new;
#pragma unroll
      for (int i = 0; i < 16; ++i) negm[i] = -m_use;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[nb][i] += shift;
    }
  };

  // The tiles whose scores this wave actually uses (visited-tile record):
  // noted where the softmax consumes a tile, not derived from the bounds.
  int v_first = -1, v_last = -1, v_count = 0;
  auto note = [&](int t) __attribute__((always_inline)) {
    if (v_count == 0) v_first = t;
    v_last = t;
    ++v_count;
  };

  // ---- prologue: K of stages 0 .. KD-1 and V of stages 0 .. KD-2 (the
  // first K and V always, later ones if the stage exists); then every one
  // but the last step's is resident, and S of the wave's first tile ----
  auto pro_k = [&](int s2) __attribute__((always_inline)) { return (s2 == 0 || s2 < n_stages) ? s2 : -1; };
  auto pro_v = [&](int s2) __attribute__((always_inline)) { return (s2 == 1 || (s2 >= 1 && s2 - 1 < n_stages)) ? s2 - 1 : -1; };
  if (paged) {
    // the pool rows of the first steps are read together, then each step's
    // loads are issued (one index round trip instead of one per step)
    uint32_t pre[KD][LD_PER_WAVE];
#pragma unroll
    for (int s2 = 0; s2 < KD; ++s2)
#pragma unroll
      for (int i = 0; i < LD_PER_WAVE; ++i)
        pre[s2][i] = (uint32_t)kv_list[piece_key(i, piece_stage(i, pro_k(s2), pro_v(s2)))];
#pragma unroll
    for (int s2 = 0; s2 < KD; ++s2) {
#pragma unroll
      for (int i = 0; i < LD_PER_WAVE; ++i) prow[i] = pre[s2][i];
      load_kv(pro_k(s2), pro_v(s2));
    }
    fetch_rows(KD < n_stages ? KD : -1, KD - 1 < n_stages ? KD - 1 : -1);
  } else {
#pragma unroll
    for (int s2 = 0; s2 < KD; ++s2) load_kv(pro_k(s2), pro_v(s2));
  }
  prepare_q<TI, KSTEPS>(qf, c, valid);
  wait_older(issues(pro_k(KD - 1), pro_v(KD - 1)));
  __syncthreads();

  f32x16 s_a[NB], s_b[NB];   // scores of the current / next tile, roles alternate
  int t_cur = 0;
  if (wave_tile(0, &t_cur)) {
    note(t_cur);
    scores(lds + sp * TILE_CH, t_cur, s_a);
    const float mx = prepare(t_cur, s_a);
    rebase(mx, s_a);
  } else {
    set_neg_inf(s_a);
  }

  // P = exp2(S) of the current tile, 16-bit; returns this lane's row sum
  auto make_p = [&](const f32x16* s_cur, u32x4* pb, u32x4* pl) __attribute__((always_inline)) {
    float rs = 0.f;
#pragma unroll
    for (int g16 = 0; g16 < NG; ++g16)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = (g16 & 1) * 8 + w * 2;
        const float p0 = __builtin_amdgcn_exp2f(s_cur[g16 >> 1][i]);
        const float p1 = __builtin_amdgcn_exp2f(s_cur[g16 >> 1][i + 1]);
        const uint32_t hi = TI::pack(p0, p1);
        pb[g16][w] = hi;
        if constexpr (TI::kSplitP) {
          pl[g16][w] = TI::pack(TI::lo_part(p0, hi, 0), TI::lo_part(p1, hi, 1));
          rs += p0 + p1;
        } else {
          rs = TI::rowsum(hi, rs);
        }
      }
    return rs;
  };
  auto pv = [&](const u32x4* vt, const u32x4* pb, const u32x4* pl) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g16 = 0; g16 < NG; ++g16) {
        const u32x4 a = v_frag<D>(vt, g16, db, lane);
        acc[db] = TI::mma(a, pb[g16], acc[db]);
        if constexpr (TI::kSplitP) acc[db] = TI::mma(a, pl[g16], acc[db]);
      }
  };

  auto stage_step = [&](int j, f32x16* s_cur, f32x16* s_nxt) __attribute__((always_inline)) {
    // K of stage j + KD (first read by step j + KD - 1) and V of stage
    // j + KD - 1 (read by that same step); their slots' last readers were
    // steps j - 1 (K) and j - 1 (V)
    const int kst = j + KD < n_stages ? j + KD : -1;
    const int vst = j + KD - 1 < n_stages ? j + KD - 1 : -1;
    const bool newest = issues(kst, vst);
    load_kv(kst, vst);
    if (paged) fetch_rows(j + 1 + KD < n_stages ? j + 1 + KD : -1, j + KD < n_stages ? j + KD : -1);

    int t_nxt = 0;
    const bool nxt_ok = wave_tile(j + 1, &t_nxt);
    const u32x4* k_nxt_slot = lds + ((j + 1) % KD) * S * TILE_CH + sp * TILE_CH;
    const u32x4* vt = lds + RING_CH + (j % KD) * S * TILE_CH + sp * TILE_CH;
    // One straight-line body for every stage (no branch on whether this wave
    // has a current or a next tile), so that the scheduler can interleave
    //   S_{i+1} (MFMA) || P_i (VALU);  PV_i (MFMA) || max of S_{i+1} (VALU)
    // and the accumulators keep one register assignment.  Without a next
    // tile the scores come from a resident (stale) slot and are replaced by
    // -inf, so that the following stage's P is exactly zero and its PV and
    // row sum add nothing.
    u32x4 pb[NG];
    u32x4 pl[NG];
    scores(k_nxt_slot, t_nxt, s_nxt);
    l_run += make_p(s_cur, pb, pl);
    pv(vt, pb, pl);
    to_exp2_units(s_nxt);
    float mx = row_max(s_nxt);
    if (nxt_ok) {
      note(t_nxt);
      // boundary tile: mask, then the max of what is kept (rare)
      if (!interior(t_nxt)) {
        apply_mask(t_nxt, s_nxt);
        mx = row_max(s_nxt);
      }
      rebase(mx, s_nxt);
    } else {
      set_neg_inf(s_nxt);
    }

    wait_older(newest);  // K of stage j + 2 and V of stage j + 1 landed in LDS
    __syncthreads();
  };

  for (int j = 0; j < n_stages; j += 2) {
    stage_step(j, s_a, s_b);
    if (j + 1 < n_stages) stage_step(j + 1, s_b, s_a);
  }

  // ---- merge the KV splits of each row group through LDS ----
  if constexpr (S > 1) {
    constexpr int NV = 2 + 16 * DB;
    static_assert(R * NV * 64 * 4 <= 2 * RING_CH * 16, "the merge fits the rings' LDS");
    float* mb = reinterpret_cast<float*>(lds);
    if (sp == 1) {
      float* dst = mb + rg * NV * 64 + lane;
      dst[0] = m_run;
      dst[64] = l_run;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(2 + db * 16 + i) * 64] = acc[db][i];
    }
    __syncthreads();
    if (sp == 0) {
      const float* src = mb + rg * NV * 64 + lane;
      const float m1 = src[0], l1 = src[64];
      const float m = fmaxf(m_run, m1);
      const float a0 = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      l_run = a0 * l_run + a1 * l1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[db][i] = a0 * acc[db][i] + a1 * src[(2 + db * 16 + i) * 64];
      m_run = m;
    }
  }

  // ---- epilogue: combine lane halves, fold the sink, normalise, store ----
  if (sp == 0) {
    const float l_kept = l_run + other_half(l_run);
    if (valid) finish_row<D, XTRA, TI, TO>(p, acc, m_run, l_kept, sink, tok0 + pos, head, half);
  }

  if (p.log != nullptr)
    write_tile_log<R, S>(p, lds, wave, v_first, v_last, v_count, slot, g * p.group + hg * p.hpack,
                         q0, q_last);
}

// ---------------------------------------------------------------------------
// Ping-pong variant: 8 waves = 2 groups x 4 row groups.  Group g (= KV split
// g) takes tiles t_lo + 2 j + g.  Each wave alternates two phases separated
// by workgroup barriers:
//   M_j  matrix work:  S_{j+1} = K_{j+1} . Q^T  and  O^T += V_j^T . P_j^T
//        from fragments already in registers, each fragment register
//        refilled (LDS reads of K_{j+2} and V_{j+1}) after the MFMA that
//        follows its reader; then the direct loads of tile j + NS;
//   V_j  vector work:  P_{j+1} = exp2(S_{j+1}) packed to 16 bits and its row
//        sums (boundary and early tiles: mask, row max and lazy rescale
//        first; interior tiles in the fast loop: P at once, the reference
//        raised only when the tile's P sum says so); the waits for the next
//        tiles and for this wave's fragment reads.
// Group 1 starts one phase late, so on every SIMD (one wave of each group)
// one wave's MFMA burst runs beside the other wave's exp2 / VALU burst.
// Each group owns an NS-slot ring of (K, V) tiles in LDS, filled by its own
// four waves.
template <int D, int BKV_REQ, int NS_REQ, bool WIN, bool XTRA, typename TI, typename TO>
__global__ __launch_bounds__(512) void attn_pp_kernel(Params p) {
  constexpr int BKV = (D == 128) ? 32 : BKV_REQ;  // ring of 2 x NS tiles must fit LDS
  constexpr int NS = (D == 128) ? 4 : NS_REQ;      // (a 5-deep ring spills at d = 128)
  constexpr int R = 4;                      // row groups (waves) per group
  constexpr int DCH = D / 8;
  constexpr int TILE_CH = BKV * DCH;        // 16-byte chunks of one K (or V) tile
  constexpr int SLOT_CH = 2 * TILE_CH;      // K and V of one tile
  constexpr int GROUP_CH = NS * SLOT_CH;    // one group's ring
  constexpr int KSTEPS = D / 16;
  constexpr int NB = BKV / 32;
  constexpr int NG = BKV / 16;
  constexpr int DB = D / 32;
  constexpr int LPW = SLOT_CH / 64 / R;     // 1-KB direct loads per wave per tile
  constexpr float kRescale = 8.f;
  constexpr float kTileSumMax = 1024.f;  // fast-path bound on a tile's P sum per lane
  static_assert(NS == 4 || NS == 5, "ring of 4 or 5 tiles per group");
  static_assert(NB <= 2, "one -m splat per 32-key block (negm, negm1)");
  static_assert(SLOT_CH % (64 * R) == 0, "direct loads tile a slot");
  static_assert(2 * GROUP_CH * 16 + (XTRA ? 2 * NS * 64 * 4 : 0) <= 160 * 1024, "LDS");
  // the token-pool row lists run two tiles ahead of the loads that use them,
  // which the waits below count for a 4-deep ring
  static_assert(!XTRA || NS == 4, "split/lse variant: ring of 4 tiles per group");

  __shared__ u32x4 lds[2 * GROUP_CH];
  // Token-pool layout (split/lse variant): each group's ring of the pool rows
  // of its tiles' keys, 64 words a slot (tile j of the group in slot j % NS)
  __shared__ int32_t kidx[XTRA ? 2 * NS * 64 : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % R;
  const int grp = wave / R;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- work item: (KV head, head group, Q tile), heaviest Q tiles first ----
  const WorkItem wi = decode_item<XTRA, D == 64>(p, blockIdx.x);
  const int g = wi.g, hg = wi.hg, bi = wi.bi;
  const int sq = wi.sq, past = wi.past, slot = wi.slot;
  const int64_t tok0 = wi.tok0;
  const int q0 = wi.q0;
  const int q_last = min(q0 + p.q_rows, sq) - 1;
  const int skv = past + sq;
  const int window = WIN ? p.window : 0;

  const int lo_key = window > 0 ? max(0, past + q0 - window + 1) : 0;
  int t_lo = lo_key / BKV;
  // non-causal (split/lse variant only): every row keeps every key of its
  // sequence above the window floor, so the ceiling is the last key's tile
  const bool causal = !XTRA || p.causal;
  int t_hi = (causal ? past + q_last : skv - 1) / BKV;
  if constexpr (XTRA) split_range(p, &t_lo, &t_hi);
  const int n_stages = max(0, (t_hi - t_lo + 2) / 2);  // group 0's tiles (group 1: same or one fewer)

  const int row = rg * 32 + col;
  const int pos = q0 + row / p.hpack;
  const int head = g * p.group + hg * p.hpack + row % p.hpack;
  const bool valid = pos < sq;
  const int row_hi = causal ? past + pos : skv - 1;
  const int row_lo = window > 0 ? past + pos - window + 1 : 0;

  const int wp0 = q0 + (rg * 32) / p.hpack;
  const int wp1 = min(q0 + (rg * 32 + 31) / p.hpack, sq - 1);
  const bool wave_live = wp0 < sq;
  const int w_lo = window > 0 ? max(0, past + wp0 - window + 1) / BKV : 0;
  const int w_hi = (causal ? past + wp1 : skv - 1) / BKV;
  const int w_full_lo = window > 0 ? past + wp1 - window + 1 : 0;
  const int w_full_hi = causal ? past + wp0 : skv - 1;

  const float c = p.scale_log2;
  const float kNegInf = -__builtin_inff();

  // Q^T fragments, loaded without a branch (rows past the chunk read its
  // last row), zeroed and pre-scaled once the first tiles' loads are in flight
  u32x4 qf[KSTEPS];
  {
    const int64_t qoff = ((tok0 + (valid ? pos : sq - 1)) * p.h_q + head) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = load16<TI>(p.q, qoff + kk * 16);
  }
  // the row's sink, read now (no branch, no use before the epilogue)
  const float sink = load_sink(p.sink, head);

  // Token-pool layout (split/lse variant only): key k of this sequence is
  // pool row kv_list[k], rows h_kv * d elements apart; otherwise the dense
  // cache of this sequence's slot and KV head.
  const bool paged = XTRA && p.kv_idx != nullptr;
  const int32_t* kv_list = paged ? p.kv_idx + wi.kv_start : nullptr;
  const int64_t kv_base =
      paged ? (int64_t)g * D : ((int64_t)slot * p.h_kv + g) * (int64_t)p.s_cap * D;
  const uint16_t* kptr = reinterpret_cast<const uint16_t*>(p.k) + kv_base;
  const uint16_t* vptr = reinterpret_cast<const uint16_t*>(p.v) + kv_base;
  u32x4* const ring = lds + grp * GROUP_CH;
  // LDS byte address of the ring (cast once: the generic -> LDS cast carries
  // a null check that per-load casts would repeat)
  const uint32_t ring_addr = lds_byte_addr(ring);

  // ---- direct loads of one tile of this group: wave rg issues loads
  // rg * LPW + i of the slot's 2 * TILE_CH / 64 one-KB pieces (K then V) ----
  int ld_key[LPW];
  uint32_t ld_off[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int qi = rg * LPW + i;
    const int tt = qi / (TILE_CH / 64);
    const int chunk = (qi % (TILE_CH / 64)) * 64 + lane;
    const int key = chunk / DCH;
    const int pch = chunk % DCH;
    const int ch = tt ? v_chunk<D>(key, pch) : k_chunk<D>(key, pch);
    ld_key[i] = key;
    ld_off[i] = (uint32_t)(key * D + ch * 8) * 2u;
  }
  // A group-local index past the group's last tile loads tile t_hi instead,
  // so every slot a wave reads holds finite cache data (a wave without a
  // tile still multiplies P = 0 by its V fragments).
  // Token-pool layout: the pool rows of tile j's keys (keys past the sequence
  // read row skv - 1).  Those of the prologue's tiles are read into registers
  // at once; every later tile's 64 rows are brought into its slot of the
  // group's LDS row ring by one 4-byte direct load per wave (each wave of the
  // group loads the same words), issued two tiles ahead of the tile's own
  // loads, so that the waits that land a tile also land the rows two tiles on
  // and no load waits for a register operand still in flight.
  auto tile_key = [&](int j, int i) __attribute__((always_inline)) {
    const int t = min(t_lo + 2 * j + grp, t_hi);
    return min(t * BKV + ld_key[i], skv - 1);
  };
  const uint32_t kidx_addr = lds_byte_addr(kidx) + (uint32_t)(grp * NS * 64) * 4u;
  auto fetch_idx = [&](int j) __attribute__((always_inline)) {
    const int t = min(t_lo + 2 * j + grp, t_hi);
    lds_dma4(kv_list, (uint32_t)min(t * BKV + lane, skv - 1) * 4u,
             kidx_addr + (uint32_t)((j % NS) * 64) * 4u);
  };
  // Token-pool layout: the pool row of this lane's piece i comes from
  // rows[i] (the prologue's registers) or, with rows = nullptr, from the
  // tile's slot of the LDS row ring.
  auto load_tile = [&](int j, const uint32_t* rows) __attribute__((always_inline)) {
    const int t = min(t_lo + 2 * j + grp, t_hi);
    const uint32_t st = ring_addr + (uint32_t)((j % NS) * SLOT_CH) * 16u;
    const bool tail = t * BKV + BKV > skv;  // the tile that crosses the end of the keys
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int qi = rg * LPW + i;
      const int tt = qi / (TILE_CH / 64);
      const int blk = qi % (TILE_CH / 64);
      if (paged) {
        // pool row (clamped into the pool) + this lane's chunk of the row
        const uint32_t row =
            rows ? rows[i] : (uint32_t)kidx[(grp * NS + j % NS) * 64 + ld_key[i]];
        const uint32_t r = min(row, p.n_pool - 1u);
        lds_dma16(tt ? vptr : kptr, r * p.kv_row_bytes + ld_off[i] - (uint32_t)ld_key[i] * (D * 2),
                  st + (uint32_t)(tt * TILE_CH + blk * 64) * 16u);
        continue;
      }
      const char* tile = reinterpret_cast<const char*>(tt ? vptr : kptr) + (int64_t)t * (BKV * D * 2);
      uint32_t voff = ld_off[i];
      if (tail) {
        const int r = min(ld_key[i], skv - 1 - t * BKV);
        voff -= (uint32_t)(ld_key[i] - r) * (D * 2);
      }
      lds_dma16(tile, voff, st + (uint32_t)(tt * TILE_CH + blk * 64) * 16u);
    }
  };

  // Stage j < n_stages - 1 of this group: tile t_lo + 2 j + grp < t_hi, so
  // no clamp to t_hi and no key past the end of the keys (dense layout).
  auto load_inner_tile = [&](int j) __attribute__((always_inline)) {
    const int t = t_lo + 2 * j + grp;
    const uint32_t st = ring_addr + (uint32_t)((j % NS) * SLOT_CH) * 16u;
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int qi = rg * LPW + i;
      const int tt = qi / (TILE_CH / 64);
      const int blk = qi % (TILE_CH / 64);
      const char* tile = reinterpret_cast<const char*>(tt ? vptr : kptr) + (int64_t)t * (BKV * D * 2);
      lds_dma16(tile, ld_off[i], st + (uint32_t)(tt * TILE_CH + blk * 64) * 16u);
    }
  };

  auto wave_tile = [&](int j, int* t) __attribute__((always_inline)) {
    *t = t_lo + 2 * j + grp;
    return wave_live && j >= 0 && j < n_stages && *t <= t_hi && *t >= w_lo && *t <= w_hi;
  };
  // The tiles this wave visits that are interior (every key visible to every
  // row of the wave) form one run tf_lo .. tf_hi of tile indices (empty when
  // tf_hi < tf_lo); wave_tile holds on each of this group's tiles in it
  // (t_lo + grp <= t <= t_hi puts the stage in range).
  const int tf_lo = max(max(t_lo + grp, w_lo), (w_full_lo + BKV - 1) / BKV);
  const int tf_hi = min(min(t_hi, w_hi), (w_full_hi + 1) / BKV - 1);

  float m_run = kNegInf, m_use = 0.f;
  // splat(-m_use), the accumulator input of the first S MFMA of each 32-key
  // block; one copy per block, since an MFMA that reads its accumulator
  // input in place would otherwise make the compiler copy it every phase
  f32x16 negm = f32x16{};
  f32x16 negm1 = f32x16{};
  // Row sums of P.  fp16 inputs: the tile's four 16-key P vectors are added
  // as packed fp16 in the V phase (no sum exceeds 2^10: the V phase raises
  // the reference max otherwise; one rounding of 2^-11 relative per add) and
  // the four pre-added words are summed into l_vec with v_dot2c.  bf16
  // inputs: on the matrix pipe, where ones . P^T puts the sum of P over the
  // tile's keys in every element of the row's column, one MFMA per 16-key
  // step for each of P's two parts.
  f32x16 lsum = f32x16{};
  const u32x4 ones = {TI::kOnePair, TI::kOnePair, TI::kOnePair, TI::kOnePair};
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  f32x16 sc[NB];
  u32x4 kf[NB][KSTEPS];
  u32x4 vf[DB][NG];
  u32x4 pb[NG], pl[NG];
  u32x4 psum = {0, 0, 0, 0};  // fp16: the tile's P pre-added (see presum)
  float l_vec = 0.f;          // fp16: this lane's part of the row sum
  bool started = false;       // wave-uniform: every row holds a reference max
#pragma unroll
  for (int g16 = 0; g16 < NG; ++g16) {
    pb[g16] = u32x4{0, 0, 0, 0};
    pl[g16] = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int db = 0; db < DB; ++db) vf[db][g16] = u32x4{0, 0, 0, 0};
  }

  auto read_k = [&](int j) __attribute__((always_inline)) {
    const u32x4* kt = ring + (j % NS) * SLOT_CH;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
        const int kr = nb * 32 + col;
        kf[nb][kk] = kt[kr * DCH + k_chunk<D>(kr, 2 * kk + half)];
      }
  };
  auto read_v = [&](int j) __attribute__((always_inline)) {
    const u32x4* vt = ring + (j % NS) * SLOT_CH + TILE_CH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g16 = 0; g16 < NG; ++g16) vf[db][g16] = v_frag<D>(vt, g16, db, lane);
  };
  // M_j: S_{j+1} = K_{j+1} . Q^T from kf and O^T += V_j^T . P_j^T from vf,
  // refilling each fragment register from the next tile (kf <- K_{j+2},
  // vf <- V_{j+1}).  Each read follows the MFMA after the one that last reads
  // the register it refills, so a load never targets an operand of the MFMA
  // just issued; one or two LDS reads between consecutive MFMAs keep this
  // wave's issue slots busy while the matrix pipe runs, without the read
  // bursts that overflow the LDS command queue (four waves of a CU are in
  // this phase at once).
  auto m_phase = [&](int j) __attribute__((always_inline)) {
    const u32x4* kt = ring + ((j + 2) % NS) * SLOT_CH;
    const u32x4* vt = ring + ((j + 1) % NS) * SLOT_CH + TILE_CH;
    constexpr int kMfma = 0x008, kDsRead = 0x100;
    constexpr int PVM = TI::kSplitP ? 2 : 1;   // MFMAs per P.V step
    auto refill_k = [&](int i) __attribute__((always_inline)) {
      const int kk = i / NB, nb = i % NB;
      const int kr = nb * 32 + col;
      kf[nb][kk] = kt[kr * DCH + k_chunk<D>(kr, 2 * kk + half)];
    };
#pragma unroll
    for (int i = 0; i < NB * KSTEPS; ++i) {
      const int kk = i / NB, nb = i % NB;
      if (kk == 0)
        sc[nb] = TI::mma(kf[nb][0], qf[0], TI::kPrescaleQ ? (nb ? negm1 : negm) : f32x16{});
      else
        sc[nb] = TI::mma(kf[nb][kk], qf[kk], sc[nb]);
      if (i > 0) refill_k(i - 1);   // the previous MFMA's operand, never the one in flight
    }
#pragma unroll
    for (int g16 = 0; g16 < NG; ++g16) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        acc[db] = TI::mma(vf[db][g16], pb[g16], acc[db]);
        if constexpr (TI::kSplitP) acc[db] = TI::mma(vf[db][g16], pl[g16], acc[db]);
        if (g16 == 0 && db == 0) refill_k(NB * KSTEPS - 1);
        else if (db > 0) vf[db - 1][g16] = v_frag<D>(vt, g16, db - 1, lane);
      }
      if constexpr (TI::kSplitP) {
        lsum = TI::mma(ones, pb[g16], lsum);
        lsum = TI::mma(ones, pl[g16], lsum);
      }
      vf[DB - 1][g16] = v_frag<D>(vt, g16, DB - 1, lane);
    }
    // issue order as written: each read follows the MFMA after the one that
    // last reads the register it refills
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
#pragma unroll
    for (int i = 1; i < NB * KSTEPS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
#pragma unroll
    for (int g16 = 0; g16 < NG; ++g16) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        __builtin_amdgcn_sched_group_barrier(kMfma, PVM, 0);
        if (g16 == 0 && db == 0) __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
        else if (db > 0) __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
      }
      if (TI::kSplitP) __builtin_amdgcn_sched_group_barrier(kMfma, PVM, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
  };
  auto make_p = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int g16 = 0; g16 < NG; ++g16)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int i = (g16 & 1) * 8 + w * 2;
        const float p0 = __builtin_amdgcn_exp2f(sc[g16 >> 1][i]);
        const float p1 = __builtin_amdgcn_exp2f(sc[g16 >> 1][i + 1]);
        const uint32_t hi = TI::pack(p0, p1);
        pb[g16][w] = hi;
        if constexpr (TI::kSplitP)
          pl[g16][w] = TI::pack(TI::lo_part(p0, hi, 0), TI::lo_part(p1, hi, 1));
      }
  };
  // in-lane part of the row max (the other 16 keys of each row are in lane ^ 32)
  auto lane_max = [&]() __attribute__((always_inline)) {
    float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; i += 2)
        m4[(i >> 1) & 3] = vmax(m4[(i >> 1) & 3], vmax(sc[nb][i], sc[nb][i + 1]));
    return vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3]));
  };
  auto apply_mask = [&](int t) __attribute__((always_inline)) {
    const int kbase = t * BKV;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kbase + nb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
        if (key > row_hi || key < row_lo) sc[nb][i] = kNegInf;
      }
  };

  // The tiles whose scores this wave actually uses (visited-tile record)
  int v_first = -1, v_last = -1, v_count = 0;
  auto note = [&](int t) __attribute__((always_inline)) {
    if (v_count == 0) v_first = t;
    v_last = t;
    ++v_count;
  };

  // One V phase: softmax of S_{j+1} into P_{j+1}.  P is formed against the
  // current reference max first; only when some row's max moved past the
  // threshold (rare: early tiles, rising scores) is the reference raised,
  // O and l rescaled and P formed again.
  // fp16: the tile's four 16-key P vectors added as packed fp16 (whole-vector
  // adds); the four pre-added words give the row sum (v_dot2c)
  auto presum = [&]() __attribute__((always_inline)) {
    if constexpr (!TI::kSplitP) {
      f16x8 sum = __builtin_bit_cast(f16x8, pb[0]);
#pragma unroll
      for (int g2 = 1; g2 < NG; ++g2) sum += __builtin_bit_cast(f16x8, pb[g2]);
      psum = __builtin_bit_cast(u32x4, sum);
    }
  };
  // Raise the reference max to the tile's row max where it exceeds it by more
  // than kRescale (or where the row had none), rescaling O and l, then form P
  // again; `mx` is the row max of S relative to the current reference.
  auto rescale = [&](float mx) __attribute__((always_inline)) {
    const float mx_abs = mx + m_use;
    const float m_new = fmaxf(m_run, mx_abs);
    const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    lsum *= alpha;
    l_vec *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    m_run = m_new;
    const float m_use_new = (m_new == kNegInf) ? 0.f : m_new;
    const float shift = m_use - m_use_new;
    m_use = m_use_new;
#pragma unroll
    for (int i = 0; i < 16; ++i) negm[i] = -m_use;
    negm1 = negm;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[nb][i] += shift;
    make_p();
  };

  // One V phase: softmax of S_{j+1} into P_{j+1} (the general path: boundary
  // tiles, a wave's first tiles, bf16, and iterations outside the steady
  // run): mask, the row max over both lane halves, and a raise of the
  // reference when some row's max exceeds it by more than kRescale or a row
  // had none.
  auto v_phase = [&](int j) __attribute__((always_inline)) {
    int t = 0;
    if (wave_tile(j + 1, &t)) {
      note(t);
      const bool inner = (t * BKV + BKV - 1 <= w_full_hi) && (t * BKV >= w_full_lo);
      if constexpr (!TI::kPrescaleQ) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[nb][i] = __builtin_fmaf(sc[nb][i], c, -m_use);
      }
      if (!inner) apply_mask(t);
      const float mx = pair_max(lane_max());
      make_p();
      presum();
      if (__builtin_amdgcn_ballot_w64((mx > kRescale) || (m_run == kNegInf && mx != kNegInf))) {
        rescale(mx);
        presum();
      }
      if constexpr (!TI::kSplitP) {
#pragma unroll
        for (int e = 0; e < 4; ++e) l_vec = TI::rowsum(psum[e], l_vec);
      }
      started = __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0;
    } else {
#pragma unroll
      for (int g16 = 0; g16 < NG; ++g16) {
        pb[g16] = u32x4{0, 0, 0, 0};
        pl[g16] = u32x4{0, 0, 0, 0};
      }
      psum = u32x4{0, 0, 0, 0};
    }
  };
  // The fp16 fast V phase, run by fast iterations only (the tile t = t_lo +
  // 2 (j + 1) + grp is visited and interior, and every row holds a
  // reference max).  P is formed against the current reference; the lane's
  // sum of it over the tile (the pre-added fp16 words, summed in fp32 by
  // v_dot2c) bounds every P and every pre-added word, so when it is at most
  // 2^10 nothing overflowed fp16 and P stands; otherwise (or inf / NaN) the
  // reference is raised and P formed again.  An earlier tile of the wave
  // went through the general V phase and set v_first, so only the count and
  // the last tile move here.
  auto v_fast = [&](int j) __attribute__((always_inline)) {
    ++v_count;
    v_last = t_lo + 2 * (j + 1) + grp;
    make_p();
    presum();
    float tsum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) tsum = TI::rowsum(psum[e], tsum);
    if (__builtin_amdgcn_ballot_w64(!(tsum <= kTileSumMax))) {
      rescale(pair_max(lane_max()));
      presum();
      tsum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) tsum = TI::rowsum(psum[e], tsum);
    }
    l_vec += tsum;
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Tile t is read by M_{t-2} (K fragments) and M_{t-1} (V fragments; the
  // reads are issued in M_{t-2}).  Its direct loads are issued in M_{t-NS}
  // (the prologue for t < NS) into the slot of tile t - NS, whose last
  // fragment reads were issued in M_{t-NS-1} and completed by every wave
  // before the barrier that ends V_{t-NS-1} (each V phase ends with
  // lgkmcnt(0)).  The end of V_j waits for tile j + 3; the tile after it may
  // still be in flight, so each load has about two phases to land.  (Issuing
  // K one tile earlier still, into the half of a slot that frees first, ran
  // slower.)
  // Token-pool layout: M_j (j >= 0) also issues the row load of tile
  // j + NS + 2 after the tile's loads, so a wait that lets M_j's tile stay in
  // flight lets its row load too (the prologue's row loads precede its tiles),
  // and the wait that lands tile j + 3 lands the rows of tile j + NS + 1,
  // which M_{j+1} reads.
  auto wait_tiles = [&](int j) __attribute__((always_inline)) {
    const int newest = min(j < 0 ? NS - 1 : j + NS, n_stages - 1);  // last tile requested
    const int ahead = newest - (j + 3);  // tiles allowed in flight
    if (NS == 5 && ahead >= 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPW));
    else if (ahead >= 1 && paged && j >= 0)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW + 1));
    else if (ahead >= 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  };

  // ---- prologue: tiles 0 .. NS-1 requested, 0 and 1 landed ----
  if (paged) {
    // the row ring's first two tiles (NS, NS + 1) before every tile load;
    // then the pool rows of the first tiles, read together into registers,
    // and each tile issued (one index round trip instead of one per tile)
    fetch_idx(NS);
    fetch_idx(NS + 1);
    uint32_t pre[NS][LPW];
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < LPW; ++i) pre[j][i] = (uint32_t)kv_list[tile_key(j, i)];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (j >= n_stages) break;
      load_tile(j, pre[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < NS; ++j)
      if (j < n_stages) load_tile(j, nullptr);
  }
  prepare_q<TI, KSTEPS>(qf, c, valid);
  {
    const int in_flight = min(NS - 1, n_stages - 1) - 1;  // tiles 2 .. newest
    if (in_flight >= 3)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * LPW));
    else if (in_flight == 2)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPW));
    else if (in_flight == 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  barrier();
  read_k(0);
  if (grp == 1) barrier();  // group 1 runs one phase behind group 0

  // Fast iterations: steady (0 <= j < n_stages - NS - 1, so tile j + NS is
  // always issued, is not the group's last tile, and NS - 3 tiles stay in
  // flight at the wait) and, for fp16,
  // the V phase's tile t = t_lo + 2 (j + 1) + grp in the wave's interior run,
  // after at least one interior tile went through the general V phase.
  // There the V phase forms P against the current reference at once (no row
  // max) and raises the reference only if the lane's sum of P over the tile
  // exceeds 2^10 (each p and each pre-added sum is at most that otherwise,
  // so the fp16 P stays finite).  They are iterations jf_lo .. jf_end - 1, with
  // 0 <= jf_lo <= jf_end <= n_stages - NS - 1, or none (jf_lo = jf_end =
  // n_stages).
  int jf_lo = n_stages, jf_end = n_stages;
  if (TI::kPrescaleQ && wave_live && tf_hi >= tf_lo) {
    const int j_first = (tf_lo - t_lo - grp + 1) / 2 - 1;  // first j with t >= tf_lo
    const int j_last = (tf_hi - t_lo - grp) / 2 - 1;       // last j with t <= tf_hi
    const int lo = max(j_first + 1, 0), hi = min(j_last, n_stages - NS - 2);
    if (hi >= lo) {
      jf_lo = lo;
      jf_end = hi + 1;
    }
  }
  // One iteration: M_j then V_j.
  auto iteration = [&](int j, auto fast) __attribute__((always_inline)) {
    constexpr bool kFast = decltype(fast)::value;
    // ---- M_j ----
    __builtin_amdgcn_s_setprio(1);
    m_phase(j);
    // the direct loads go after the MFMAs: issued while the last ones drain
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kFast) {
      if (paged) {
        load_tile(j + NS, nullptr);
        fetch_idx(j + NS + 2);
      } else {
        load_inner_tile(j + NS);
      }
    } else if (j >= 0 && j + NS < n_stages) {
      load_tile(j + NS, nullptr);
      if (paged) fetch_idx(j + NS + 2);
    }
    __builtin_amdgcn_s_setprio(0);
    barrier();
    // ---- V_j ----
    if constexpr (kFast) {
      v_fast(j);
      if constexpr (NS >= 5)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * LPW));
      else if (paged)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW + 1));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(LPW));
    } else {
      v_phase(j);
      wait_tiles(j);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's fragment reads done
    barrier();
  };
  // three runs of iterations, one loop each (one V-phase variant per loop
  // body keeps the register allocation of the single-loop form); `started`
  // fails only for non-finite scores, and then every iteration is general
  int j = -1;
  for (; j < jf_lo; ++j) iteration(j, std::false_type{});
  if (started)
    for (; j < jf_end; ++j) iteration(j, std::true_type{});
  for (; j < n_stages; ++j) iteration(j, std::false_type{});
  // the last prefetch reads must be done before LDS is reused for the merge
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  if (grp == 0) barrier();

  // the row's full sum (both lane halves' keys)
  float l_run = TI::kSplitP ? lsum[0] : l_vec + other_half(l_vec);
  // ---- merge the two groups' partial (m, l, O) through LDS ----
  {
    constexpr int NV = 2 + 16 * DB;
    float* mb = reinterpret_cast<float*>(lds);
    if (grp == 1) {
      float* dst = mb + rg * NV * 64 + lane;
      dst[0] = m_run;
      dst[64] = l_run;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) dst[(2 + db * 16 + i) * 64] = acc[db][i];
    }
    __syncthreads();
    if (grp == 0) {
      const float* src = mb + rg * NV * 64 + lane;
      const float m1 = src[0], l1 = src[64];
      const float m = fmaxf(m_run, m1);
      const float a0 = (m_run == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
      const float a1 = (m1 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
      l_run = a0 * l_run + a1 * l1;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[db][i] = a0 * acc[db][i] + a1 * src[(2 + db * 16 + i) * 64];
      m_run = m;
    }
  }

  if (grp == 0 && valid)
    finish_row<D, XTRA, TI, TO>(p, acc, m_run, l_run, sink, tok0 + pos, head, half);

  if (p.log != nullptr)
    write_tile_log<R, 2>(p, lds, wave, v_first, v_last, v_count, slot, g * p.group + hg * p.hpack,
                         q0, q_last);
}

template <int D, int BKV, int NS, bool XTRA, typename TI, typename TO>
void launch_pp_x(const Params& p, int n_items, hipStream_t stream) {
  if (p.window > 0)
    hipLaunchKernelGGL((attn_pp_kernel<D, BKV, NS, true, XTRA, TI, TO>),
                       dim3(n_items, p.n_split), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_pp_kernel<D, BKV, NS, false, XTRA, TI, TO>),
                       dim3(n_items, p.n_split), dim3(512), 0, stream, p);
}

template <int D, int BKV, int NS, typename TI, typename TO>
hipError_t launch_pp(const Params& p, int n_items, hipStream_t stream) {
  if (p.n_split > 1 || p.lse != nullptr || !p.causal || p.kv_idx != nullptr)
    launch_pp_x<D, BKV, NS, true, TI, TO>(p, n_items, stream);
  else
    launch_pp_x<D, BKV, NS, false, TI, TO>(p, n_items, stream);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Streaming window kernel, for sliding windows much shorter than the chunk.
// One workgroup walks a run of consecutive Q tiles of one sequence, KV head
// and head group.  Its eight waves form two streams of four 32-row waves:
// stream s takes tile j + s of each pair (j, j + 1), and both read the
// window's K/V from one LDS ring of 32-key blocks (block kb in slot kb % NR).
// Consecutive tiles share all but q_rows of their keys, so each pair loads
// only the blocks the next pair adds -- issued at the pair's start, waited
// for at its end -- instead of a whole window per tile; and each wave loads
// the Q of its next tile into its Q registers as soon as its last S MFMA has
// read them.  Per block a wave runs S^T = K . Q^T, the mask where the block
// is not interior to its rows, the online softmax with the lazy rescale, and
// O^T += V^T . P^T, as attn_fwd_kernel does per tile; the two streams' waves
// share each SIMD, one's matrix work beside the other's vector work.
// Causal, window > 0, one KV part; XTRA adds the log-sum-exp output and the
// token-pool layout.  The ring holds two pairs' keys when
// (4 q_rows + window - 2) / 32 + 2 <= NR (swin_applies).
constexpr int kSwinRing = 9;

bool swin_applies(int d, int window, int q_rows, bool split_or_noncausal) {
  return !split_or_noncausal && window > 0 && (d == 64 || d == 128) && q_rows > 0 &&
         ((int64_t)4 * q_rows + window - 2) / 32 + 2 <= kSwinRing;
}

template <int D, bool XTRA, typename TI, typename TO>
__global__ __launch_bounds__(512) void attn_swin_kernel(Params p) {
  constexpr int BKV = 32;
  constexpr int R = 4;                  // row waves per stream
  constexpr int NW = 2 * R;
  constexpr int NR = kSwinRing;
  constexpr int DCH = D / 8;
  constexpr int BLK_CH = BKV * DCH;     // 16-byte chunks of one K (or V) block
  constexpr int SLOT_CH = 2 * BLK_CH;   // K, then V
  constexpr int KSTEPS = D / 16;
  constexpr int NG = BKV / 16;
  constexpr int DB = D / 32;
  constexpr int PPW = SLOT_CH / 64 / NW;  // 1-KB direct loads per wave per block
  constexpr float kRescale = 8.f;
  static_assert(SLOT_CH % (64 * NW) == 0, "direct loads tile a block");
  static_assert(NR * SLOT_CH * 16 + 2 * NW * 3 * 4 + 64 * 16 <= 160 * 1024, "LDS");

  __shared__ u32x4 ring[NR * SLOT_CH];
  __shared__ int rec_wl[2][NW * 3];     // per pair parity: each wave's (first, last, count)
  __shared__ u32x4 pf_sink[64];         // landing place of the Q prefetch (never read)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave % R;
  const int st = wave / R;
  const int half = lane >> 5;
  const int col = lane & 31;

  // ---- the run: KV head g, head group hg, sequence b, its tiles j_first .. j_last ----
  const int h_kv = p.h_kv, n_hg = p.n_hgroups, run = max(1, p.swin_run);
  const int g = blockIdx.x % h_kv;
  const int r0 = blockIdx.x / h_kv;
  const int hg = r0 % n_hg;
  int rr = r0 / n_hg;  // run index over the sequences, ceil(tiles / run) runs each
  int b = 0;
  for (;;) {
    const int nr_b = (p.seq.cu_tiles[b + 1] - p.seq.cu_tiles[b] + run - 1) / run;
    if (rr < nr_b || b + 1 >= p.seq.n_seq) break;
    rr -= nr_b;
    ++b;
  }
  const int nt = p.seq.cu_tiles[b + 1] - p.seq.cu_tiles[b];
  const int j_first = rr * run;
  const int j_last = min(nt, j_first + run) - 1;
  if (j_first > j_last) return;  // the whole workgroup: nothing to do
  const int cu0 = p.seq.cu_q[b];
  const int sq = p.seq.cu_q[b + 1] - cu0;
  const int past = p.seq.past[b];
  const int slot = p.seq.slot[b];
  const int skv = past + sq;
  const int W = p.window;
  const int q_rows = p.q_rows;
  const int tile0 = p.seq.cu_tiles[b];
  const float c = p.scale_log2;
  const float kNegInf = -__builtin_inff();

  const int row = rg * 32 + col;
  const int psub = row / p.hpack;  // position within the Q tile
  const int head = g * p.group + hg * p.hpack + row % p.hpack;
  const float sink = load_sink(p.sink, head);

  // Token-pool layout (XTRA only): key k of this sequence is pool row
  // kv_list[k], rows h_kv * d elements apart; otherwise the dense cache of
  // this sequence's slot and KV head.
  const bool paged = XTRA && p.kv_idx != nullptr;
  const int32_t* kv_list = paged ? p.kv_idx + p.seq.kv_start[b] : nullptr;
  const int64_t kv_base =
      paged ? (int64_t)g * D : ((int64_t)slot * h_kv + g) * (int64_t)p.s_cap * D;
  const uint16_t* kptr = reinterpret_cast<const uint16_t*>(p.k) + kv_base;
  const uint16_t* vptr = reinterpret_cast<const uint16_t*>(p.v) + kv_base;
  const uint32_t ring_addr = lds_byte_addr(ring);

  // ---- direct loads: wave w issues pieces w * PPW + i of a block's 2 * BLK_CH
  // / 64 one-KB pieces (K, then V); lane l of a piece fills chunk 64 * piece + l
  // of its tensor block: key (64 * piece + l) / DCH, physical chunk l % DCH ----
  int ld_key[PPW];
  uint32_t ld_off[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int qi = wave * PPW + i;
    const int tt = qi / (BLK_CH / 64);
    const int chunk = (qi % (BLK_CH / 64)) * 64 + lane;
    const int key = chunk / DCH;
    const int pch = chunk % DCH;
    const int ch = tt ? v_chunk<D>(key, pch) : k_chunk<D>(key, pch);
    ld_key[i] = key;
    ld_off[i] = (uint32_t)(key * D + ch * 8) * 2u;
  }
  // Blocks kb_from .. kb_to (at most NR) into their slots; rows at or past
  // skv read row skv - 1 (finite data whose scores the causal mask removes).
  auto load_blocks = [&](int kb_from, int kb_to) __attribute__((always_inline)) {
    uint32_t prow[NR][PPW];
    if (paged) {
      // every pool row first, then the loads (one index round trip)
#pragma unroll
      for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int i = 0; i < PPW; ++i)
          prow[n][i] = kb_from + n <= kb_to
                           ? (uint32_t)kv_list[min((kb_from + n) * BKV + ld_key[i], skv - 1)]
                           : 0u;
    }
#pragma unroll
    for (int n = 0; n < NR; ++n) {
      const int kb = kb_from + n;
      if (kb > kb_to) break;
      const uint32_t dst = ring_addr + (uint32_t)((kb % NR) * SLOT_CH) * 16u;
#pragma unroll
      for (int i = 0; i < PPW; ++i) {
        const int qi = wave * PPW + i;
        const int tt = qi / (BLK_CH / 64);
        const int blk = qi % (BLK_CH / 64);
        const uint32_t ldst = dst + (uint32_t)(tt * BLK_CH + blk * 64) * 16u;
        if (paged) {
          const uint32_t r = min(prow[n][i], p.n_pool - 1u);
          lds_dma16(tt ? vptr : kptr, r * p.kv_row_bytes + ld_off[i] - (uint32_t)ld_key[i] * (D * 2),
                    ldst);
          continue;
        }
        const char* blkp =
            reinterpret_cast<const char*>(tt ? vptr : kptr) + (int64_t)kb * (BKV * D * 2);
        uint32_t voff = ld_off[i];
        if (kb * BKV + BKV > skv) {
          const int r = min(ld_key[i], skv - 1 - kb * BKV);
          voff -= (uint32_t)(ld_key[i] - r) * (D * 2);
        }
        lds_dma16(blkp, voff, ldst);
      }
    }
  };
  // blocks of the pair starting at tile j: from the first row's window floor
  // to the key of the pair's last row
  auto pair_lo = [&](int j) __attribute__((always_inline)) {
    return max(0, past + j * q_rows - W + 1) / BKV;
  };
  auto pair_hi = [&](int j) __attribute__((always_inline)) {
    const int je = min(j + 1, j_last);
    return (past + min((je + 1) * q_rows, sq) - 1) / BKV;
  };

  // Q^T fragments of this lane's row of tile jt (rows past the chunk read its
  // last row; prepare_q zeroes them)
  u32x4 qf[KSTEPS];
  auto load_q = [&](int jt) __attribute__((always_inline)) {
    const int pos = jt * q_rows + psub;
    const int64_t qoff = ((int64_t)(cu0 + min(pos, sq - 1)) * p.h_q + head) * D + half * 8;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk] = load16<TI>(p.q, qoff + kk * 16);
  };

  // The Q rows of this stream's tile jt brought into L2 a pair ahead: one
  // 16-byte direct load into pf_sink per 128-byte line of the tile's 2 D
  // lines (each position's hpack rows are hpack D / 64 consecutive lines),
  // one load a wave, so that the register loads at the end of the previous
  // tile find them in L2 instead of HBM.
  const uint32_t pf_addr = lds_byte_addr(pf_sink);
  auto prefetch_q = [&](int jt) __attribute__((always_inline)) {
    const int q0 = jt * q_rows;
    const char* qtile = reinterpret_cast<const char*>(p.q) +
                        (((int64_t)(cu0 + q0) * p.h_q + g * p.group + hg * p.hpack) * D) * 2;
    const int lpp = p.hpack * D / 64;             // lines per position
    const int line = (rg * 64 + lane) % (2 * D);  // the tile's lines
    const int pr = min(q0 + line / lpp, sq - 1) - q0;  // positions past the chunk: its last
    lds_dma16(qtile, (uint32_t)((pr * p.h_q * D + (line % lpp) * 64) * 2), pf_addr);
  };

  // One Q tile of this wave's stream: every block of its rows' window, then
  // the epilogue; the visited blocks are noted in (*vf, *vl, *vc).
  auto tile = [&](int jt, int* vf, int* vl, int* vc) __attribute__((always_inline)) {
    const int q0 = jt * q_rows;
    const int pos = q0 + psub;
    const bool valid = pos < sq;
    const int row_hi = past + pos;           // last kept key
    const int row_lo = past + pos - W + 1;   // first kept key
    const int wp0 = q0 + (rg * 32) / p.hpack;
    const int wp1 = min(q0 + (rg * 32 + 31) / p.hpack, sq - 1);
    const bool wave_live = wp0 < sq;
    const int w_lo = max(0, past + wp0 - W + 1) / BKV;
    const int w_hi = (past + wp1) / BKV;
    const int w_full_lo = past + wp1 - W + 1;  // max row lower bound
    const int w_full_hi = past + wp0;          // min row upper bound
    const bool next = jt + 2 <= j_last;
    prepare_q<TI, KSTEPS>(qf, c, valid);
    float m_run = kNegInf, l_run = 0.f, m_use = 0.f;
    f32x16 negm = f32x16{};  // splat(-m_use): MFMA accumulator input (prescaled-Q path)
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    // S^T of block kb relative to the current reference (fp16: -m enters
    // as the accumulator input; bf16: scaled and shifted on the VALU later)
    auto scores = [&](int kb) __attribute__((always_inline)) {
      const u32x4* kt = ring + (kb % NR) * SLOT_CH;
      f32x16 sc = TI::mma(kt[col * DCH + k_chunk<D>(col, half)], qf[0],
                          TI::kPrescaleQ ? negm : f32x16{});
#pragma unroll
      for (int kk = 1; kk < KSTEPS; ++kk)
        sc = TI::mma(kt[col * DCH + k_chunk<D>(col, 2 * kk + half)], qf[kk], sc);
      return sc;
    };
    // exp2 units (bf16), the mask where block kb is not interior to this
    // wave's rows, the row max, and a raise of the reference max where the
    // block needs it (wave-uniform; rescales O and l, shifts sc)
    auto prepare = [&](int kb, f32x16& sc) __attribute__((always_inline)) {
      if constexpr (!TI::kPrescaleQ) {
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] = __builtin_fmaf(sc[i], c, -m_use);
      }
      const int kbase = kb * BKV;
      if (!((kbase + BKV - 1 <= w_full_hi) && (kbase >= w_full_lo))) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kbase + (i >> 2) * 8 + half * 4 + (i & 3);
          if (key > row_hi || key < row_lo) sc[i] = kNegInf;
        }
      }
      float m4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
      for (int i = 0; i < 16; i += 2)
        m4[(i >> 1) & 3] = vmax(m4[(i >> 1) & 3], vmax(sc[i], sc[i + 1]));
      const float mx = pair_max(vmax(vmax(m4[0], m4[1]), vmax(m4[2], m4[3])));
      if (__builtin_amdgcn_ballot_w64((mx > kRescale) || (m_run == kNegInf && mx != kNegInf))) {
        const float m_new = fmaxf(m_run, mx + m_use);
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m_run = m_new;
        const float m_use_new = (m_new == kNegInf) ? 0.f : m_new;
        const float shift = m_use - m_use_new;
        m_use = m_use_new;
#pragma unroll
        for (int i = 0; i < 16; ++i) negm[i] = -m_use;
#pragma unroll
        for (int i = 0; i < 16; ++i) sc[i] += shift;
      }
      if (*vc == 0) *vf = kb;
      *vl = kb;
      ++*vc;
    };
    // P = exp2(S) of block kb, 16-bit (bf16: hi + lo parts), its row sum into
    // l_run, and O^T += V^T . P^T (consecutive MFMAs on different output
    // blocks; bf16: every block's hi part, then its lo part)
    auto pv = [&](int kb, const f32x16& sc) __attribute__((always_inline)) {
      const u32x4* vt = ring + (kb % NR) * SLOT_CH + BLK_CH;
      u32x4 pb[NG], pl[NG];
      float rs = 0.f;
#pragma unroll
      for (int g16 = 0; g16 < NG; ++g16)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int i = (g16 & 1) * 8 + w * 2;
          const float p0 = __builtin_amdgcn_exp2f(sc[i]);
          const float p1 = __builtin_amdgcn_exp2f(sc[i + 1]);
          const uint32_t hi = TI::pack(p0, p1);
          pb[g16][w] = hi;
          if constexpr (TI::kSplitP) {
            pl[g16][w] = TI::pack(TI::lo_part(p0, hi, 0), TI::lo_part(p1, hi, 1));
            rs += p0 + p1;
          } else {
            rs = TI::rowsum(hi, rs);
          }
        }
      l_run += rs;
#pragma unroll
      for (int g16 = 0; g16 < NG; ++g16) {
        u32x4 a[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) a[db] = v_frag<D>(vt, g16, db, lane);
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = TI::mma(a[db], pb[g16], acc[db]);
        if constexpr (TI::kSplitP) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = TI::mma(a[db], pl[g16], acc[db]);
        }
      }
    };
    if (wave_live) {
      // two-stage pipeline: the next block's S MFMAs go out beside this
      // block's exponentials, then this block's P.V, then the next block's
      // mask, max and rescale (which rescales O after this block's P.V)
      f32x16 s_cur = scores(w_lo);
      // the last S of this tile has read qf: the next tile's Q goes in
      if (w_lo == w_hi && next) load_q(jt + 2);
      prepare(w_lo, s_cur);
      for (int kb = w_lo; kb < w_hi; ++kb) {
        f32x16 s_nxt = scores(kb + 1);
        pv(kb, s_cur);
        if (kb + 1 == w_hi && next) load_q(jt + 2);
        prepare(kb + 1, s_nxt);
        s_cur = s_nxt;
      }
      pv(w_hi, s_cur);
    } else if (next) {
      load_q(jt + 2);
    }
    // this pair's block loads and the next tile's Q landed; waited for here,
    // before the stores, since the vector-memory counter also counts stores
    // (the stores then complete under the next pair)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    const float l_kept = l_run + other_half(l_run);
    if (valid) finish_row<D, XTRA, TI, TO>(p, acc, m_run, l_kept, sink, cu0 + pos, head, half);
  };

  // ---- prologue: the first pair's blocks and each stream's first Q ----
  int ring_hi = pair_hi(j_first);
  load_blocks(pair_lo(j_first), ring_hi);
  if (j_first + st <= j_last) load_q(j_first + st);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  int par = 0;
  for (int j = j_first; j <= j_last; j += 2, par ^= 1) {
    // the blocks the next pair adds: their slots held blocks below this
    // pair's floor (the ring holds both pairs' keys)
    if (j + 2 <= j_last) {
      const int nh = pair_hi(j + 2);
      if (nh > ring_hi) {
        load_blocks(ring_hi + 1, nh);
        ring_hi = nh;
      }
    }
    const int jt = j + st;
    if (jt + 2 <= j_last) prefetch_q(jt + 2);
    int v_first = -1, v_last = -1, v_count = 0;
    if (jt <= j_last) tile(jt, &v_first, &v_last, &v_count);
    if (p.log != nullptr && lane == 0) {
      rec_wl[par][3 * wave + 0] = v_first;
      rec_wl[par][3 * wave + 1] = v_last;
      rec_wl[par][3 * wave + 2] = v_count;
    }
    // the next pair's blocks landed (a wave with a tile waited before its
    // stores); every wave done with this pair's blocks
    if (jt > j_last) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __syncthreads();
    if (p.log != nullptr && lane == 0 && rg == 0 && jt <= j_last) {
      const int64_t item = ((int64_t)(tile0 + jt) * n_hg + hg) * h_kv + g;
      store_tile_record<R, 1>(p.log + item * kLogFields, &rec_wl[par][3 * R * st], slot,
                              g * p.group + hg * p.hpack, p.hpack, jt * q_rows,
                              min((jt + 1) * q_rows, sq) - 1, 0, 1);
    }
  }
}

template <int D, bool XTRA, typename TI, typename TO>
void launch_swin_x(const Params& p, unsigned grid, hipStream_t stream) {
  hipLaunchKernelGGL((attn_swin_kernel<D, XTRA, TI, TO>), dim3(grid), dim3(512), 0, stream, p);
}

// Runs of an even number of Q tiles (both streams busy), a run within one
// sequence: the shortest runs whose workgroups all fit the chip at once (one
// per CU: eight waves of 160-250 VGPRs fill the register file), so that no
// second round of a few workgroups follows the first.
template <int D, typename TI, typename TO>
hipError_t launch_swin(const Params& p_in, int /*n_items*/, hipStream_t stream) {
  Params p = p_in;
  constexpr int64_t kSlots = 256;
  const int heads = p.h_kv * p.n_hgroups;
  auto count_runs = [&](int run) {
    int64_t runs = 0;
    for (int b = 0; b < p.seq.n_seq; ++b)
      runs += (p.seq.cu_tiles[b + 1] - p.seq.cu_tiles[b] + run - 1) / run;
    return runs * heads;
  };
  int run = (int)(((int64_t)p.seq.n_tiles * heads + kSlots - 1) / kSlots);
  run = max(2, run + (run & 1));
  while (run < 512 && count_runs(run) > kSlots) run += 2;
  p.swin_run = run;
  const int64_t grid = count_runs(run);
  if (grid <= 0) return hipSuccess;
  if (p.lse != nullptr || p.kv_idx != nullptr)
    launch_swin_x<D, true, TI, TO>(p, (unsigned)grid, stream);
  else
    launch_swin_x<D, false, TI, TO>(p, (unsigned)grid, stream);
  return hipGetLastError();
}

template <int D, int BKV, int R, int S, int NS, bool XTRA, typename TI, typename TO>
void launch_x(const Params& p, int n_items, hipStream_t stream) {
  constexpr int threads = R * (D >= 128 ? 1 : S) * 64;
  if (p.window > 0)
    hipLaunchKernelGGL((attn_fwd_kernel<D, BKV, R, S, NS, true, XTRA, TI, TO>),
                       dim3(n_items, p.n_split), dim3(threads), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, BKV, R, S, NS, false, XTRA, TI, TO>),
                       dim3(n_items, p.n_split), dim3(threads), 0, stream, p);
}

template <int D, int BKV, int R, int S, int NS, typename TI, typename TO>
hipError_t launch(const Params& p, int n_items, hipStream_t stream) {
  if (p.n_split > 1 || p.lse != nullptr || !p.causal || p.kv_idx != nullptr)
    launch_x<D, BKV, R, S, NS, true, TI, TO>(p, n_items, stream);
  else
    launch_x<D, BKV, R, S, NS, false, TI, TO>(p, n_items, stream);
  return hipGetLastError();
}

// d = 256 runs 32-key tiles (a stage of 64-key d 256 K and V tiles is 64 KB)
template <int BKV, int R, int S, int NS = 3>
constexpr KernelConfig make_config(const char* name) {
  return KernelConfig{
      name, {BKV, BKV, 32}, R * 32,
      {{{launch<64, BKV, R, S, NS, F16, uint16_t>, launch<64, BKV, R, S, NS, F16, float>},
        {launch<64, BKV, R, S, NS, BF16, uint16_t>, launch<64, BKV, R, S, NS, BF16, float>}},
       {{launch<128, BKV, R, S, NS, F16, uint16_t>, launch<128, BKV, R, S, NS, F16, float>},
        {launch<128, BKV, R, S, NS, BF16, uint16_t>, launch<128, BKV, R, S, NS, BF16, float>}},
       {{launch<256, 32, R, S, NS, F16, uint16_t>, launch<256, 32, R, S, NS, F16, float>},
        {launch<256, 32, R, S, NS, BF16, uint16_t>, launch<256, 32, R, S, NS, BF16, float>}}}};
}

// ---------------------------------------------------------------------------
// Merge of KV-split partial results (one thread per 4 output columns of a
// row).  With lse_s the partials' log2 log-sum-exp and M their maximum:
// out = sum_s 2^(lse_s - M) o_s / (sum_s 2^(lse_s - M) + 2^(sink log2 e - M)),
// lse = (M + log2 sum_s 2^(lse_s - M)) ln 2; a row no part kept gives 0, -inf.
template <int D, int OUT>  // OUT: 0 fp16, 1 bf16, 2 fp32
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeParams mp) {
  constexpr int TPR = D / 4;
  const int64_t rows = (int64_t)mp.tokens * mp.h_q;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= rows) return;
  const int c = (threadIdx.x % TPR) * 4;
  const int head = (int)(row % mp.h_q);
  const float kNegInf = -__builtin_inff();
  float mx = kNegInf;
  for (int s = 0; s < mp.n_split; ++s) mx = fmaxf(mx, mp.ws_lse[s * rows + row]);
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != kNegInf) {
    for (int s = 0; s < mp.n_split; ++s) {
      const float w = __builtin_amdgcn_exp2f(mp.ws_lse[s * rows + row] - mx);
      den += w;
      o += w * *reinterpret_cast<const f32x4*>(mp.ws_o + (s * rows + row) * D + c);
    }
  }
  float tot = den;
  if (mp.sink != nullptr && mx != kNegInf)
    tot += __builtin_amdgcn_exp2f(mp.sink[head] * kLog2e - mx);
  const float inv = mx != kNegInf ? 1.f / tot : 0.f;
  o *= inv;
  if constexpr (OUT == 2) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(mp.out) + row * D + c) = o;
  } else if constexpr (OUT == 1) {
    bf16x2 a = {(__bf16)o[0], (__bf16)o[1]}, b = {(__bf16)o[2], (__bf16)o[3]};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(mp.out) + row * D + c) =
        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  } else {
    f16x2 a = {(_Float16)o[0], (_Float16)o[1]}, b = {(_Float16)o[2], (_Float16)o[3]};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(mp.out) + row * D + c) =
        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
  }
  if (mp.lse != nullptr && c == 0)
    mp.lse[row] = mx != kNegInf ? (mx + __builtin_amdgcn_logf(den)) * kLn2 : kNegInf;
}

template <int D, int OUT>
hipError_t launch_merge_t(const MergeParams& mp, hipStream_t stream) {
  constexpr int rows_per_block = 256 / (D / 4);
  const int64_t rows = (int64_t)mp.tokens * mp.h_q;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((attn_merge_kernel<D, OUT>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     mp);
  return hipGetLastError();
}

// Ping-pong configuration for d = 64; at d = 128 and 256 (where its register
// budget does not hold two groups' fragments) the same entry runs the
// split-free kernel with the same 128-row Q tiles.
template <int BKV, int NS>
constexpr KernelConfig make_pp_config(const char* name) {
  return KernelConfig{
      name, {BKV, 64, 32}, 128,
      {{{launch_pp<64, BKV, NS, F16, uint16_t>, launch_pp<64, BKV, NS, F16, float>},
        {launch_pp<64, BKV, NS, BF16, uint16_t>, launch_pp<64, BKV, NS, BF16, float>}},
       {{launch<128, 64, 4, 1, 3, F16, uint16_t>, launch<128, 64, 4, 1, 3, F16, float>},
        {launch<128, 64, 4, 1, 3, BF16, uint16_t>, launch<128, 64, 4, 1, 3, BF16, float>}},
       {{launch<256, 32, 4, 1, 3, F16, uint16_t>, launch<256, 32, 4, 1, 3, F16, float>},
        {launch<256, 32, 4, 1, 3, BF16, uint16_t>, launch<256, 32, 4, 1, 3, BF16, float>}}}};
}

// The streaming window kernel (d 64 and 128; calls it does not run fall back
// to the default configuration, see swin_applies).
constexpr KernelConfig make_swin_config(const char* name) {
  return KernelConfig{
      name, {32, 32, 32}, 128,
      {{{launch_swin<64, F16, uint16_t>, launch_swin<64, F16, float>},
        {launch_swin<64, BF16, uint16_t>, launch_swin<64, BF16, float>}},
       {{launch_swin<128, F16, uint16_t>, launch_swin<128, F16, float>},
        {launch_swin<128, BF16, uint16_t>, launch_swin<128, BF16, float>}},
       {{nullptr, nullptr}, {nullptr, nullptr}}},
      swin_applies};
}

}  // namespace

#if defined(ATTN_CONFIG) && ATTN_CONFIG >= 0
// The library is compiled from this file once per kernel configuration
// (ATTN_CONFIG = its index in the table below), so that the configurations'
// instantiations build in parallel; ATTN_CONFIG = -1 compiles the table, the
// merge kernel and the lookups.
// (Each entry is a host function, so the device pass never sees the table.)
#define ATTN_CONFIG_ENTRY(i, ...)                     \
  const KernelConfig& config_entry_##i() {            \
    static constexpr KernelConfig entry = __VA_ARGS__; \
    return entry;                                      \
  }
#if ATTN_CONFIG == 0
ATTN_CONFIG_ENTRY(0, make_pp_config<64, 4>("pp_r128_kv64_ring4"))
#elif ATTN_CONFIG == 1
ATTN_CONFIG_ENTRY(1, make_config<64, 4, 2, 4>("r128_kv64_s2_ring4"))
#elif ATTN_CONFIG == 2
ATTN_CONFIG_ENTRY(2, make_config<64, 4, 2>("r128_kv64_s2"))
#elif ATTN_CONFIG == 3
ATTN_CONFIG_ENTRY(3, make_config<64, 4, 1>("r128_kv64_s1"))
#elif ATTN_CONFIG == 4
ATTN_CONFIG_ENTRY(4, make_config<32, 2, 2>("r64_kv32_s2"))
#elif ATTN_CONFIG == 5
// 32-row Q tiles (one row group, two KV-split waves, 48 KB of LDS) for calls
// with few rows per sequence, e.g. decode steps (one position x the KV
// group's heads)
ATTN_CONFIG_ENTRY(5, make_config<32, 1, 2>("r32_kv32_s2"))
#elif ATTN_CONFIG == 6
// streaming window kernel: runs of consecutive 128-row Q tiles per workgroup
// over an LDS ring of 32-key blocks (window calls of long chunks)
ATTN_CONFIG_ENTRY(6, make_swin_config("swin_r128_kv32"))
#else
#error "ATTN_CONFIG out of range"
#endif

#else  // the table, the merge kernel and the lookups

const KernelConfig& config_entry_0();
const KernelConfig& config_entry_1();
const KernelConfig& config_entry_2();
const KernelConfig& config_entry_3();
const KernelConfig& config_entry_4();
const KernelConfig& config_entry_5();
const KernelConfig& config_entry_6();
namespace {
const KernelConfig& (*const kConfigs[])() = {config_entry_0, config_entry_1, config_entry_2,
                                             config_entry_3, config_entry_4, config_entry_5,
                                             config_entry_6};
}  // namespace

hipError_t launch_merge(const MergeParams& mp, int out_is_f32, int out_is_bf16,
                        hipStream_t stream) {
  const int out = out_is_f32 ? 2 : (out_is_bf16 ? 1 : 0);
  if (mp.d == 64)
    return out == 2 ? launch_merge_t<64, 2>(mp, stream)
                    : (out == 1 ? launch_merge_t<64, 1>(mp, stream)
                                : launch_merge_t<64, 0>(mp, stream));
  if (mp.d == 128)
    return out == 2 ? launch_merge_t<128, 2>(mp, stream)
                    : (out == 1 ? launch_merge_t<128, 1>(mp, stream)
                                : launch_merge_t<128, 0>(mp, stream));
  return out == 2 ? launch_merge_t<256, 2>(mp, stream)
                  : (out == 1 ? launch_merge_t<256, 1>(mp, stream)
                              : launch_merge_t<256, 0>(mp, stream));
}

// Scratch of attn_prefill_split_noalloc (the KV-split partials of one call),
// so that callers that cannot allocate need not pass a workspace.  In host
// code `scratch` names a host-side stand-in, never the device array: its
// device address is taken once per device with hipGetSymbolAddress (with
// that device current) and only that address reaches kernels.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

int config_count() { return (int)(sizeof(kConfigs) / sizeof(kConfigs[0])); }
const KernelConfig& config(int i) { return kConfigs[i](); }
int default_config(int /*d*/, int /*dtype*/, int /*window*/) { return 0; }
bool config_applies(int i, int d, int window, int q_rows, bool split_or_noncausal) {
  const AppliesFn f = config(i).applies;
  return f == nullptr || f(d, window, q_rows, split_or_noncausal);
}
#endif

}  // namespace attn
