// Internal definitions shared by the host library and the HIP kernels.
//
// Nothing here is part of the C ABI; include/skv.h is.
#pragma once

#include <stdint.h>

#include "skv.h"

namespace skv {

// Everything a kernel needs, passed by value as one kernel argument.
struct Params {
  const void* q;
  const void* k;
  const void* v;
  const float* ks;
  const float* vs;
  const int32_t* table;
  const int32_t* ctx;
  const float* sinks;
  void* o;
  const uint64_t* tree_mask;  // verify masks [B][R][ceil(R / 64)], or nullptr
  float* pm;
  float* pl;
  void* pacc;            // fp32 or (rec_bf16) bf16 record accumulators
  const int32_t* plan;   // device plan metadata, or nullptr for uniform splits
  int32_t* counters;     // single-kernel merge: arrival counters [B * Hkv], or nullptr
  int32_t B, R, Hq, Hkv, D, G, rho;
  int32_t causal, window;
  float scale_log2;      // scale * log2(e)
  int32_t bs_shift;      // log2(block_size) (paged)
  int32_t max_pages;     // page-table row stride (paged)
  int32_t cap;           // context clamp: max_pages * block_size or kv_capacity
  int32_t kv_cap;        // contiguous token stride
  int32_t num_splits;    // uniform S; with a plan, the plan capacity C
  int32_t has_sink;
  int32_t paged;
  int32_t finalize;      // 1: single pass, write o instead of a partial record
  int32_t n_items;       // work items in the grid
  int32_t row_groups;    // row groups per (item, KV head)
  int32_t q_dtype, kv_dtype, v_layout, block_size, impl;
  int32_t rec_bf16;      // 1: record acc in bf16
  // A plan passed by value (skv_attention_decode_paged_planned_host): the
  // metadata block is plan_blob itself, read from the kernel's argument
  // block; plan is then nullptr. Last, so the fields above keep their offsets.
  int32_t plan_inline;
  int32_t plan_blob[SKV_PLAN_INLINE_MAX];
};

// Resolved planner hints for the device-side planner.
struct PlanDev {
  int32_t B, R, Hkv, causal, window, cus, ctas, wph, explicit_p, maxp, work, min_tokens, C;
};

// Query rows one workgroup of the matrix-core partial kernel covers: two row
// halves of 32 when a KV head has more than 32 rows, one at D 256 (its
// accumulators need the registers).
inline int mfma_group_rows(int D, int rho) { return (D == 256 || rho <= 32) ? 32 : 64; }
// Query rows one wave (workgroup) of the vector partial kernel covers.
constexpr int kValuRows = 8;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSplitAlign = SKV_SPLIT_ALIGN;
// Lazy rescaling: the running reference maximum is only raised when a new
// logit exceeds it by more than this many powers of two.
constexpr float kRescaleSlack = 8.0f;
constexpr float kRescaleLimit = 256.0f;   // 2^kRescaleSlack: the largest probability kept

// Host + device helpers --------------------------------------------------------

#if defined(__HIPCC__)
#define SKV_HD __host__ __device__ __forceinline__
#else
#define SKV_HD inline
#endif

// Split s of S over the visible union of a request of length ctx:
// [u, ctx) with u = 0 or the earliest row's window start aligned down;
// chunk = ceil((ctx - u) / S) rounded up to kSplitAlign.
// Start u of the visible union and chunk length of S splits of a request of
// length ctx > 0.
SKV_HD void split_geometry(int ctx, int R, int causal, int window, int S, int* u_out, int* chunk_out) {
  int u = 0;
  if (window > 0) {
    int pmin = causal ? ctx - R : ctx - 1;
    u = pmin - window + 1;
    u = u < 0 ? 0 : u;
    u = (u / kSplitAlign) * kSplitAlign;
  }
  int span = ctx - u;
  int chunk = (span + S - 1) / S;
  chunk = ((chunk + kSplitAlign - 1) / kSplitAlign) * kSplitAlign;
  *u_out = u;
  *chunk_out = chunk;
}

SKV_HD void split_range(int ctx, int R, int causal, int window, int S, int s, int* lo, int* hi) {
  if (ctx <= 0) {
    *lo = 0;
    *hi = 0;
    return;
  }
  int u, chunk;
  split_geometry(ctx, R, causal, window, S, &u, &chunk);
  long long l0 = (long long)u + (long long)s * chunk;
  if (l0 >= ctx) {
    *lo = ctx;
    *hi = ctx;
    return;
  }
  long long h0 = l0 + chunk;
  *lo = (int)l0;
  *hi = (int)(h0 < ctx ? h0 : ctx);
}

// Visible key range [vlo, vhi) of query row j.
// Words of a row's verify mask.
SKV_HD int verify_words(int R) { return (R + 63) >> 6; }

// Bit of a verify mask for key t of a row whose (up to four) words are w
// (draft keys start at dbase = ctx - R; the prefix is always visible). Word
// and shift are clamped so that keys past ctx, which other tests mask, stay
// defined.
SKV_HD bool tree_visible(const uint64_t (&w)[4], int t, int dbase) {
  if (t < dbase) return true;
  const unsigned i = (unsigned)(t - dbase);
  const unsigned q = i >> 6;
  const uint64_t x = q == 0 ? w[0] : q == 1 ? w[1] : q == 2 ? w[2] : w[3];
  return ((x >> (i & 63u)) & 1ull) != 0;
}

// The same, reading the row's words from memory (only for keys past dbase).
SKV_HD bool tree_visible_mem(const uint64_t* row, int t, int dbase) {
  if (t < dbase) return true;
  const unsigned i = (unsigned)(t - dbase);
  return ((row[(i >> 6) & 3u] >> (i & 63u)) & 1ull) != 0;
}

SKV_HD void row_range(int ctx, int R, int causal, int window, int j, int* vlo, int* vhi) {
  int p = causal ? ctx - R + j : ctx - 1;
  int hi = p + 1;
  if (hi > ctx) hi = ctx;
  int lo = 0;
  if (window > 0) lo = p - window + 1;
  if (lo < 0) lo = 0;
  if (hi < 0) hi = 0;
  *vlo = lo;
  *vhi = hi;
}

// The matrix-core kernel addresses a transposed-V row of a contiguous cache
// with a 32-bit per-lane byte offset from the (request, KV head) base:
// (D - 1) * kv_capacity * bytes + 16 must stay below 2^31, else the call goes
// to the vector kernel (64-bit addressing throughout).
SKV_HD bool mfma_offsets_fit(int paged, int v_layout, int D, int kv_cap, int kv_bytes) {
  if (paged || v_layout != SKV_V_TRANSPOSED) return true;
  return (long long)D * kv_cap * kv_bytes < (1ll << 31);
}

// Work item -> (request, split, splits of the request, record item index);
// decoded by decode_item in skv_device.h.
struct Item {
  int b, s, S, slot_item;
};

}  // namespace skv

// Host-side launchers (defined in the .hip files) ---------------------------------
namespace skv {
int launch_partial_valu(Params p, void* stream);
int launch_partial_mfma(Params p, void* stream);
int launch_combine(Params p, void* stream);
int launch_plan_device(const PlanDev& h, const int32_t* ctx, int32_t* meta, void* stream);
int launch_gather_ceiling(Params p, uint32_t* sink, void* stream);
bool mfma_supported(const Params& p);
// Host checks of a uniform split call other than its partial buffers
// (descriptor, arguments, split count, grid limits, kernel family).
int check_split_call(const skv_desc* d, const skv_args* a, int paged, int32_t num_splits);
}  // namespace skv
