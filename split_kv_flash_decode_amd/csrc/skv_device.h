// Device-side helpers shared by the HIP kernels: vector types, storage
// conversions, address arithmetic of the KV layouts, wave reductions and the
// split merge formula.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "skv_internal.h"

namespace skv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Storage tags.
struct F32 {};
struct BF16 {};
struct I8 {};
struct FP8 {};
struct F16 {};   // Q/O only: IEEE binary16

template <class T> struct Storage;
template <> struct Storage<F32> { static constexpr int bytes = 4; static constexpr bool quant = false; };
template <> struct Storage<BF16> { static constexpr int bytes = 2; static constexpr bool quant = false; };
template <> struct Storage<I8> { static constexpr int bytes = 1; static constexpr bool quant = true; };
template <> struct Storage<FP8> { static constexpr int bytes = 1; static constexpr bool quant = true; };
template <> struct Storage<F16> { static constexpr int bytes = 2; static constexpr bool quant = false; };

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// Round-to-nearest-even fp32 -> fp16 pair.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  floatx2 x = {a, b};
  f16x2 y = __builtin_convertvector(x, f16x2);
  return __builtin_bit_cast(uint32_t, y);
}

__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t lo16) { return __uint_as_float(lo16 << 16); }

// Round-to-nearest-even fp32 -> bf16 pair (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  floatx2 x = {a, b};
  bf16x2 y = __builtin_convertvector(x, bf16x2);
  return __builtin_bit_cast(uint32_t, y);
}

// Two e4m3fn codes (bytes 0-1 or, with HI, 2-3 of w) -> two fp32 values, exact.
template <bool HI>
__device__ __forceinline__ floatx2 fp8x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// Two e4m3fn codes -> packed bf16 pair, exact (every e4m3 value is a bf16 value).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  bf16x2 y = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, y);
}

template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_f16x2(uint32_t w) {
  f16x2 y = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
  return __builtin_bit_cast(uint32_t, y);
}

// Byte n of w as a signed int8 -> fp32 (exact).
__device__ __forceinline__ float i8_to_f32(uint32_t w, int n) {
  return (float)(int32_t)((int32_t)(w << (24 - 8 * n)) >> 24);
}

// ---- wave-wide reductions (butterflies: every lane ends with the same bits) --
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---- KV addressing -----------------------------------------------------------
// Element offset of K[token t][d] of KV head g of request b (row-major rows of D).
__device__ __forceinline__ int64_t k_row(const Params& p, int page, int b, int g, int t) {
  if (p.paged) {
    int slot = t & ((1 << p.bs_shift) - 1);
    return ((((int64_t)page * p.Hkv + g) << p.bs_shift) + slot) * p.D;
  }
  return (((int64_t)b * p.Hkv + g) * p.kv_cap + t) * p.D;
}
// Offset of scale of token t (paged [page][Hkv][bs], contiguous [B][Hkv][cap]).
__device__ __forceinline__ int64_t scale_idx(const Params& p, int page, int b, int g, int t) {
  if (p.paged) {
    int slot = t & ((1 << p.bs_shift) - 1);
    return (((int64_t)page * p.Hkv + g) << p.bs_shift) + slot;
  }
  return ((int64_t)b * p.Hkv + g) * p.kv_cap + t;
}
// Offset of V^T[d][t] in the transposed layouts ([page][Hkv][D][bs] or [B][Hkv][D][cap]).
__device__ __forceinline__ int64_t vt_idx(const Params& p, int page, int b, int g, int d, int t) {
  if (p.paged) {
    int slot = t & ((1 << p.bs_shift) - 1);
    return ((((int64_t)page * p.Hkv + g) * p.D + d) << p.bs_shift) + slot;
  }
  return (((int64_t)b * p.Hkv + g) * p.D + d) * p.kv_cap + t;
}
// Pool page holding token t of request b (paged), read only for t < ctx.
__device__ __forceinline__ int page_of(const Params& p, int b, int t) {
  return p.paged ? p.table[(int64_t)b * p.max_pages + (t >> p.bs_shift)] : 0;
}

// ---- direct-to-LDS loads ----------------------------------------------------------
// Wait until at most n vector-memory operations of this wave are outstanding.
// Direct-to-LDS loads count in vmcnt; the compiler does not order later LDS
// reads after them, so every stage is consumed after an explicit wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)p);
}

// One direct-to-LDS load per lane (16 or 4 bytes): lane l's bytes land at
// lds + l * size. Issued as inline assembly so that the compiler neither
// reorders LDS reads around it nor adds its own (draining) waits; every
// consumer waits with wait_vm.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(base) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}

// Page-table entry read through the constant address space: the table is
// read-only for the whole call, so uniform reads become scalar loads.
__device__ __forceinline__ int cload(const int* p) {
  return *(const __attribute__((address_space(4))) int*)p;
}

// ---- the plan ------------------------------------------------------------------
__device__ __forceinline__ bool planned(const Params& p) { return p.plan != nullptr || p.plan_inline; }

// The plan's metadata block: in device memory, or (a plan passed by value)
// in the kernel's own argument block, found through the kernarg segment
// pointer (the parameter block is the kernel's first and only argument, at
// offset 0), so the block is never copied into private memory. One generic
// pointer for both cases keeps the scalar registers free.
__device__ __forceinline__ const int32_t* plan_base(const Params& p) {
  if (p.plan_inline) {
    typedef const __attribute__((address_space(4))) char kchar;
    kchar* blob = (kchar*)__builtin_amdgcn_kernarg_segment_ptr() + offsetof(Params, plan_blob);
    return (const int32_t*)(const char*)blob;
  }
  return p.plan;
}

// Work item -> (request, split, splits of the request, record item index);
// false for an unused plan item.
__device__ __forceinline__ bool decode_item(const Params& p, int item, Item* it) {
  if (planned(p)) {
    // (values the whole workgroup shares: kept in scalar registers)
    const int32_t* plan = plan_base(p);
    const int w = __builtin_amdgcn_readfirstlane(plan[4 + 2 * p.B + item]);
    if (w < 0) return false;
    it->b = w >> 8;
    it->s = w & 255;
    it->S = __builtin_amdgcn_readfirstlane(plan[4 + it->b]);
    it->slot_item = __builtin_amdgcn_readfirstlane(plan[4 + p.B + it->b]) + it->s;
  } else {
    it->b = item / p.num_splits;
    it->s = item - it->b * p.num_splits;
    it->S = p.num_splits;
    it->slot_item = item;
  }
  return true;
}

__device__ __forceinline__ int clamp_ctx(const Params& p, int b) {
  int c = p.ctx[b];
  c = c < 0 ? 0 : c;
  return c > p.cap ? p.cap : c;
}

// ---- the merge of split records ----------------------------------------------
// One output element from one record (single pass). Written exactly like one
// iteration of the combine kernel's loop so that a one-split combine gives the
// same bits: M = max(m, sink); w = 2^(m - M); L = 0 + w l (+ 2^(sink - M));
// O = (0 + w acc) * (1 / (L + 1e-9)); a record with l = 0 gives 0.
__device__ __forceinline__ float finalize_one(float m, float l, float acc, int has_sink, float s2) {
  if (!(l > 0.0f)) return 0.0f;
  float M = fmaxf(-INFINITY, m);
  if (has_sink) M = fmaxf(M, s2);
  float L = 0.0f;
  float a = 0.0f;
  float w = fexp2(m - M);
  L += w * l;
  a += w * acc;
  if (has_sink) L += fexp2(s2 - M);
  float inv = 1.0f / (L + 1e-9f);
  return a * inv;
}

// Output element store: fp32 or bf16 (RNE).
__device__ __forceinline__ void store_o1(const Params& p, int64_t idx, float x) {
  if (p.q_dtype == SKV_BF16 || p.q_dtype == SKV_F16) {
    uint32_t w = p.q_dtype == SKV_BF16 ? pack_bf16x2(x, 0.0f) : pack_f16x2(x, 0.0f);
    reinterpret_cast<uint16_t*>(p.o)[idx] = (uint16_t)(w & 0xFFFF);
  } else {
    reinterpret_cast<float*>(p.o)[idx] = x;
  }
}

__device__ __forceinline__ void store_o4(const Params& p, int64_t idx, floatx4 x) {
  if (p.q_dtype == SKV_BF16) {
    u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + idx) = w;
  } else if (p.q_dtype == SKV_F16) {
    u32x2 w = {pack_f16x2(x[0], x[1]), pack_f16x2(x[2], x[3])};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(p.o) + idx) = w;
  } else {
    *reinterpret_cast<floatx4*>(reinterpret_cast<float*>(p.o) + idx) = x;
  }
}

// Offset of q/o element [b][j][h][d].
__device__ __forceinline__ int64_t qo_idx(const Params& p, int b, int j, int h, int d) {
  return (((int64_t)b * p.R + j) * p.Hq + h) * p.D + d;
}

// Query row r (0 <= r < rho) of KV head g: query token j and head h.
__device__ __forceinline__ void row_jh(const Params& p, int g, int r, int* j, int* h) {
  *j = r / p.G;
  *h = g * p.G + (r - (r / p.G) * p.G);
}

// Partial-record accumulator stores: fp32, or bf16 by round to nearest even.
__device__ __forceinline__ void store_rec1(const Params& p, int64_t idx, float x) {
  if (p.rec_bf16)
    static_cast<uint16_t*>(p.pacc)[idx] = (uint16_t)(pack_bf16x2(x, 0.0f) & 0xFFFF);
  else
    static_cast<float*>(p.pacc)[idx] = x;
}

__device__ __forceinline__ void store_rec4(const Params& p, int64_t idx, floatx4 x) {
  if (p.rec_bf16)
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.pacc) + idx) =
        u32x2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
  else
    *reinterpret_cast<floatx4*>(static_cast<float*>(p.pacc) + idx) = x;
}

// Running state of a split merge: maximum M, sum L and accumulators a (for
// four d), all relative to M.
struct MergeState {
  float M, L;
  floatx4 a;
};

// Take one record (m, l, acc) into the running state: a record that raises
// the maximum rescales the sums first; empty records (l = 0) are skipped.
__device__ __forceinline__ void merge_absorb(MergeState& t, float m, float l, floatx4 acc) {
  if (!(l > 0.0f)) return;
  if (m > t.M) {
    const float sc = fexp2(t.M - m);                // 0 while M is -inf
    t.L *= sc;
    t.a[0] *= sc;
    t.a[1] *= sc;
    t.a[2] *= sc;
    t.a[3] *= sc;
    t.M = m;
  }
  const float w = fexp2(m - t.M);
  t.L += w * l;
  t.a[0] += w * acc[0];
  t.a[1] += w * acc[1];
  t.a[2] += w * acc[2];
  t.a[3] += w * acc[3];
}

// Records of splits [s_begin, s_end) in increasing order, read in batches of
// NB whose loads are all in flight together (indices past the range re-read
// its last split and are skipped). RBF: bf16 record accumulators (widened
// after the whole batch is loaded).
template <int NB, bool RBF>
__device__ __forceinline__ MergeState merge_range(const Params& p, int64_t rec0, int64_t rs, int d, int s_begin,
                                                  int s_end) {
  MergeState t{-INFINITY, 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}};
  for (int s0 = s_begin; s0 < s_end; s0 += NB) {
    float lb[NB], mb[NB];
    floatx4 ab[NB];
    u32x2 hb[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = s0 + i < s_end ? s0 + i : s_end - 1;
      lb[i] = p.pl[rec0 + s * rs];
      mb[i] = p.pm[rec0 + s * rs];
      const int64_t e = (rec0 + s * rs) * p.D + d;
      if constexpr (RBF)
        hb[i] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.pacc) + e);
      else
        ab[i] = *reinterpret_cast<const floatx4*>(static_cast<const float*>(p.pacc) + e);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (RBF)
        ab[i] = floatx4{__uint_as_float(hb[i][0] << 16), __uint_as_float(hb[i][0] & 0xFFFF0000u),
                        __uint_as_float(hb[i][1] << 16), __uint_as_float(hb[i][1] & 0xFFFF0000u)};
      if (s0 + i < s_end) merge_absorb(t, mb[i], lb[i], ab[i]);
    }
  }
  return t;
}

// ---- the combine of a request's records ----------------------------------------
// The flash-decoding merge (tiny-llm #11 split-KV design record, "Design";
// aiter #5628 "tune MTP work budgets and planned reduction", Changes: only
// the partitions a request actually has). A request with S splits owns S
// work items; each item gives the merge K workgroups per KV head, so the
// request's S * K workgroups share its rho * D / 4 output units (four
// consecutive d of one query row) whatever S is: every thread loads about
// eight records, and a long request is merged by as many workgroups as it
// has splits. Inside a workgroup, L lanes (a power of two) share a unit and
// take consecutive runs of its splits in increasing order; their states are
// then merged by a fixed butterfly, each pair in split order, so the result
// does not depend on timing (deterministic), only on (S, K, rho, D).

constexpr int kMergeThreads = 256;

// Workgroups per (item, KV head) of the combine: about eight record loads per
// thread (2048 units per workgroup of 256 threads).
SKV_HD int merge_wgs_per_item(int rho, int D) { return (rho * (D / 4) + 2047) / 2048; }

// Merge of two states, a holding earlier splits than b.
__device__ __forceinline__ MergeState merge_pair(const MergeState& a, const MergeState& b) {
  if (!(b.L > 0.0f)) return a;
  if (!(a.L > 0.0f)) return b;
  const float M = fmaxf(a.M, b.M);
  const float wa = fexp2(a.M - M), wb = fexp2(b.M - M);
  MergeState t;
  t.M = M;
  t.L = wa * a.L + wb * b.L;
  t.a[0] = wa * a.a[0] + wb * b.a[0];
  t.a[1] = wa * a.a[1] + wb * b.a[1];
  t.a[2] = wa * a.a[2] + wb * b.a[2];
  t.a[3] = wa * a.a[3] + wb * b.a[3];
  return t;
}

__device__ __forceinline__ MergeState shfl_state(const MergeState& s, int off) {
  MergeState o;
  o.M = __shfl_xor(s.M, off, 64);
  o.L = __shfl_xor(s.L, off, 64);
  o.a[0] = __shfl_xor(s.a[0], off, 64);
  o.a[1] = __shfl_xor(s.a[1], off, 64);
  o.a[2] = __shfl_xor(s.a[2], off, 64);
  o.a[3] = __shfl_xor(s.a[3], off, 64);
  return o;
}

// Part w (of S * K) of the merge of request b, KV head g, whose S records
// start at slot item slot0, as thread t (0 <= t < 256) of a 256-thread group:
// output units [w U / (S K), (w + 1) U / (S K)), U = rho * D / 4. Lanes of one
// unit are consecutive threads, so a group of 64 threads (a wave) holds whole
// units and may run on its own.
template <bool RBF>
__device__ __forceinline__ void merge_part(const Params& p, int b, int g, int S, int slot0, int w, int K, int t) {
  const int tpr = p.D >> 2;
  const int64_t U = (int64_t)p.rho * tpr;
  const int64_t parts = (int64_t)S * K;
  const int u0 = (int)(w * U / parts), u1 = (int)((w + 1) * U / parts);
  const int nu = u1 - u0;
  if (nu <= 0) return;
  int L = 1;                                     // lanes per unit: the most that keep one pass
  while (L < 64 && 2 * L * nu <= kMergeThreads) L <<= 1;
  const int q = t & (L - 1);
  const int c = (S + L - 1) / L;                 // splits per lane
  const int sb = q * c < S ? q * c : S, se = q * c + c < S ? q * c + c : S;
  const int64_t rs = (int64_t)p.Hkv * p.rho;     // record stride between splits
  for (int u = u0 + t / L; u < u1; u += kMergeThreads / L) {
    const int r = u / tpr, d = 4 * (u - r * tpr);
    const int64_t rec0 = (int64_t)slot0 * rs + (int64_t)g * p.rho + r;
    MergeState st = c <= 4 ? merge_range<4, RBF>(p, rec0, rs, d, sb, se) : merge_range<8, RBF>(p, rec0, rs, d, sb, se);
    for (int off = L >> 1; off > 0; off >>= 1) {
      const MergeState o = shfl_state(st, off);
      st = (q & off) ? merge_pair(o, st) : merge_pair(st, o);
    }
    if (q == 0) {
      int j, h;
      row_jh(p, g, r, &j, &h);
      floatx4 out = {0.0f, 0.0f, 0.0f, 0.0f};
      if (st.L > 0.0f) {
        float L2 = st.L;
        floatx4 acc = st.a;
        if (p.has_sink) {
          const float s2 = p.sinks[h] * kLog2e;
          const float M2 = fmaxf(st.M, s2);
          const float sc = fexp2(st.M - M2);
          L2 *= sc;
          acc[0] *= sc;
          acc[1] *= sc;
          acc[2] *= sc;
          acc[3] *= sc;
          L2 += fexp2(s2 - M2);
        }
        const float inv = 1.0f / (L2 + 1e-9f);
        out[0] = acc[0] * inv;
        out[1] = acc[1] * inv;
        out[2] = acc[2] * inv;
        out[3] = acc[3] * inv;
      }
      store_o4(p, qo_idx(p, b, j, h, d), out);
    }
  }
}

// Single-kernel split + merge (tiny-llm #11 split-KV design record, points
// for reviewer decision, Q1): called by every workgroup of a partial kernel
// after it wrote its records. The workgroups of one (request, KV head) count
// themselves on a device-scope counter; the last one to arrive runs every
// part of that pair's merge (merge_part for w = 0 .. S K - 1, with the same
// thread numbering as the combine kernel, so the output has the same bits
// whichever workgroup arrives last) and resets the counter to zero for the
// next call. One agent-scope release fence per workgroup before it counts
// (after a barrier, so it covers every wave's stores), an acquire fence in
// the merging workgroup after: the records of workgroups on other XCDs are
// then visible to it. it is the calling workgroup's decoded work item;
// nthreads is a multiple of 64.
__device__ __forceinline__ void fused_merge_tail(const Params& p, const Item& it, int g, int nthreads) {
  __shared__ int last_s;
  const int tid = threadIdx.x;
  const int b = it.b, S = it.S, slot0 = it.slot_item - it.s;   // the request's split 0
  __syncthreads();                                 // the workgroup's record stores are done
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // ... and visible device-wide
    int* cnt = p.counters + (int64_t)b * p.Hkv + g;
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == S * p.row_groups - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = last;
  }
  __syncthreads();
  if (!last_s) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int K = merge_wgs_per_item(p.rho, p.D);
  const int total = S * K * kMergeThreads;
  for (int vt = tid; vt < total; vt += nthreads) {
    const int w = vt / kMergeThreads, t = vt - w * kMergeThreads;
    if (p.rec_bf16)
      merge_part<true>(p, b, g, S, slot0, w, K, t);
    else
      merge_part<false>(p, b, g, S, slot0, w, K, t);
  }
}

}  // namespace skv
