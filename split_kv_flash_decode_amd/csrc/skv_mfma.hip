// Matrix-core partial kernel for BF16 queries over BF16, INT8 or FP8 KV and
// FP16 queries over INT8 or FP8 KV.
//
// What it computes is one split of the split-KV method (tiny-llm #11 split-KV
// design record, "Design": a partial kernel over (head, split) that derives its
// key range from the device visible length and emits (m_i, l_i, acc_i); hipfire
// #760 "split packed-Q8 verifier KV scans", Summary: a multi-row causal verifier
// whose KV loads are shared by every query row inside a tile; aiter #5628 "tune
// MTP work budgets and planned reduction": MTP rows over FP8 KV with per-token
// FP32 scales, page sizes 16 and 128, plain and transposed V).
//
// gfx950 design
//  * One workgroup per (work item, KV head, group of up to 64 query rows).
//    Every query row of a KV head (R * Hq / Hkv rows: GQA heads times MTP or
//    verify rows) shares each key and value loaded, so a block of 32 keys is a
//    dense contraction: S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//  * Four key streams take interleaved 32-key blocks of the item's key range.
//    With more than 32 rows, each stream has two waves (rows 0-31 and 32-63),
//    eight waves in all, two per SIMD: one wave's vector work then fills the
//    issue slots around the other's matrix-core and memory work. Each wave
//    keeps the online-softmax state of its 32 rows for its stream; the four
//    streams' states are merged through LDS at the end, in stream order.
//  * K, V and the per-token scales go from HBM straight into a per-stream LDS
//    ring (global_load_lds of whole key rows, NS stages). Of the two waves of
//    a stream one issues the K and scale loads, the other the V loads. With
//    four stages one workgroup barrier per two blocks publishes them and
//    frees the two stages refilled meanwhile; otherwise one barrier per
//    block, with NS - 1 blocks in flight. With one row half a stream is
//    one wave that loads everything it reads: its own load counter is the
//    only wait, and the key loop has no barrier.
//  * Per block a wave reads from LDS only its K operand rows, V (issued
//    before the softmax, whose vector work hides the read latency) and one K
//    and one V scale per lane; DPP row broadcasts hand each lane the scales
//    of its 16 keys. Q (fp8 or int8 parts, or bf16) stays in registers for
//    the whole key loop (the int8 parts at D 256 are re-read from LDS per
//    block), and the accumulators stay in arch VGPRs (AGPRs with one row
//    half).
//  * Key order inside a 32-key block is permuted (tau) so that the S^T output
//    a lane holds is 16 consecutive keys of one query row: exactly the P^T
//    operand of the P.V product. Plain-layout V reaches the V^T operand through
//    gfx950's transposing LDS reads (8 keys of one d per lane), from rows whose
//    16-byte chunks the loads permute to keep those reads conflict-free.
//  * FP8 K feeds the fp8 matrix cores directly (v_mfma_scale_f32_32x32x64_
//    f8f6f4): Q is split once per workgroup, per row and 32-d block, into an
//    fp8 high part and an fp8 residual with power-of-two block scales, which
//    reproduces every bf16 element within 2^13 of its block maximum exactly;
//    these products accumulate at about 2^-14 of the sum of their magnitudes
//    (measured), not at fp32. INT8 K with a bf16 query feeds the int8 matrix
//    cores directly (v_mfma_i32_32x32x32_i8): Q is split once per workgroup,
//    per row, into two int8 parts with one power-of-two scale (every bf16
//    element within 2^7 of the row's maximum exactly, the rest within 2^-14
//    of the maximum), and the two int32 sums combine exactly before one
//    conversion per logit. BF16 K converts to bf16 (no-op) for
//    v_mfma_f32_32x32x16_bf16. With an fp16 query, INT8 and FP8 K convert to
//    fp16 (exactly) for v_mfma_f32_32x32x16_f16, the query keeping all its
//    bits. V codes always convert to bf16 exactly. The
//    per-token K scale multiplies the logits and the per-token V scale the
//    probabilities, so the other rounding is P -> bf16.
//  * The softmax is online with lazy rescaling: the running maximum of a row
//    is only raised (and acc, l rescaled) when a logit exceeds it by more than
//    2^8, which a wave vote detects; the row max needs one cross-half shuffle.
//  * Blocks that lie wholly inside the split and inside every row's visible
//    range skip all masking; boundary blocks mask logits with selects (never
//    multiply-by-zero, so NaN-poisoned cache slots past a request's context
//    never reach an accumulator) and zero V codes and scales of keys past the
//    split.

#include <type_traits>
#include <utility>

#include "skv_device.h"

namespace skv {

namespace {

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v4i32 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

// MFMA row i of the K operand of a 32-key block holds key tau(i); then output
// value v of a lane in wave half h is key 16 h + v.
__device__ __forceinline__ int tau(int i) { return ((i & 4) << 2) | ((i >> 1) & 0xC) | (i & 3); }

// y[v] = x of lane 16 (lane / 16) + v: a broadcast inside each 16-lane row
// (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, true));
}
template <int... V>
__device__ __forceinline__ void row_bcast16(float x, float (&y)[16], std::integer_sequence<int, V...>) {
  ((y[V] = row_bcast<V>(x)), ...);
}
// y[B + v] = (x of lane 16 (lane / 16) + B + v) * a[B + v], v < 8: the
// broadcast rides on the multiply (v_mul_f32_dpp). The leading s_nop covers
// the wait states a DPP source needs after a VALU write.
template <int B>
__device__ __forceinline__ void row_bcast_mul8(float x, const float (&a)[16], float (&y)[16]) {
  asm("s_nop 1\n\t"
      "v_mul_f32_dpp %0, %8, %9 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %1, %8, %10 row_newbcast:%18 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %2, %8, %11 row_newbcast:%19 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %3, %8, %12 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %4, %8, %13 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %5, %8, %14 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %6, %8, %15 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
      "v_mul_f32_dpp %7, %8, %16 row_newbcast:%24 row_mask:0xf bank_mask:0xf"
      : "=&v"(y[B]), "=&v"(y[B + 1]), "=&v"(y[B + 2]), "=&v"(y[B + 3]), "=&v"(y[B + 4]), "=&v"(y[B + 5]),
        "=&v"(y[B + 6]), "=&v"(y[B + 7])
      : "v"(x), "v"(a[B]), "v"(a[B + 1]), "v"(a[B + 2]), "v"(a[B + 3]), "v"(a[B + 4]), "v"(a[B + 5]),
        "v"(a[B + 6]), "v"(a[B + 7]), "n"(B), "n"(B + 1), "n"(B + 2), "n"(B + 3), "n"(B + 4), "n"(B + 5),
        "n"(B + 6), "n"(B + 7));
}

template <class KT>
__device__ __forceinline__ bf16x8 cvt8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  u32x4 r;
  if constexpr (__is_same(KT, FP8)) {
    r = u32x4{fp8x2_to_bf16x2<false>(w0), fp8x2_to_bf16x2<true>(w0), fp8x2_to_bf16x2<false>(w1),
              fp8x2_to_bf16x2<true>(w1)};
  } else if constexpr (__is_same(KT, I8)) {
    r = u32x4{pack_bf16x2(i8_to_f32(w0, 0), i8_to_f32(w0, 1)), pack_bf16x2(i8_to_f32(w0, 2), i8_to_f32(w0, 3)),
              pack_bf16x2(i8_to_f32(w1, 0), i8_to_f32(w1, 1)), pack_bf16x2(i8_to_f32(w1, 2), i8_to_f32(w1, 3))};
  } else {
    r = u32x4{w0, w1, w2, w3};
  }
  return __builtin_bit_cast(bf16x8, r);
}

// 8-bit K codes as fp16 operands for an fp16 query (both conversions exact:
// e4m3 and int8 values are fp16 values).
template <class KT>
__device__ __forceinline__ f16x8 cvt8h(uint32_t w0, uint32_t w1) {
  u32x4 r;
  if constexpr (__is_same(KT, FP8)) {
    r = u32x4{fp8x2_to_f16x2<false>(w0), fp8x2_to_f16x2<true>(w0), fp8x2_to_f16x2<false>(w1),
              fp8x2_to_f16x2<true>(w1)};
  } else {
    static_assert(__is_same(KT, I8), "fp16 queries take 8-bit K codes");
    r = u32x4{pack_f16x2(i8_to_f32(w0, 0), i8_to_f32(w0, 1)), pack_f16x2(i8_to_f32(w0, 2), i8_to_f32(w0, 3)),
              pack_f16x2(i8_to_f32(w1, 0), i8_to_f32(w1, 1)), pack_f16x2(i8_to_f32(w1, 2), i8_to_f32(w1, 3))};
  }
  return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ floatx16 mfma(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ floatx16 mfma(f16x8 a, f16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Query operand type of S^T = K Q^T: the query's own 16-bit format.
template <class QT> struct QOperand { typedef bf16x8 type; };
template <> struct QOperand<F16> { typedef f16x8 type; };

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Keep only the keys with index < nv of a word holding keys
// [first, first + per_word) (per_word = 4 for 8-bit codes, 2 for 16-bit);
// branch-free.
__device__ __forceinline__ uint32_t keep_bytes(uint32_t w, int first, int nv, int per_word) {
  int k = nv - first;
  k = k < 0 ? 0 : (k > per_word ? per_word : k);
  const uint32_t m = (uint32_t)((1ull << (k * (32 / per_word))) - 1ull);
  return w & m;
}

}  // namespace

template <class QT, class KT, int D, int NRH, bool VT, bool TM>
__global__ __launch_bounds__(256 * NRH) void partial_mfma(Params p) {
  constexpr int EB = Storage<KT>::bytes;
  constexpr bool QUANT = Storage<KT>::quant;
  constexpr int DB = D / 32;                     // P.V d-blocks of 32
  constexpr int NT = 256 * NRH;                  // threads: 4 key streams x NRH row halves
  constexpr int ROWS = 32 * NRH;
  constexpr int RB = D * EB;                     // bytes of one key row
  constexpr int NCH = RB / 32;                   // 16-byte K chunks per lane and block
  // Stage: K rows (32 RB bytes), V (plain: two 16-key groups of rows, the
  // second shifted by 128 bytes so the two lane halves read different LDS
  // banks; transposed: 16-byte key runs of V^T rows), then 32 K and 32 V
  // scales.
  constexpr int KSZ = 32 * RB;
  constexpr int VGS = 16 * RB + 128;             // plain V: group stride
  constexpr int VSZ = VT ? 32 * RB : 2 * VGS;
  constexpr int STAGE = KSZ + VSZ + (QUANT ? 256 : 0);
  constexpr int KIG = RB / 64;                   // 1 KiB loads per 16-key group, K (and plain V)
  constexpr int U = DB * EB;                     // transposed V: 512-byte units per group
  static_assert(RB >= 64 && RB % 64 == 0, "key rows of 64, 128 or 256 bytes");
  constexpr int QS = D + 8;                      // LDS row stride of Q (bf16), padded
  // FP8 K with a bf16 query: S^T = K Q^T runs on the fp8 matrix cores
  // (32x32x64 with block scales), Q split once per workgroup into an fp8 high
  // part and an fp8 residual; otherwise K is converted to the query's 16-bit
  // format (bf16 or fp16) and multiplied on the 16-bit matrix cores. P V is
  // always a bf16 product.
  constexpr bool F8QK = __is_same(KT, FP8) && __is_same(QT, BF16);
  // INT8 K with a bf16 query: S^T = K Q^T runs on the int8 matrix cores
  // (32x32x32, exact int32 sums), Q split once per workgroup into two int8
  // parts with one power-of-two scale per row.
  constexpr bool I8QK = __is_same(KT, I8) && __is_same(QT, BF16);
  typedef typename QOperand<QT>::type qop;
  constexpr int QS8 = D + 16;                    // LDS row stride of the 8-bit Q parts, padded
  constexpr int QBYTES = F8QK ? 2 * ROWS * QS8 + ROWS * (D / 32) * 2
                              : (I8QK ? 2 * ROWS * QS8 + ROWS * 4 : ROWS * QS * 2);
  constexpr int BUDGET = 156 * 1024;
  constexpr int NS0 = (BUDGET - QBYTES) / (4 * STAGE);
  constexpr int NS = NS0 > 4 ? 4 : (NS0 < 2 ? 2 : NS0);   // ring stages per key stream
  constexpr int RING = 4 * NS * STAGE;
  constexpr int PD = D + 4;                      // merge buffer row stride (floats, 16-byte aligned)
  constexpr int MERGE = 4 * ROWS * PD * 4;       // one slice per key stream
  constexpr int SMEM0 = RING > MERGE ? RING : MERGE;
  // Plain V rows sit in LDS with their 16-byte chunks permuted, chunk c of
  // row r (key r of a 16-key group) at c ^ vswz(r), so that the transposing
  // LDS reads of the P.V operand (8 keys of one d per lane for 8-bit codes,
  // 4 for bf16) hit distinct banks across a half-wave. Rows of one 256-byte
  // bank line (KPR of them) share their banks; the XOR separates the keys
  // that would collide.
  constexpr int NCK = RB / 16;                   // 16-byte chunks per key row
  constexpr int KPR = RB >= 256 ? 1 : 256 / RB;  // key rows per 256-byte bank line
  constexpr int SPAN = EB == 1 ? 2 : 4;          // chunks per key one half-wave reads
  auto vswz = [](int r) __attribute__((always_inline)) {
    return SPAN * ((r / KPR) % (NCK / SPAN));
  };
  // K rows (key r of a 32-key block) are permuted the same way with a finer
  // XOR: the S^T operand reads 16 bytes of each of 32 keys per half-wave.
  auto kswz = [](int r) __attribute__((always_inline)) { return (r / KPR) % NCK; };
  // Direct-to-LDS loads per block: K, V and (quantized) one of scales. With
  // two row halves the first half's wave of a stream issues K and the
  // scales, the second half's wave V.
  constexpr int NVL = VT ? U / 2 : KIG;          // V loads per 16-key group
  constexpr int NK = 2 * KIG + (QUANT ? 1 : 0);
  constexpr int NV = 2 * NVL;

  __shared__ __attribute__((aligned(16))) char smem[SMEM0 + QBYTES];
  __shared__ float ml_s[4][ROWS][2];
  __shared__ float fin_s[ROWS][2];
  uint16_t* q_s = reinterpret_cast<uint16_t*>(smem + SMEM0);
  float* acc_s = reinterpret_cast<float*>(smem);   // reused after the key loop

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sid = w & 3;                         // key stream
  const int rh = w >> 2;                         // row half
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int hh = lane >> 5;
  char* ring = smem + sid * NS * STAGE;

  // Block order: the row groups of one (item, KV head) read the same keys.
  // Workgroups are dealt to the eight XCDs (each with its own L2) in turn
  // by block index, so consecutive indices would put those readers on
  // different L2s; blocks 8 k + x of the first whole multiple of 8 tiles are
  // therefore mapped so that every row group of a tile has the same x (one
  // XCD, one L2), the rest in plain order.
  int blk = blockIdx.x;
  if (p.row_groups > 1) {
    const int RG = p.row_groups;
    const int T8 = ((int)gridDim.x / RG) & ~7;
    if (blk < T8 * RG) {
      const int x = blk & 7, k = blk >> 3;
      blk = ((k / RG) * 8 + x) * RG + k % RG;
    }
  }
  const int rg = blk % p.row_groups;
  blk /= p.row_groups;
  const int g = blk % p.Hkv;
  const int item = blk / p.Hkv;
  Item it;
  if (!decode_item(p, item, &it)) return;
  const int b = it.b;
  const int ctx = clamp_ctx(p, b);
  int lo, hi;
  split_range(ctx, p.R, p.causal, p.window, it.S, it.s, &lo, &hi);
  const int rbase = rg * ROWS;
  const int nrow = (p.rho - rbase) < ROWS ? (p.rho - rbase) : ROWS;

  uint8_t* qh_s = reinterpret_cast<uint8_t*>(smem + SMEM0);   // fp8 Q parts (F8QK)
  uint8_t* ql_s = qh_s + ROWS * QS8;
  uint8_t* qe_s = ql_s + ROWS * QS8;             // [row][32-d block]: E8M0 scales of both parts
  float* qr_s = reinterpret_cast<float*>(ql_s + ROWS * QS8);   // I8QK: [row] scale 2^(e - 7)
  // This wave's query rows: rbase + 32 rh + [0, 32); lane i32 owns one.
  const int wrow0 = rbase + 32 * rh;
  int vlo = 0, vhi = 0;
  uint64_t tmask[4] = {~0ull, ~0ull, ~0ull, ~0ull};   // TM: this lane's row's verify mask words
  if (wrow0 + i32 < p.rho) {
    row_range(ctx, p.R, p.causal, p.window, (wrow0 + i32) / p.G, &vlo, &vhi);
    if constexpr (TM) {
      const int nw = verify_words(p.R);
      const uint64_t* mrow = p.tree_mask + ((int64_t)b * p.R + (wrow0 + i32) / p.G) * nw;
#pragma unroll
      for (int w = 0; w < 4; ++w) tmask[w] = w < nw ? mrow[w] : 0ull;
    }
  }
  // with verify masks, blocks reaching the draft keys take the masked path
  const int dbase = TM ? ctx - p.R : 0x7FFFFFFF;
  // Keys every row of the wave sees: [ilo, ihi) (empty for a wave past rho).
  int ilo = 0, ihi = 0;
  if (wrow0 < p.rho) {
    const int last = (wrow0 + 31 < p.rho ? wrow0 + 31 : p.rho - 1);
    int a0, a1, c0, c1;
    row_range(ctx, p.R, p.causal, p.window, wrow0 / p.G, &a0, &a1);
    row_range(ctx, p.R, p.causal, p.window, last / p.G, &c0, &c1);
    ilo = a0 > c0 ? a0 : c0;
    ihi = a1 < c1 ? a1 : c1;
  }
  ilo = __builtin_amdgcn_readfirstlane(ilo);
  ihi = __builtin_amdgcn_readfirstlane(ihi);
  // 8-bit score paths: this thread's 32 query elements (one row, one 32-d
  // block), loaded before the first blocks' page-table reads
  u32x4 qpre[4] = {};
  if constexpr (__is_same(KT, FP8) || __is_same(KT, I8)) {
    if constexpr (__is_same(QT, BF16)) {
      static_assert(32 * NRH * (D / 32) <= 256 * NRH, "one query block per thread");
      const int row = tid / (D / 32), blk = tid - row * (D / 32);
      const int r = rbase + row;
      if (row < 32 * NRH && r < p.rho) {
        int j, hq;
        row_jh(p, g, r, &j, &hq);
        const uint16_t* src = reinterpret_cast<const uint16_t*>(p.q) + qo_idx(p, b, j, hq, 32 * blk);
#pragma unroll
        for (int u = 0; u < 4; ++u) qpre[u] = ld16(src + 8 * u);
      }
    }
  }

  floatx16 acc[DB];
  float mrun = -INFINITY, lrun = 0.0f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[db][v] = 0.0f;
  // Register file of the accumulators. Two row halves (two waves per SIMD):
  // arch VGPRs, which then hold nothing else the key loop needs, so no value
  // is copied in and out of AGPRs. One row half (one wave per SIMD, up to
  // 8 x 16 accumulators at D 256): AGPRs, which the matrix cores accumulate
  // into directly, leaving the arch VGPRs to the operands (measured 8-14 %
  // faster at D 256 and for int8 at D 128, equal for bf16 at D 128).
  auto pin_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      if constexpr (NRH == 1)
        asm volatile("" : "+a"(acc[db]));
      else
        asm volatile("" : "+v"(acc[db]));
    }
  };

  const char* kbase = reinterpret_cast<const char*>(p.k);
  const char* vbase = reinterpret_cast<const char*>(p.v);
  const int* trow = p.paged ? p.table + (int64_t)b * p.max_pages : nullptr;

  struct Ids {       // pool pages of a 32-key block's two halves (page size >= 16)
    int p0, p1;
  };
  auto load_ids = [&](int t0) __attribute__((always_inline)) {
    Ids id{0, 0};
    if (p.paged) {
      id.p0 = cload(trow + (t0 >> p.bs_shift));
      id.p1 = (p.bs_shift == 4 && t0 + 16 < hi) ? cload(trow + (t0 >> 4) + 1) : id.p0;
    }
    return id;
  };
  // Row index of the first key of 16-key group gp of the block at t0 (keys of
  // a group are consecutive rows of one page): K and plain V rows are at
  // base + R * RB, scales at scale + R. A group that starts at or past hi
  // reuses group 0 (inside the split), so no page past the request's context
  // is addressed; keys past hi inside a live group stay inside their page.
  auto grp_row = [&](const Ids& id, int t0, int gp) __attribute__((always_inline)) {
    const int tg = (t0 + 16 * gp < hi) ? t0 + 16 * gp : t0;
    if (p.paged) {
      const int pg = (gp && p.bs_shift == 4 && t0 + 16 < hi) ? id.p1 : id.p0;
      return (((int64_t)pg * p.Hkv + g) << p.bs_shift) + (tg & ((1 << p.bs_shift) - 1));
    }
    return ((int64_t)b * p.Hkv + g) * p.kv_cap + tg;
  };
  // Transposed V: element index of V^T row 0 at the group's first key.
  auto grp_vt = [&](const Ids& id, int t0, int gp) __attribute__((always_inline)) {
    const int tg = (t0 + 16 * gp < hi) ? t0 + 16 * gp : t0;
    if (p.paged) {
      const int pg = (gp && p.bs_shift == 4 && t0 + 16 < hi) ? id.p1 : id.p0;
      return ((((int64_t)pg * p.Hkv + g) * D) << p.bs_shift) + (tg & ((1 << p.bs_shift) - 1));
    }
    return (((int64_t)b * p.Hkv + g) * D) * p.kv_cap + tg;
  };

  // Per-lane byte offsets of the direct-to-LDS loads (fixed for the kernel).
  //  K, group gp, load n: whole key rows, like plain V: row n * (1024 / RB) +
  //    l / (RB / 16) of the group, LDS chunk l % (RB / 16) receiving global
  //    chunk (l % (RB / 16)) ^ kswz(row in the block), so that the consumer's
  //    16-byte reads of 32 different keys hit each bank at most twice.
  //  plain V, load n: row n * (1024 / RB) + l / (RB / 16), 16-byte column
  //    l % (RB / 16) (the group's rows, in key order).
  //  transposed V, load n: unit u = 2 n + l / 32 (d-block u / EB, 16-byte key
  //    run u % EB) of V^T row d = 32 (u / EB) + l % 32.
  uint32_t koffs[2][KIG];
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int n = 0; n < KIG; ++n)
    {
      const int row = n * (1024 / RB) + lane / (RB / 16);
      koffs[gp][n] = (uint32_t)(row * RB + (((lane % (RB / 16)) ^ kswz(16 * gp + row)) * 16));
    }
  uint32_t voffs[NVL];
  {
    const int dstride = (p.paged ? (1 << p.bs_shift) : p.kv_cap) * EB;
#pragma unroll
    for (int n = 0; n < NVL; ++n) {
      if constexpr (VT) {
        const int u = 2 * n + (lane >> 5);
        voffs[n] = (uint32_t)((32 * (u / EB) + i32) * dstride + (u % EB) * 16);
      } else {
        // LDS slot (row, chunk c) of the group receives global chunk
        // c ^ vswz(row) of that row
        constexpr int LPR = RB / 16;
        const int row = n * (1024 / RB) + lane / LPR;
        voffs[n] = (uint32_t)(row * RB + ((lane % LPR) ^ vswz(row)) * 16);
      }
    }
  }

  // Issue this wave's share of the direct-to-LDS loads of the block at t0
  // into stage st: K and the scales (first row half), V (second row half),
  // or all of them (one row half).
  auto issue = [&](int t0, const Ids& id, int st) __attribute__((always_inline)) {
    const uint32_t S = lds_addr(ring + st * STAGE);
    const int64_t R0 = grp_row(id, t0, 0), R1 = grp_row(id, t0, 1);
    if (NRH == 1 || rh == 0) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        const char* kb = kbase + (gp ? R1 : R0) * RB;
#pragma unroll
        for (int n = 0; n < KIG; ++n) dma16s(kb, koffs[gp][n], S + (gp * KIG + n) * 1024);
      }
      if constexpr (QUANT) {
        // lane l < 32: K scale of key l; l >= 32: V scale of key l - 32
        const int k = i32;
        const int64_t r = ((k >= 16) ? R1 : R0) + (k & 15);
        dma4((hh ? p.vs : p.ks) + r, S + KSZ + VSZ);
      }
    }
    if (NRH == 1 || rh == 1) {
      if constexpr (VT) {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const char* vb = vbase + grp_vt(id, t0, gp) * EB;
#pragma unroll
          for (int n = 0; n < NVL; ++n) dma16s(vb, voffs[n], S + KSZ + (gp * NVL + n) * 1024);
        }
      } else {
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const char* vb = vbase + (gp ? R1 : R0) * RB;
#pragma unroll
          for (int n = 0; n < NVL; ++n) dma16s(vb, voffs[n], S + KSZ + gp * VGS + n * 1024);
        }
      }
    }
  };
  // Wait until at most `blocks` of this wave's later blocks are in flight.
  auto wait_own = [&](int blocks) __attribute__((always_inline)) {
    constexpr int A = NRH == 1 ? NK + NV : NK;   // loads per block of a first-half wave
    constexpr int B = NRH == 1 ? NK + NV : NV;   // ... of a second-half wave
    if (rh == 0) {
      if (blocks >= 2) wait_vm<2 * A>();
      else if (blocks == 1) wait_vm<A>();
      else wait_vm<0>();
    } else {
      if (blocks >= 2) wait_vm<2 * B>();
      else if (blocks == 1) wait_vm<B>();
      else wait_vm<0>();
    }
  };

  // Consumer side of the K layout: row tau(i32) of the block; its 16-byte
  // chunk j sits at j ^ kswz(tau). This lane reads chunks hh * NCH + c.
  const int krow = tau(i32) * RB;
  const int kx = (hh * NCH) ^ kswz(tau(i32));
  // B operand of S^T = K Q^T, read from LDS at every block: k-step kk of lane
  // (i32, hh) is row 32 rh + i32, d in [hh D/2 + 8 kk, +8).
  const int qoff0 = (32 * rh + i32) * QS + hh * (D / 2);
  // fp8 path: k-step ks (64 d) of lane (i32, hh) covers d in [64 ks + 32 hh,
  // +32) of K (row tau(i32)) and of Q (row 32 rh + i32): one 32-d block, whose
  // two E8M0 scales are loop-invariant per lane.
  constexpr int KS8 = D / 64;
  int qsh[KS8], qsl[KS8];
  const int q8off = (32 * rh + i32) * QS8 + 16 * hh;
  // Q stays in registers for the whole key loop (fp8 parts, or bf16; the
  // int8 parts too, except at D 256).
  u32x4 qa[KS8][2], qb[KS8][2];
  constexpr int KPC = 16 / (8 * EB);              // k-steps per 16-byte chunk
  constexpr int KS = NCH * KPC;                   // k-steps of 16 d
  qop qf[(F8QK || I8QK) ? 1 : KS];
  // int8 path: k-step ks (32 d) of lane (i32, hh) covers the 16 d
  // [hh D/2 + 16 ks, +16) of K row tau(i32) and of Q row 32 rh + i32
  constexpr int KSI = D / 32;
  u32x4 qih[I8QK ? KSI : 1], qil[I8QK ? KSI : 1];
  float qrs = 1.0f;                               // this lane's row scale 2^(e - 7)
  // Stage the group's query rows in LDS and read this lane's operand parts
  // back (called once the first blocks' loads are in flight, so their
  // latency overlaps the query loads).
  auto stage_q = [&]() __attribute__((always_inline)) {
    // Query rows of the group -> LDS (bf16 or fp16 as given, rows padded by 16 bytes); rows past
    // rho are zero. The B operand of S^T = K Q^T is read back per k-step:
    // lane holds row i32 of the wave's rows, d in [hh * D/2 + 8 kk, +8).
    if constexpr (F8QK) {
      // Per (row, 32-d block): x = q 2^-e with max |x| in [128, 256), x = hi +
      // lo / 16 with hi = fp8(x) and lo = fp8(16 (x - hi)). A bf16 q has 8
      // significant bits, hi keeps 4 and the remainder fits the 4 of lo, so the
      // split is exact for every element within 2^13 of the block's maximum;
      // the products then carry the scales 2^e and 2^(e - 4).
      for (int idx = tid; idx < ROWS * (D / 32); idx += NT) {
        const int row = idx / (D / 32), blk = idx - row * (D / 32);
        const int r = rbase + row;
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = 0.0f;
        {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4 w = qpre[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[8 * u + 2 * e] = __uint_as_float(w[e] << 16);
              x[8 * u + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
          }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
        int e = 0;
        if (amax > 0.0f) e = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 7;
        e = e < -123 ? -123 : (e > 127 ? 127 : e);
        const float sc = __builtin_ldexpf(1.0f, -e);
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float a0 = x[4 * k] * sc, a1 = x[4 * k + 1] * sc, a2 = x[4 * k + 2] * sc, a3 = x[4 * k + 3] * sc;
          int h = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
          h = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, h, true);
          const float r0 = 16.0f * (a0 - __builtin_amdgcn_cvt_f32_fp8(h, 0));
          const float r1 = 16.0f * (a1 - __builtin_amdgcn_cvt_f32_fp8(h, 1));
          const float r2 = 16.0f * (a2 - __builtin_amdgcn_cvt_f32_fp8(h, 2));
          const float r3 = 16.0f * (a3 - __builtin_amdgcn_cvt_f32_fp8(h, 3));
          int l = __builtin_amdgcn_cvt_pk_fp8_f32(r0, r1, 0, false);
          l = __builtin_amdgcn_cvt_pk_fp8_f32(r2, r3, l, true);
          hw[k] = (uint32_t)h;
          lw[k] = (uint32_t)l;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          *reinterpret_cast<u32x4*>(&qh_s[row * QS8 + 32 * blk + 16 * u]) =
              u32x4{hw[4 * u], hw[4 * u + 1], hw[4 * u + 2], hw[4 * u + 3]};
          *reinterpret_cast<u32x4*>(&ql_s[row * QS8 + 32 * blk + 16 * u]) =
              u32x4{lw[4 * u], lw[4 * u + 1], lw[4 * u + 2], lw[4 * u + 3]};
        }
        qe_s[(row * (D / 32) + blk) * 2] = (uint8_t)(e + 127);
        qe_s[(row * (D / 32) + blk) * 2 + 1] = (uint8_t)(e - 4 + 127);
      }
    } else if constexpr (I8QK) {
      // Per row: x = q 2^-e with max |x| in [64, 128); hi = rne(x) clamped to
      // [-128, 127], lo = rne(128 (x - hi)), |lo| <= 64, so x = hi + lo / 128
      // exactly for every element within 2^7 of the row's maximum (and within
      // 2^-8 of it otherwise: 2^-14 of the maximum). Thread (row, 32-d block)
      // converts its block; the row's maximum comes from a shuffle over the
      // D / 32 consecutive threads of the row.
      constexpr int NB = D / 32;
      for (int idx = tid; idx < ROWS * NB; idx += NT) {
        const int row = idx / NB, blk = idx - row * NB;
        const int r = rbase + row;
        float x[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = 0.0f;
        {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const u32x4 w = qpre[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[8 * u + 2 * e] = __uint_as_float(w[e] << 16);
              x[8 * u + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
            }
          }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
        for (int o = 1; o < NB; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
        int e = 0;
        if (amax > 0.0f) e = (int)((__float_as_uint(amax) >> 23) & 255u) - 127 - 6;
        e = e < -100 ? -100 : (e > 127 ? 127 : e);
        const float sc = __builtin_ldexpf(1.0f, -e);
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          uint32_t hb = 0, lb = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float a = x[4 * k + i] * sc;
            float hi = __builtin_rintf(a);
            hi = fminf(fmaxf(hi, -128.0f), 127.0f);
            const float lo = __builtin_rintf(128.0f * (a - hi));
            hb |= ((uint32_t)(int32_t)hi & 0xFFu) << (8 * i);
            lb |= ((uint32_t)(int32_t)lo & 0xFFu) << (8 * i);
          }
          hw[k] = hb;
          lw[k] = lb;
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          *reinterpret_cast<u32x4*>(&qh_s[row * QS8 + 32 * blk + 16 * u]) =
              u32x4{hw[4 * u], hw[4 * u + 1], hw[4 * u + 2], hw[4 * u + 3]};
          *reinterpret_cast<u32x4*>(&ql_s[row * QS8 + 32 * blk + 16 * u]) =
              u32x4{lw[4 * u], lw[4 * u + 1], lw[4 * u + 2], lw[4 * u + 3]};
        }
        if (blk == 0) qr_s[row] = __builtin_ldexpf(1.0f, e - 7);
      }
    } else {
      for (int idx = tid; idx < ROWS * (D / 8); idx += NT) {
        const int row = idx / (D / 8), c8 = idx - row * (D / 8);
        const int r = rbase + row;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (r < p.rho) {
          int j, hq;
          row_jh(p, g, r, &j, &hq);
          x = ld16(reinterpret_cast<const uint16_t*>(p.q) + qo_idx(p, b, j, hq, 8 * c8));
        }
        *reinterpret_cast<u32x4*>(&q_s[row * QS + 8 * c8]) = x;
      }
    }
    __syncthreads();
    if constexpr (I8QK) {
      const int qrow = (32 * rh + i32) * QS8 + hh * (D / 2);
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks) {
        if constexpr (D != 256) {
          qih[ks] = *reinterpret_cast<const u32x4*>(&qh_s[qrow + 16 * ks]);
          qil[ks] = *reinterpret_cast<const u32x4*>(&ql_s[qrow + 16 * ks]);
        }
      }
      qrs = qr_s[32 * rh + i32];
    } else if constexpr (!F8QK) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qf[kk] = __builtin_bit_cast(qop, *reinterpret_cast<const u32x4*>(&q_s[qoff0 + 8 * kk]));
    }
    if constexpr (F8QK) {                          // (the split Q rows are in LDS: barrier above)
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const int blk = 2 * ks + hh;
        qsh[ks] = qe_s[((32 * rh + i32) * (D / 32) + blk) * 2];
        qsl[ks] = qe_s[((32 * rh + i32) * (D / 32) + blk) * 2 + 1];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          qa[ks][u] = *reinterpret_cast<const u32x4*>(&qh_s[q8off + 64 * ks + 32 * u]);
          qb[ks][u] = *reinterpret_cast<const u32x4*>(&ql_s[q8off + 64 * ks + 32 * u]);
        }
      }
    }

  };
  // ---- one 32-key block in stage st ------------------------------------------
  // Blocks wholly inside the split and inside every row's visible range skip
  // all masking; on the others (a wave-uniform test) small branches mask
  // logits, V scales and V codes. The matrix-core code is shared by both
  // kinds, so the accumulators keep one register assignment.
  //
  // A block runs in five pieces: the K operand reads (kread), S^T = K Q^T
  // (scores), the V operand reads, scales and logits (prep), the
  // probabilities and their sum (expsum), and the rescale and
  // O^T += V^T P^T (finish).
  constexpr int NKR = F8QK ? 2 * KS8 : (I8QK ? KSI : NCH);
  struct KOp {
    u32x4 r[NKR];
  };
  auto kread = [&](int st) __attribute__((always_inline)) {
    const char* S = ring + st * STAGE;
    KOp k;
    if constexpr (F8QK) {
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int c = 4 * ks + hh + 2 * u;       // 16-byte chunk of the key row
          k.r[2 * ks + u] = *reinterpret_cast<const u32x4*>(S + krow + ((c ^ kswz(tau(i32))) * 16));
        }
    } else if constexpr (I8QK) {
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks) k.r[ks] = *reinterpret_cast<const u32x4*>(S + krow + ((kx ^ ks) * 16));
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) k.r[c] = *reinterpret_cast<const u32x4*>(S + krow + ((kx ^ c) * 16));
    }
    return k;
  };
  // ---- S^T = K Q^T (the first k-step starts from an inline zero accumulator)
  auto scores = [&](const KOp& k) __attribute__((always_inline)) {
    floatx16 s;
    if constexpr (F8QK) {
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks) {
        const u32x4 k0 = k.r[2 * ks], k1 = k.r[2 * ks + 1];
        const i32x8 a = __builtin_bit_cast(i32x8, u32x8{k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]});
        const i32x8 bh = __builtin_bit_cast(i32x8, u32x8{qa[ks][0][0], qa[ks][0][1], qa[ks][0][2], qa[ks][0][3],
                                                             qa[ks][1][0], qa[ks][1][1], qa[ks][1][2], qa[ks][1][3]});
        const i32x8 bl = __builtin_bit_cast(i32x8, u32x8{qb[ks][0][0], qb[ks][0][1], qb[ks][0][2], qb[ks][0][3],
                                                             qb[ks][1][0], qb[ks][1][1], qb[ks][1][2], qb[ks][1][3]});
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bh, ks == 0 ? floatx16{} : s, 0, 0, 0, 127, 0, qsh[ks]);
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, bl, s, 0, 0, 0, 127, 0, qsl[ks]);
      }
    } else if constexpr (I8QK) {
      // int8 codes straight from LDS; S = (S_hi << 7) + S_lo is exact (|S| < 2^30)
      i32x16 sh, sl;
#pragma unroll
      for (int ks = 0; ks < KSI; ++ks) {
        const v4i32 a = __builtin_bit_cast(v4i32, k.r[ks]);
        // at D 256 the two parts are read from LDS per k-step: held in
        // registers they push the kernel past its arch VGPRs, and the
        // compiler then serializes the K operand reads
        u32x4 qh, ql;
        if constexpr (D == 256) {
          qh = *reinterpret_cast<const u32x4*>(&qh_s[(32 * rh + i32) * QS8 + hh * (D / 2) + 16 * ks]);
          ql = *reinterpret_cast<const u32x4*>(&ql_s[(32 * rh + i32) * QS8 + hh * (D / 2) + 16 * ks]);
        } else {
          qh = qih[ks];
          ql = qil[ks];
        }
        sh = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, __builtin_bit_cast(v4i32, qh), ks == 0 ? i32x16{} : sh,
                                                   0, 0, 0);
        sl = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, __builtin_bit_cast(v4i32, ql), ks == 0 ? i32x16{} : sl,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) s[v] = (float)((sh[v] << 7) + sl[v]);
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
#pragma unroll
        for (int h2 = 0; h2 < KPC; ++h2) {
          const int kk = c * KPC + h2;
          qop kf;
          if constexpr (__is_same(QT, F16)) {
            kf = cvt8h<KT>(k.r[c][2 * h2], k.r[c][2 * h2 + 1]);
          } else if constexpr (EB == 1) {
            kf = cvt8<KT>(k.r[c][2 * h2], k.r[c][2 * h2 + 1], 0u, 0u);
          } else {
            kf = cvt8<KT>(k.r[c][0], k.r[c][1], k.r[c][2], k.r[c][3]);
          }
          s = mfma(kf, qf[kk], kk == 0 ? floatx16{} : s);
        }
      }
    }
    return s;
  };
  struct Blk {
    floatx16 t;                                   // logits t = s * c - mu (masked: -inf)
    float pe[16];                                 // probabilities exp2(t) (expsum)
    float lsum, xv, mu;
    int nv;                                       // keys of this lane's 16 inside the split
    bool boundary;
    uint32_t xr[DB][8];                           // V^T operand words
  };
  auto prep = [&](int t0, int st, const floatx16& s, Blk& B) __attribute__((always_inline)) {
    const char* S = ring + st * STAGE;
    B.boundary =
        __builtin_amdgcn_readfirstlane((int)((t0 + 32 > hi) | (t0 < ilo) | (t0 + 32 > ihi) | (TM && t0 + 32 > dbase))) != 0;
    const int kb = 16 * hh;                       // first key of this lane's 16
    // ---- V^T operand reads, ahead of the softmax that hides their latency:
    // xr[db] holds d-block db (transposed V: EB 16-byte key runs; plain V: per
    // key half kh, words 4 kh + [0, 4))
    if constexpr (VT) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          const u32x4 vc = *reinterpret_cast<const u32x4*>(S + KSZ + hh * U * 512 + (db * EB + e) * 512 + i32 * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) B.xr[db][4 * e + q] = vc[q];
        }
    } else {
      // transposing LDS reads: in each 16-lane group (wave half hh, d half mh
      // of a 32-d block), lane i gets 8 (8-bit) or 4 (bf16) consecutive keys
      // of d = 32 db + 16 mh + i; lane r of the group supplies the address of
      // the row segment that the transpose distributes (key 2 j + r / 2 ...)
      const int gi = lane & 15;
      const int mh = (lane >> 4) & 1;
      const char* vg = S + KSZ + hh * VGS;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if constexpr (EB == 1) {
            const int key = 8 * kh + (gi >> 1);
            const int c = 2 * db + mh;
            const char* a8 = vg + key * RB + ((c ^ vswz(key)) * 16) + 8 * (gi & 1);
            const v2i32 t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i32*)(a8));
            B.xr[db][4 * kh] = (uint32_t)t[0];
            B.xr[db][4 * kh + 1] = (uint32_t)t[1];
            B.xr[db][4 * kh + 2] = B.xr[db][4 * kh + 3] = 0u;
          } else {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const int key = 8 * kh + 4 * q + (gi >> 2);
              const int c = 4 * db + 2 * mh + ((gi & 3) >> 1);
              const char* a16 = vg + key * RB + ((c ^ vswz(key)) * 16) + 8 * (gi & 1);
              const v4i16 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (__attribute__((address_space(3))) v4i16*)(a16));
              const u32x2 u = __builtin_bit_cast(u32x2, t);
              B.xr[db][4 * kh + 2 * q] = u[0];
              B.xr[db][4 * kh + 2 * q + 1] = u[1];
            }
          }
        }
      }
    }
    // ---- per-key scales (K scale folded into c, V scale into the probabilities):
    // lane l reads the scales of key kb + l % 16 only; row broadcasts hand
    // each lane those of its 16 keys
    float c[16];
    B.xv = 1.0f;
    B.nv = hi - (t0 + kb);
    if constexpr (QUANT) {
      const float* sc = reinterpret_cast<const float*>(S + KSZ + VSZ);
      const float xk = sc[kb + (lane & 15)] * p.scale_log2;
      B.xv = sc[32 + kb + (lane & 15)];
      if (B.boundary) {
        // the V scales of keys past the split may be NaN: zero them, so masked
        // keys give exactly zero (the empty asm keeps this a branch)
        int n = B.nv;
        asm volatile("" : "+v"(n));
        B.xv = ((lane & 15) < n) ? B.xv : 0.0f;
      }
      if constexpr (I8QK) {
        // the query row's scale 2^(e - 7) rides on the broadcast (v_mul_f32_dpp)
        float qr[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) qr[v] = qrs;
        row_bcast_mul8<0>(xk, qr, c);
        row_bcast_mul8<8>(xk, qr, c);
      } else {
        row_bcast16(xk, c, std::make_integer_sequence<int, 16>{});
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) c[v] = p.scale_log2;
    }
    // ---- logits t = s * c - mu (mu: the running reference maximum), so that
    // the probability is exp2(t); boundary blocks then replace masked logits
    // by -inf with selects (never by multiplying with zero)
    B.mu = (mrun == -INFINITY) ? 0.0f : mrun;
#pragma unroll
    for (int v = 0; v < 16; ++v) B.t[v] = __builtin_fmaf(s[v], c[v], -B.mu);
    if (B.boundary) {
      asm volatile("");
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int k = t0 + kb + v;
        bool vis = (k < hi) & (k >= vlo) & (k < vhi);
        if constexpr (TM) vis &= tree_visible(tmask, k, dbase);
        B.t[v] = vis ? B.t[v] : -INFINITY;
      }
    }
  };
  // ---- probabilities against the current reference
  auto expsum = [&](Blk& B) __attribute__((always_inline)) {
    float lsum = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      B.pe[v] = fexp2(B.t[v]);
      lsum += B.pe[v];
    }
    B.lsum = lsum;
  };
  auto finish = [&](Blk& B) __attribute__((always_inline)) {
    // The reference only rises when a probability would exceed 2^8 (a logit
    // more than 2^8 above it), which a lane's sum above 2^8 reveals without a
    // row maximum (rare: the wave votes first; rows without a reference yet
    // always take that path, which sets it from the row maximum and
    // recomputes the block)
    bf16x8 pf[2];
    {
      float lsum = B.lsum;
      float pv[16];
      const bool need = (mrun == -INFINITY) || !(lsum <= kRescaleLimit);
      if (__any(need)) {
        pin_acc();
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, B.t[v]);
        const float mt = fmaxf(mx, __shfl_xor(mx, 32, 64));   // row max - mu
        const float mnew = fmaxf(mrun, mt + B.mu);
        const float alpha = (mnew == -INFINITY) ? 1.0f : fexp2(mrun - mnew);   // 0 when mrun = -inf
        const float shift = (mnew == -INFINITY) ? 0.0f : mnew - B.mu;
        lrun *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[db][v] *= alpha;
        lsum = 0.0f;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          B.pe[v] = fexp2(B.t[v] - shift);
          lsum += B.pe[v];
        }
        mrun = mnew;
        pin_acc();
      }
      lrun += lsum;
      if constexpr (QUANT) {
        row_bcast_mul8<0>(B.xv, B.pe, pv);
        row_bcast_mul8<8>(B.xv, B.pe, pv);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) pv[v] = B.pe[v];
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const u32x4 pk = {pack_bf16x2(pv[8 * kh], pv[8 * kh + 1]), pack_bf16x2(pv[8 * kh + 2], pv[8 * kh + 3]),
                          pack_bf16x2(pv[8 * kh + 4], pv[8 * kh + 5]), pack_bf16x2(pv[8 * kh + 6], pv[8 * kh + 7])};
        pf[kh] = __builtin_bit_cast(bf16x8, pk);
      }
    }
    // ---- O^T += V^T P^T (V codes of keys past the split zeroed on boundary
    // blocks: they may be NaN-poisoned)
    if (B.boundary) {
      asm volatile("");
      const int nv = B.nv;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        if constexpr (VT) {
#pragma unroll
          for (int q = 0; q < 4 * EB; ++q) B.xr[db][q] = keep_bytes(B.xr[db][q], q * (4 / EB), nv, 4 / EB);
        } else {
          constexpr int PW = 4 / EB;               // keys per word
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int q = 0; q < 2 * EB; ++q)
              B.xr[db][4 * kh + q] = keep_bytes(B.xr[db][4 * kh + q], 8 * kh + q * PW, nv, PW);
        }
      }
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        bf16x8 vf;
        if constexpr (VT && EB == 1) {
          vf = cvt8<KT>(B.xr[db][2 * kh], B.xr[db][2 * kh + 1], 0u, 0u);
        } else {
          vf = cvt8<KT>(B.xr[db][4 * kh], B.xr[db][4 * kh + 1], B.xr[db][4 * kh + 2], B.xr[db][4 * kh + 3]);
        }
        acc[db] = mfma(vf, pf[kh], acc[db]);
      }
    // The accumulators only meet VALU code in the rare rescale and at the
    // end: keep them in one register assignment across blocks.
    pin_acc();
  };
  auto compute = [&](int t0, int st, auto&& mid) __attribute__((always_inline)) {
    const floatx16 s = scores(kread(st));
    mid();                                        // e.g. the next block's loads
    Blk B;
    prep(t0, st, s, B);
    expsum(B);
    finish(B);
  };

  // ---- the key loop ----------------------------------------------------------
  // Key stream sid takes the split's 32-key blocks sid, sid + 4, ...; both
  // row halves of a stream consume every block of it. All waves step together
  // through workgroup barriers (the same number for every wave); each wave
  // first waits for its own loads of the blocks a barrier publishes.
  const int nblk = hi > lo ? (hi - lo + 31) / 32 : 0;
  const int mine = nblk > sid ? (nblk - 1 - sid) / 4 + 1 : 0;
  const int steps = (nblk + 3) / 4;
  auto t0_of = [&](int j) __attribute__((always_inline)) { return lo + (sid + 4 * j) * 32; };
  // Two blocks per barrier with four stages; one block per barrier when the
  // ring holds fewer (D 256, 16-bit codes at D 128).
  if constexpr (NS >= 4) {
    // Two blocks per barrier: it publishes blocks j, j + 1 and frees the
    // stages of j - 2, j - 1, into which j + 2 and j + 3 are loaded while j
    // and j + 1 are computed. The loads of j + 2 go out between the two
    // matrix-core phases of block j and those of j + 3 between the two
    // blocks, so both are in flight through block j + 1's whole step and the
    // waves do not all queue on the vector memory unit at once. Page ids are
    // read one barrier step ahead.
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (j < mine) issue(t0_of(j), load_ids(t0_of(j)), j);
    Ids ids0{0, 0}, ids1{0, 0};
    if (2 < mine) ids0 = load_ids(t0_of(2));
    if (3 < mine) ids1 = load_ids(t0_of(3));
    stage_q();
    for (int j = 0; j < steps; j += 2) {
      wait_vm<0>();                               // blocks j, j + 1: everything this wave issued
      if constexpr (NRH != 1) __syncthreads();
      auto loads0 = [&]() __attribute__((always_inline)) {
        if (j + 2 < mine) issue(t0_of(j + 2), ids0, (j + 2) % NS);
      };
      auto loads1 = [&]() __attribute__((always_inline)) {
        if (j + 3 < mine) issue(t0_of(j + 3), ids1, (j + 3) % NS);
      };
      auto none = []() __attribute__((always_inline)) {};
      if (j < mine)
        compute(t0_of(j), j % NS, loads0);
      else
        loads0();
      loads1();
      if (j + 1 < mine) compute(t0_of(j + 1), (j + 1) % NS, none);
      if (j + 4 < mine) ids0 = load_ids(t0_of(j + 4));
      if (j + 5 < mine) ids1 = load_ids(t0_of(j + 5));
    }
  } else {
    // One block per barrier: it publishes block j and frees the stage of
    // block j - 1, into which block j + NS - 1 is loaded while j is computed.
#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
      if (j < mine) issue(t0_of(j), load_ids(t0_of(j)), j);
    Ids ids{0, 0};                                 // page ids of the next step's block
    if (NS - 1 < mine) ids = load_ids(t0_of(NS - 1));
    stage_q();
    for (int j = 0; j < steps; ++j) {
      {
        const int r = mine - 1 - j;               // own blocks issued after block j: min(r, NS - 2)
        wait_own(r < NS - 2 ? r : NS - 2);
      }
      // With one row half every wave reads only the blocks it loads itself,
      // so its own wait suffices; two row halves share each stream's blocks.
      if constexpr (NRH != 1) __syncthreads();
      const int jn = j + NS - 1;
      auto next_loads = [&]() __attribute__((always_inline)) {
        if (jn < mine) issue(t0_of(jn), ids, jn % NS);
      };
      if (j < mine)
        compute(t0_of(j), j % NS, next_loads);
      else
        next_loads();
      if (jn + 1 < mine) ids = load_ids(t0_of(jn + 1));
    }
  }

  // ---- merge the four streams' states through LDS (stream order) ------------
  const int row = 32 * rh + i32;                  // this lane's row within the group
  const float lrow = lrun + __shfl_xor(lrun, 32, 64);
  if (hh == 0) {
    ml_s[sid][row][0] = mrun;
    ml_s[sid][row][1] = lrow;
  }
  __syncthreads();                                 // every wave is past its key loop
  float wgt;
  {
    float M = -INFINITY;
#pragma unroll
    for (int ss = 0; ss < 4; ++ss)
      if (ml_s[ss][row][1] > 0.0f) M = fmaxf(M, ml_s[ss][row][0]);
    wgt = lrow > 0.0f ? fexp2(mrun - M) : 0.0f;
    if (sid == 0 && hh == 0) {
      float L = 0.0f;
#pragma unroll
      for (int ss = 0; ss < 4; ++ss) {
        const float lw = ml_s[ss][row][1];
        if (lw > 0.0f) L += fexp2(ml_s[ss][row][0] - M) * lw;
      }
      fin_s[row][0] = M;
      fin_s[row][1] = L;
    }
  }
  // Each stream writes its weighted accumulators to its own slice; after one
  // barrier every thread sums the four slices of its outputs in stream order.
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * db + 8 * q + 4 * hh;       // values 4 q .. 4 q + 3: d .. d + 3
      const floatx4 val = {wgt * acc[db][4 * q], wgt * acc[db][4 * q + 1], wgt * acc[db][4 * q + 2],
                           wgt * acc[db][4 * q + 3]};
      *reinterpret_cast<floatx4*>(&acc_s[(sid * ROWS + row) * PD + d]) = val;
    }
  __syncthreads();
  auto merged = [&](int rr, int d) __attribute__((always_inline)) {
    floatx4 v = *reinterpret_cast<const floatx4*>(&acc_s[rr * PD + d]);
#pragma unroll
    for (int ss = 1; ss < 4; ++ss) {
      const floatx4 x = *reinterpret_cast<const floatx4*>(&acc_s[(ss * ROWS + rr) * PD + d]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = v[e] + x[e];
    }
    return v;
  };

  // A request with one split writes its output here (the merge of one record
  // is exactly this finalize, so the result is the same bits) and the
  // combine skips it.
  if (p.finalize || it.S == 1) {
    for (int idx = tid; idx < nrow * (D / 4); idx += NT) {
      const int rr = idx / (D / 4), d = 4 * (idx - rr * (D / 4));
      const int r = rbase + rr;
      int j, hq;
      row_jh(p, g, r, &j, &hq);
      const float s2 = p.has_sink ? p.sinks[hq] * kLog2e : 0.0f;
      const floatx4 v = merged(rr, d);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        store_o1(p, qo_idx(p, b, j, hq, d + e), finalize_one(fin_s[rr][0], fin_s[rr][1], v[e], p.has_sink, s2));
    }
  } else {
    const int64_t slot = (int64_t)it.slot_item * p.Hkv + g;
    for (int idx = tid; idx < nrow * (D / 4); idx += NT) {
      const int rr = idx / (D / 4), d = 4 * (idx - rr * (D / 4));
      const int64_t rec = slot * p.rho + rbase + rr;
      store_rec4(p, rec * D + d, merged(rr, d));
      if (d == 0) {
        p.pm[rec] = fin_s[rr][0];
        p.pl[rec] = fin_s[rr][1];
      }
    }
    if (p.counters) fused_merge_tail(p, it, g, NT);
  }
}

namespace {

template <class QT, class KT, int D, int NRH, bool VT>
void launch_tm(const Params& p, void* stream, int64_t grid) {
  // verify masks get their own instantiation: the plain kernels keep no mask
  // registers and no extra boundary test
  if (p.tree_mask)
    hipLaunchKernelGGL((partial_mfma<QT, KT, D, NRH, VT, true>), dim3((unsigned)grid), dim3(256 * NRH), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((partial_mfma<QT, KT, D, NRH, VT, false>), dim3((unsigned)grid), dim3(256 * NRH), 0,
                       (hipStream_t)stream, p);
}

template <class QT, class KT, int D, int NRH>
int launch_v(const Params& p, void* stream, int64_t grid) {
  if (p.v_layout == SKV_V_TRANSPOSED)
    launch_tm<QT, KT, D, NRH, true>(p, stream, grid);
  else
    launch_tm<QT, KT, D, NRH, false>(p, stream, grid);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

template <class QT, class KT>
int launch_d(const Params& p, int nrh, void* stream, int64_t grid) {
  switch (p.D) {
    case 64: return nrh == 2 ? launch_v<QT, KT, 64, 2>(p, stream, grid) : launch_v<QT, KT, 64, 1>(p, stream, grid);
    case 128: return nrh == 2 ? launch_v<QT, KT, 128, 2>(p, stream, grid) : launch_v<QT, KT, 128, 1>(p, stream, grid);
    case 256:
      if constexpr (Storage<KT>::bytes == 1) return launch_v<QT, KT, 256, 1>(p, stream, grid);
      return SKV_ERR_UNSUPPORTED;
  }
  return SKV_ERR_SHAPE;
}

}  // namespace

bool mfma_supported(const Params& p) {
  // bf16 queries with bf16 or 8-bit KV; fp16 queries with 8-bit KV (a bf16
  // key is not an fp16 value: that pair stays on the vector kernel)
  if (p.q_dtype == SKV_BF16) {
    if (p.kv_dtype != SKV_BF16 && p.kv_dtype != SKV_INT8 && p.kv_dtype != SKV_FP8_E4M3) return false;
  } else if (p.q_dtype == SKV_F16) {
    if (p.kv_dtype != SKV_INT8 && p.kv_dtype != SKV_FP8_E4M3) return false;
  } else {
    return false;
  }
  if (p.D != 64 && p.D != 128 && p.D != 256) return false;
  // a 32-key block of bf16 rows at D = 256 is 32 KiB of K and V: too big for the
  // per-wave LDS ring, so that shape stays on the vector kernel
  if (p.D == 256 && p.kv_dtype == SKV_BF16) return false;
  if (p.paged) return p.block_size >= 16;
  const int eb = p.kv_dtype == SKV_BF16 ? 2 : 1;
  return p.kv_cap % 16 == 0 && mfma_offsets_fit(0, p.v_layout, p.D, p.kv_cap, eb);
}

int launch_partial_mfma(Params p, void* stream) {
  // two row halves (eight waves, two per SIMD) when a KV head has more than
  // 32 query rows; D = 256 keeps one (its accumulators need the registers)
  const int rows = mfma_group_rows(p.D, p.rho);
  const int nrh = rows / 32;
  p.row_groups = (p.rho + rows - 1) / rows;
  const int64_t grid = (int64_t)p.n_items * p.Hkv * p.row_groups;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  if (p.q_dtype == SKV_F16) {
    switch (p.kv_dtype) {
      case SKV_INT8: return launch_d<F16, I8>(p, nrh, stream, grid);
      case SKV_FP8_E4M3: return launch_d<F16, FP8>(p, nrh, stream, grid);
    }
    return SKV_ERR_DTYPE;
  }
  switch (p.kv_dtype) {
    case SKV_BF16: return launch_d<BF16, BF16>(p, nrh, stream, grid);
    case SKV_INT8: return launch_d<BF16, I8>(p, nrh, stream, grid);
    case SKV_FP8_E4M3: return launch_d<BF16, FP8>(p, nrh, stream, grid);
  }
  return SKV_ERR_DTYPE;
}

}  // namespace skv
