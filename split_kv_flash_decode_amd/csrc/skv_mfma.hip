// Matrix-core partial kernel for BF16 queries over BF16, INT8 or FP8 KV.
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
//  * One 256-thread workgroup per (work item, KV head, group of 32*NRB query
//    rows). Its four waves take interleaved 32*TB-key tiles of the item's key
//    range and each keeps its own online-softmax state for all of the group's
//    rows; the four states are merged through LDS at the end, in wave order.
//  * Every query row of a KV head (R * Hq / Hkv rows: GQA heads times MTP or
//    verify rows) shares each key and value a wave loads, so a tile is a
//    dense contraction: S^T = K Q^T and O^T += V^T P^T run on
//    v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//  * K and V go straight from HBM to registers with 16-byte loads; no LDS
//    staging, since no other wave reads them. Key order inside a 32-key block
//    is permuted (tau) so that the S^T output a lane holds is 16 consecutive
//    keys of one query row: exactly the P^T operand the P.V product needs and,
//    for transposed V, exactly 16 contiguous bytes of a V^T row (one load).
//  * FP8 codes become BF16 with v_cvt_scalef32_pk_bf16_fp8 and INT8 codes via
//    fp32, both exactly; the per-token K scale multiplies the logits and the
//    per-token V scale the probabilities, so the only rounding besides fp32
//    accumulation is P -> bf16.
//  * The softmax is online with lazy rescaling: the running maximum of a row
//    is only raised (and acc, l rescaled) when a logit exceeds it by more than
//    2^8, which a wave vote detects; the row max needs one cross-half shuffle.
//  * Tiles that lie wholly inside the split and inside every row's visible
//    range skip all masking; boundary tiles mask logits with selects (never
//    multiply-by-zero, so NaN-poisoned cache slots past a request's context
//    never reach an accumulator) and zero V bytes of keys past the split.

#include <type_traits>

#include "skv_device.h"

namespace skv {

namespace {

// MFMA row i of the K operand of a 32-key block holds key tau(i); then output
// value v of a lane in wave half h is key 16 h + v.
__device__ __forceinline__ int tau(int i) { return ((i & 4) << 2) | ((i >> 1) & 0xC) | (i & 3); }

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

// Element c of a token's V chunk (plain layout) for two tokens -> packed bf16
// pair (token0 in the low half).
template <class KT>
__device__ __forceinline__ uint32_t vpair(uint32_t t0, uint32_t t1, int c) {
  if constexpr (__is_same(KT, FP8)) {
    const uint32_t sel = (uint32_t)(c & 3) | ((uint32_t)(4 + (c & 3)) << 8) | 0x0C0C0000u;
    return fp8x2_to_bf16x2<false>(__builtin_amdgcn_perm(t1, t0, sel));
  } else if constexpr (__is_same(KT, I8)) {
    return pack_bf16x2(i8_to_f32(t0, c & 3), i8_to_f32(t1, c & 3));
  } else {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    return __builtin_amdgcn_perm(t1, t0, sel);
  }
}

__device__ __forceinline__ floatx16 mfma(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

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

template <class KT, int D, int NRB, bool VT>
__global__ __launch_bounds__(256) void partial_mfma(Params p) {
  constexpr int EB = Storage<KT>::bytes;
  constexpr bool QUANT = Storage<KT>::quant;
  constexpr int KS = D / 16;                     // Q.K^T k-steps of 16 d
  constexpr int DB = D / 32;                     // P.V d-blocks of 32
  constexpr int ROWS = 32 * NRB;
  constexpr int RB = D * EB;                     // bytes of one key row
  constexpr int NCH = RB / 32;                   // 1 KiB load chunks of K (and of V) per 32-key block
  constexpr int NI = 2 * NCH + (QUANT ? 1 : 0);  // direct-to-LDS loads per block
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
  constexpr int QBYTES = ROWS * QS * 2;
  constexpr int BUDGET = 156 * 1024;
  constexpr int NS0 = (BUDGET - QBYTES) / (4 * STAGE);
  constexpr int NS = NS0 > 4 ? 4 : (NS0 < 2 ? 2 : NS0);   // ring stages per wave
  constexpr int RING = 4 * NS * STAGE;
  constexpr int PD = D + 1;                      // merge buffer row stride (floats)
  constexpr int MERGE = ROWS * PD * 4;
  constexpr int SMEM0 = RING > MERGE ? RING : MERGE;
  constexpr int VB = (D / 32) * EB;              // plain V: bytes of a lane's d chunk per key

  __shared__ __attribute__((aligned(16))) char smem[SMEM0 + QBYTES];
  __shared__ float ml_s[4][ROWS][2];
  __shared__ float fin_s[ROWS][2];
  uint16_t* q_s = reinterpret_cast<uint16_t*>(smem + SMEM0);
  float* acc_s = reinterpret_cast<float*>(smem);   // reused after the key loop

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int hh = lane >> 5;
  char* ring = smem + w * NS * STAGE;

  int blk = blockIdx.x;
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

  // Query rows of the group -> LDS (bf16, rows padded by 16 bytes); rows past
  // rho are zero. The B operand of S^T = K Q^T is read back per k-step:
  // lane holds row i32 of a row block, d in [hh * D/2 + 8 kk, +8).
  for (int idx = tid; idx < ROWS * (D / 8); idx += 256) {
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
  int vlo[NRB], vhi[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = rbase + rb * 32 + i32;
    vlo[rb] = 0;
    vhi[rb] = 0;
    if (r < p.rho) row_range(ctx, p.R, p.causal, p.window, r / p.G, &vlo[rb], &vhi[rb]);
  }
  // Keys every row of the group sees: [ilo, ihi).
  int ilo, ihi;
  {
    int a0, a1, c0, c1;
    row_range(ctx, p.R, p.causal, p.window, rbase / p.G, &a0, &a1);
    row_range(ctx, p.R, p.causal, p.window, (rbase + nrow - 1) / p.G, &c0, &c1);
    ilo = __builtin_amdgcn_readfirstlane(a0 > c0 ? a0 : c0);
    ihi = __builtin_amdgcn_readfirstlane(a1 < c1 ? a1 : c1);
  }
  __syncthreads();

  floatx16 acc[NRB][DB];
  float mrun[NRB], lrun[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    mrun[rb] = -INFINITY;
    lrun[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[rb][db][v] = 0.0f;
  }

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
  //  K, group gp, load n: lane l fetches 16 bytes of key (l % 16) ^ (8 gp) of
  //    the group at row byte (4 n + l / 16) * 16; the XOR spreads the
  //    consumer's 16-byte LDS reads over all banks.
  //  plain V, load n: row n * (1024 / RB) + l / (RB / 16), 16-byte column
  //    l % (RB / 16) (the group's rows, in key order).
  //  transposed V, load n: unit u = 2 n + l / 32 (d-block u / EB, 16-byte key
  //    run u % EB) of V^T row d = 32 (u / EB) + l % 32.
  uint32_t koffs[2][KIG];
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int n = 0; n < KIG; ++n)
      koffs[gp][n] = (uint32_t)(((lane & 15) ^ (8 * gp)) * RB + (4 * n + (lane >> 4)) * 16);
  constexpr int NVL = VT ? U / 2 : KIG;          // V loads per group
  uint32_t voffs[NVL];
  {
    const int dstride = (p.paged ? (1 << p.bs_shift) : p.kv_cap) * EB;
#pragma unroll
    for (int n = 0; n < NVL; ++n) {
      if constexpr (VT) {
        const int u = 2 * n + (lane >> 5);
        voffs[n] = (uint32_t)((32 * (u / EB) + i32) * dstride + (u % EB) * 16);
      } else {
        constexpr int LPR = RB / 16;
        voffs[n] = (uint32_t)((n * (1024 / RB) + lane / LPR) * RB + (lane % LPR) * 16);
      }
    }
  }

  // Issue the direct-to-LDS loads of the 32-key block at t0 into stage st.
  auto issue = [&](int t0, const Ids& id, int st) __attribute__((always_inline)) {
    const uint32_t S = lds_addr(ring + st * STAGE);
    const int64_t R0 = grp_row(id, t0, 0), R1 = grp_row(id, t0, 1);
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const char* kb = kbase + (gp ? R1 : R0) * RB;
#pragma unroll
      for (int n = 0; n < KIG; ++n) dma16s(kb, koffs[gp][n], S + (gp * KIG + n) * 1024);
    }
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
    if constexpr (QUANT) {
      // lane l < 32: K scale of key l; l >= 32: V scale of key l - 32
      const int k = i32;
      const int64_t r = ((k >= 16) ? R1 : R0) + (k & 15);
      dma4((hh ? p.vs : p.ks) + r, S + KSZ + VSZ);
    }
  };

  // Consumer side of the K layout: key tau(i32) sits in group tau / 16 at
  // position (tau % 16) ^ (8 group); its 16-byte chunk j of the row is at
  // + j * 256.
  const int kread = ((tau(i32) >> 4) * KIG) * 1024 + ((tau(i32) & 15) ^ (8 * (tau(i32) >> 4))) * 16;

  // Logits of one 32-key block: t = s * c - mu, with c = scale * log2(e) *
  // k_scale and mu the running reference maximum, so that the probability is
  // exp2(t). MASK selects the boundary version (causal / window / split end by
  // select, never by multiplying with zero). Returns whether a row's reference
  // must rise (a logit more than 2^8 above it).
  auto logits = [&](auto mask_tag, floatx16 (&s)[NRB], const float (&c)[16], int t0, int kb,
                    float (&mloc)[NRB]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    bool need = false;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mu = (mrun[rb] == -INFINITY) ? 0.0f : mrun[rb];
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float t = __builtin_fmaf(s[rb][v], c[v], -mu);
        if constexpr (MASK) {
          const int k = t0 + kb + v;
          const bool vis = (k < hi) & (k >= vlo[rb]) & (k < vhi[rb]);
          t = vis ? t : -INFINITY;
        }
        s[rb][v] = t;
        mx = fmaxf(mx, t);
      }
      mloc[rb] = mx;
      need |= (mrun[rb] == -INFINITY) ? (mx > -INFINITY) : (mx > kRescaleSlack);
    }
    return need;
  };
  // Probabilities times the V scale as the bf16 P^T operand; l accumulates.
  auto probs = [&](auto mask_tag, const floatx16 (&s)[NRB], const float (&sv)[16],
                   bf16x8 (&pf)[NRB][2]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      float lsum = 0.0f;
      float pv[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pe = fexp2(s[rb][v]);
        lsum += pe;
        if constexpr (QUANT) {
          if constexpr (MASK) {
            pv[v] = pe > 0.0f ? pe * sv[v] : 0.0f;    // NaN scales of masked keys stay out
          } else {
            pv[v] = pe * sv[v];
          }
        } else {
          pv[v] = pe;
        }
      }
      lrun[rb] += lsum;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const u32x4 pk = {pack_bf16x2(pv[8 * kh], pv[8 * kh + 1]), pack_bf16x2(pv[8 * kh + 2], pv[8 * kh + 3]),
                          pack_bf16x2(pv[8 * kh + 4], pv[8 * kh + 5]), pack_bf16x2(pv[8 * kh + 6], pv[8 * kh + 7])};
        pf[rb][kh] = __builtin_bit_cast(bf16x8, pk);
      }
    }
  };
  // Raise the references of rows whose logits exceeded them (rare: the wave
  // votes first); alpha = 1 and shift = 0 leave the other rows unchanged.
  auto rescale = [&](floatx16 (&s)[NRB], const float (&mloc)[NRB]) __attribute__((always_inline)) {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(acc[rb][db]));
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const float mu = (mrun[rb] == -INFINITY) ? 0.0f : mrun[rb];
      const float mt = fmaxf(mloc[rb], __shfl_xor(mloc[rb], 32, 64));   // row max - mu
      const float mnew = fmaxf(mrun[rb], mt + mu);
      const float alpha = (mnew == -INFINITY) ? 1.0f : fexp2(mrun[rb] - mnew);   // 0 when mrun = -inf
      const float shift = (mnew == -INFINITY) ? 0.0f : mnew - mu;
      lrun[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[rb][db][v] *= alpha;
#pragma unroll
      for (int v = 0; v < 16; ++v) s[rb][v] -= shift;
      mrun[rb] = mnew;
    }
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(acc[rb][db]));
  };

  auto compute = [&](int t0, int st) __attribute__((always_inline)) {
    const char* S = ring + st * STAGE;
    const bool interior =
        __builtin_amdgcn_readfirstlane((int)((t0 + 32 <= hi) && (t0 >= ilo) && (t0 + 32 <= ihi))) != 0;
    const int kb = 16 * hh;                       // first key of this lane's 16
    // ---- S^T = K Q^T for this 32-key block
    floatx16 s[NRB];
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[rb][v] = 0.0f;
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) asm volatile("" : "+v"(s[rb]));
    int qoff = i32 * QS + hh * (D / 2);
    asm volatile("" : "+v"(qoff));                // re-read Q from LDS every block
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4 kc = *reinterpret_cast<const u32x4*>(S + kread + (hh * NCH + c) * 256);
      constexpr int KPC = 16 / (8 * EB);          // k-steps per 16-byte chunk
#pragma unroll
      for (int h2 = 0; h2 < KPC; ++h2) {
        const int kk = c * KPC + h2;
        bf16x8 kf;
        if constexpr (EB == 1) {
          kf = cvt8<KT>(kc[2 * h2], kc[2 * h2 + 1], 0u, 0u);
        } else {
          kf = cvt8<KT>(kc[0], kc[1], kc[2], kc[3]);
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const bf16x8 qf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&q_s[qoff + rb * 32 * QS + 8 * kk]));
          s[rb] = mfma(kf, qf, s[rb]);
        }
      }
    }
    // S feeds VALU code: keep it in VGPRs (the MFMA writes them directly).
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) asm volatile("" : "+v"(s[rb]));
    // ---- per-key scales (K scale folded into c, V scale into the probabilities)
    float c[16], sv[16];
    if constexpr (QUANT) {
      const float* sc = reinterpret_cast<const float*>(S + KSZ + VSZ);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(sc + kb + 4 * q);
        const floatx4 z = *reinterpret_cast<const floatx4*>(sc + 32 + kb + 4 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          c[4 * q + e] = a[e] * p.scale_log2;
          sv[4 * q + e] = z[e];
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        c[v] = p.scale_log2;
        sv[v] = 1.0f;
      }
    }
    float mloc[NRB];
    const bool need = interior ? logits(std::false_type{}, s, c, t0, kb, mloc)
                               : logits(std::true_type{}, s, c, t0, kb, mloc);
    if (__any(need)) rescale(s, mloc);
    bf16x8 pf[NRB][2];
    if (interior)
      probs(std::false_type{}, s, sv, pf);
    else
      probs(std::true_type{}, s, sv, pf);
    // ---- O^T += V^T P^T
    const int nv = hi - (t0 + kb);                // keys of this lane's 16 inside the split
    if constexpr (VT) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        uint32_t x[4 * EB];
#pragma unroll
        for (int e = 0; e < EB; ++e) {
          const u32x4 vc = *reinterpret_cast<const u32x4*>(S + KSZ + hh * U * 512 + (db * EB + e) * 512 + i32 * 16);
#pragma unroll
          for (int q = 0; q < 4; ++q) x[4 * e + q] = vc[q];
        }
        if (!interior) {
#pragma unroll
          for (int q = 0; q < 4 * EB; ++q) x[q] = keep_bytes(x[q], q * (4 / EB), nv, 4 / EB);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          bf16x8 vf;
          if constexpr (EB == 1) {
            vf = cvt8<KT>(x[2 * kh], x[2 * kh + 1], 0u, 0u);
          } else {
            vf = cvt8<KT>(x[4 * kh], x[4 * kh + 1], x[4 * kh + 2], x[4 * kh + 3]);
          }
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[rb][db] = mfma(vf, pf[rb][kh], acc[rb][db]);
        }
      }
    } else {
      constexpr int VPW = VB >= 4 ? VB / 4 : 1;
      uint32_t vr[16][VPW];
      const char* vrow = S + KSZ + hh * VGS + VB * i32;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const char* src = vrow + e * RB;
        if constexpr (VB == 2) {
          vr[e][0] = *reinterpret_cast<const uint16_t*>(src);
        } else if constexpr (VB == 4) {
          vr[e][0] = *reinterpret_cast<const uint32_t*>(src);
        } else if constexpr (VB == 8) {
          const u32x2 x = *reinterpret_cast<const u32x2*>(src);
          vr[e][0] = x[0];
          vr[e][1] = x[1];
        } else {
          const u32x4 x = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
          for (int q = 0; q < 4; ++q) vr[e][q] = x[q];
        }
      }
      if (!interior) {                            // keys past the split may be NaN-poisoned
#pragma unroll
        for (int e = 0; e < 16; ++e)
#pragma unroll
          for (int q = 0; q < VPW; ++q) vr[e][q] = (e < nv) ? vr[e][q] : 0u;
      }
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int wi = (EB == 1) ? (db >> 2) : (db >> 1);
          u32x4 rr;
#pragma unroll
          for (int u = 0; u < 4; ++u) rr[u] = vpair<KT>(vr[8 * kh + 2 * u][wi], vr[8 * kh + 2 * u + 1][wi], db);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, rr);
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[rb][db] = mfma(vf, pf[rb][kh], acc[rb][db]);
        }
      }
    }
    // The accumulators only meet VALU code in the rare rescale and at the
    // end: keep them in AGPRs across blocks.
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
      for (int db = 0; db < DB; ++db) asm volatile("" : "+a"(acc[rb][db]));
  };

  // ---- the key loop: this wave's 32-key blocks w, w + 4, ... of the split,
  // NS - 1 blocks in flight ahead of the one being computed. Page ids are read
  // two blocks before their loads are issued (two alternating sets, so no
  // copy forces an early wait on a scalar load).
  const int nblk = hi > lo ? (hi - lo + 31) / 32 : 0;
  const int mine = nblk > w ? (nblk - 1 - w) / 4 + 1 : 0;
  auto t0_of = [&](int j) __attribute__((always_inline)) { return lo + (w + 4 * j) * 32; };
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < mine) issue(t0_of(j), load_ids(t0_of(j)), j);
  Ids ids_a{0, 0}, ids_b{0, 0};
  if (NS - 1 < mine) ids_a = load_ids(t0_of(NS - 1));
  if (NS < mine) ids_b = load_ids(t0_of(NS));
  auto step = [&](int j, Ids& ids) __attribute__((always_inline)) {
    const int jn = j + NS - 1;
    if (jn < mine) issue(t0_of(jn), ids, jn % NS);
    const int later = (mine - 1 - j) < (NS - 1) ? (mine - 1 - j) : (NS - 1);
    if (later >= 3) wait_vm<3 * NI>();
    else if (later == 2) wait_vm<2 * NI>();
    else if (later == 1) wait_vm<NI>();
    else wait_vm<0>();
    compute(t0_of(j), j % NS);
    if (jn + 2 < mine) ids = load_ids(t0_of(jn + 2));
  };
  for (int j = 0; j < mine; j += 2) {
    step(j, ids_a);
    if (j + 1 < mine) step(j + 1, ids_b);
  }

  // ---- merge the four waves' states through LDS (wave order) -------------------
  float lrow[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    lrow[rb] = lrun[rb] + __shfl_xor(lrun[rb], 32, 64);
    if (hh == 0) {
      ml_s[w][rb * 32 + i32][0] = mrun[rb];
      ml_s[w][rb * 32 + i32][1] = lrow[rb];
    }
  }
  __syncthreads();                                 // every wave is past its key loop
  float wgt[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int row = rb * 32 + i32;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww)
      if (ml_s[ww][row][1] > 0.0f) M = fmaxf(M, ml_s[ww][row][0]);
    wgt[rb] = lrow[rb] > 0.0f ? fexp2(mrun[rb] - M) : 0.0f;
    if (w == 0 && hh == 0) {
      float L = 0.0f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float lw = ml_s[ww][row][1];
        if (lw > 0.0f) L += fexp2(ml_s[ww][row][0] - M) * lw;
      }
      fin_s[row][0] = M;
      fin_s[row][1] = L;
    }
  }
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int di = 8 * (v >> 2) + 4 * hh + (v & 3);
            const int d = VT ? 32 * db + di : (D / 32) * di + db;
            const int idx = (rb * 32 + i32) * PD + d;
            const float val = wgt[rb] * acc[rb][db][v];
            acc_s[idx] = (ww == 0) ? val : acc_s[idx] + val;
          }
        }
      }
    }
    __syncthreads();
  }

  if (p.finalize) {
    for (int idx = tid; idx < nrow * D; idx += 256) {
      const int row = idx / D, d = idx - (idx / D) * D;
      const int r = rbase + row;
      int j, hq;
      row_jh(p, g, r, &j, &hq);
      const float s2 = p.has_sink ? p.sinks[hq] * kLog2e : 0.0f;
      store_o1(p, qo_idx(p, b, j, hq, d),
               finalize_one(fin_s[row][0], fin_s[row][1], acc_s[row * PD + d], p.has_sink, s2));
    }
  } else {
    const int64_t slot = (int64_t)it.slot_item * p.Hkv + g;
    for (int idx = tid; idx < nrow * D; idx += 256) {
      const int row = idx / D, d = idx - (idx / D) * D;
      const int64_t rec = slot * p.rho + rbase + row;
      p.pacc[rec * D + d] = acc_s[row * PD + d];
      if (d == 0) {
        p.pm[rec] = fin_s[row][0];
        p.pl[rec] = fin_s[row][1];
      }
    }
  }
}

namespace {

template <class KT, int D, int NRB>
int launch_v(const Params& p, void* stream, int64_t grid) {
  if (p.v_layout == SKV_V_TRANSPOSED)
    hipLaunchKernelGGL((partial_mfma<KT, D, NRB, true>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((partial_mfma<KT, D, NRB, false>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

template <class KT>
int launch_d(const Params& p, int nrb, void* stream, int64_t grid) {
  switch (p.D) {
    case 64: return nrb == 2 ? launch_v<KT, 64, 2>(p, stream, grid) : launch_v<KT, 64, 1>(p, stream, grid);
    case 128: return nrb == 2 ? launch_v<KT, 128, 2>(p, stream, grid) : launch_v<KT, 128, 1>(p, stream, grid);
    case 256:
      if constexpr (Storage<KT>::bytes == 1) return launch_v<KT, 256, 1>(p, stream, grid);
      return SKV_ERR_UNSUPPORTED;
  }
  return SKV_ERR_SHAPE;
}

}  // namespace

bool mfma_supported(const Params& p) {
  if (p.q_dtype != SKV_BF16) return false;
  if (p.kv_dtype != SKV_BF16 && p.kv_dtype != SKV_INT8 && p.kv_dtype != SKV_FP8_E4M3) return false;
  if (p.D != 64 && p.D != 128 && p.D != 256) return false;
  // a 32-key block of bf16 rows at D = 256 is 32 KiB of K and V: too big for the
  // per-wave LDS ring, so that shape stays on the vector kernel
  if (p.D == 256 && p.kv_dtype == SKV_BF16) return false;
  if (p.paged) return p.block_size >= 16;
  return p.kv_cap % 16 == 0;
}

int launch_partial_mfma(Params p, void* stream) {
  const int nrb = (p.D == 256 || p.rho <= 32) ? 1 : 2;
  const int rows = 32 * nrb;
  p.row_groups = (p.rho + rows - 1) / rows;
  const int64_t grid = (int64_t)p.n_items * p.Hkv * p.row_groups;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  switch (p.kv_dtype) {
    case SKV_BF16: return launch_d<BF16>(p, nrb, stream, grid);
    case SKV_INT8: return launch_d<I8>(p, nrb, stream, grid);
    case SKV_FP8_E4M3: return launch_d<FP8>(p, nrb, stream, grid);
  }
  return SKV_ERR_DTYPE;
}

}  // namespace skv
