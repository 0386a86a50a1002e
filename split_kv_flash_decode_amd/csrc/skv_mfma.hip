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

template <class KT, int D, int NRB, bool VT>
__global__ __launch_bounds__(256) void partial_mfma(Params p) {
  constexpr int EB = Storage<KT>::bytes;
  constexpr bool QUANT = Storage<KT>::quant;
  constexpr int TB = (D * EB <= 128 && NRB == 1) ? 2 : 1;   // 32-key blocks per tile
  constexpr int T = 32 * TB;                     // keys per tile
  constexpr int KS = D / 16;                     // Q.K^T k-steps of 16 d
  constexpr int DB = D / 32;                     // P.V d-blocks of 32
  constexpr int KW = D * EB / 8;                 // dwords of a lane's half K row
  constexpr int ROWS = 32 * NRB;
  constexpr int PD = D + 1;                      // LDS row stride (floats)
  constexpr int VTW = 4 * EB;                    // dwords of 16 transposed keys
  constexpr int VB = (D / 32) * EB;              // bytes of a plain V chunk per key
  constexpr int VPW = VB >= 4 ? VB / 4 : 1;      // dwords of that chunk
  constexpr int VW = VT ? DB * VTW : 16 * VPW;   // V dwords per key block per lane
  constexpr bool PF = TB * (KW + VW) <= 64;      // double-buffer raw tiles in registers

  struct Raw {
    uint32_t k[TB][KW];
    uint32_t v[TB][VW];
    float sk, sv;
  };
  struct Ids {       // pool pages of the tile's keys (page size >= 16, tile <= 64 keys)
    int p0, p1, p2, p3;
  };

  __shared__ float acc_s[ROWS * PD];
  __shared__ float ml_s[4][ROWS][2];
  __shared__ float fin_s[ROWS][2];
  __shared__ float sc_s[4][2][T];
  constexpr int QS = D + 8;                      // LDS row stride of Q (bf16), padded
  __shared__ __attribute__((aligned(16))) uint16_t q_s[ROWS * QS];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int i32 = lane & 31;
  const int hh = lane >> 5;

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
  __syncthreads();
  // Keys every row of the group sees: [ilo, ihi).
  int ilo, ihi;
  {
    int a0, a1, c0, c1;
    row_range(ctx, p.R, p.causal, p.window, rbase / p.G, &a0, &a1);
    row_range(ctx, p.R, p.causal, p.window, (rbase + nrow - 1) / p.G, &c0, &c1);
    ilo = a0 > c0 ? a0 : c0;
    ihi = a1 < c1 ? a1 : c1;
  }

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
  const int bs_mask = (1 << p.bs_shift) - 1;

  // Page ids of the tile at t0 (scalar loads; entries past the split are not read).
  auto load_ids = [&](int t0) __attribute__((always_inline)) {
    Ids id{0, 0, 0, 0};
    if (p.paged) {
      const int base = t0 >> p.bs_shift;
      const int bs = 1 << p.bs_shift;
      id.p0 = trow[base];
      id.p1 = (bs < T && t0 + bs < hi) ? trow[base + 1] : id.p0;
      id.p2 = (2 * bs < T && t0 + 2 * bs < hi) ? trow[base + 2] : id.p0;
      id.p3 = (3 * bs < T && t0 + 3 * bs < hi) ? trow[base + 3] : id.p0;
    }
    return id;
  };
  auto pick = [&](const Ids& id, int kk) __attribute__((always_inline)) {
    const int x = kk >> p.bs_shift;
    const int a = (x & 1) ? id.p1 : id.p0;
    const int c = (x & 1) ? id.p3 : id.p2;
    return (x & 2) ? c : a;
  };
  // Raw K, V codes and scales of the tile at t0. Keys at or past hi are
  // redirected to key t0 (inside the split) so that no page past the
  // request's context is ever addressed.
  auto load_raw = [&](int t0, const Ids& id) __attribute__((always_inline)) {
    Raw r;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      int kk = tb * 32 + tau(i32);
      if (t0 + kk >= hi) kk = 0;
      const char* src = kbase + (k_row(p, pick(id, kk), b, g, t0 + kk) + hh * (D / 2)) * EB;
#pragma unroll
      for (int c = 0; c < KW / 4; ++c) {
        const u32x4 x = ld16(src + 16 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) r.k[tb][4 * c + e] = x[e];
      }
      if constexpr (VT) {
        int gk = tb * 32 + 16 * hh;
        if (t0 + gk >= hi) gk = 0;
        const int pg = pick(id, gk);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* vs = vbase + vt_idx(p, pg, b, g, 32 * db + i32, t0 + gk) * EB;
#pragma unroll
          for (int c = 0; c < VTW / 4; ++c) {
            const u32x4 x = ld16(vs + 16 * c);
#pragma unroll
            for (int e = 0; e < 4; ++e) r.v[tb][db * VTW + 4 * c + e] = x[e];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          int kv = tb * 32 + 16 * hh + e;
          if (t0 + kv >= hi) kv = 0;
          const char* vs = vbase + (k_row(p, pick(id, kv), b, g, t0 + kv) + (D / 32) * i32) * EB;
          if constexpr (VB == 2) {
            r.v[tb][e] = *reinterpret_cast<const uint16_t*>(vs);
          } else if constexpr (VB == 4) {
            r.v[tb][e] = *reinterpret_cast<const uint32_t*>(vs);
          } else if constexpr (VB == 8) {
            const u32x2 x = *reinterpret_cast<const u32x2*>(vs);
            r.v[tb][2 * e] = x[0];
            r.v[tb][2 * e + 1] = x[1];
          } else {
            const u32x4 x = ld16(vs);
#pragma unroll
            for (int q = 0; q < 4; ++q) r.v[tb][4 * e + q] = x[q];
          }
        }
      }
    }
    if constexpr (QUANT) {
      int kk = lane & (T - 1);
      if (t0 + kk >= hi) kk = 0;
      const int64_t si = scale_idx(p, pick(id, kk), b, g, t0 + kk);
      r.sk = p.ks[si];
      r.sv = p.vs[si];
    } else {
      r.sk = 1.0f;
      r.sv = 1.0f;
    }
    return r;
  };

  auto compute = [&](const Raw& r, int t0) __attribute__((always_inline)) {
    const bool interior = (t0 + T <= hi) && (t0 >= ilo) && (t0 + T <= ihi);
    if constexpr (QUANT) {
      if (lane < T) {
        sc_s[w][0][lane] = r.sk * p.scale_log2;
        sc_s[w][1][lane] = r.sv;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int kb = tb * 32 + 16 * hh;        // first key (in the tile) of this lane's 16
      // ---- S^T = K Q^T for this 32-key block
      floatx16 s[NRB];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[rb][v] = 0.0f;
      int qoff = i32 * QS + hh * (D / 2);
      asm volatile("" : "+v"(qoff));          // re-read Q from LDS every block
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        bf16x8 kf;
        if constexpr (EB == 1) {
          kf = cvt8<KT>(r.k[tb][2 * kk], r.k[tb][2 * kk + 1], 0u, 0u);
        } else {
          kf = cvt8<KT>(r.k[tb][4 * kk], r.k[tb][4 * kk + 1], r.k[tb][4 * kk + 2], r.k[tb][4 * kk + 3]);
        }
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const bf16x8 qf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&q_s[qoff + rb * 32 * QS + 8 * kk]));
          s[rb] = mfma(kf, qf, s[rb]);
        }
      }
      // ---- logits and masks
      float c[16], sv[16];
      if constexpr (QUANT) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const floatx4 a = *reinterpret_cast<const floatx4*>(&sc_s[w][0][kb + 4 * q]);
          const floatx4 z = *reinterpret_cast<const floatx4*>(&sc_s[w][1][kb + 4 * q]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            c[4 * q + e] = a[e];
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
      bool need = false;
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = s[rb][v] * c[v];
          if (!interior) {
            const int t = t0 + kb + v;
            const bool vis = t < hi && t >= vlo[rb] && t < vhi[rb];
            x = vis ? x : -INFINITY;
          }
          s[rb][v] = x;
          mx = fmaxf(mx, x);
        }
        mloc[rb] = mx;
        need |= mx > mrun[rb] + kRescaleSlack;
      }
      // ---- lazy rescale: raise the reference max only when it is exceeded by > 2^8
      if (__any(need)) {
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
          const float mt = fmaxf(mloc[rb], __shfl_xor(mloc[rb], 32, 64));
          const float mnew = fmaxf(mrun[rb], mt);
          const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
          const float alpha = fexp2(mrun[rb] - mu);
          lrun[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[rb][db][v] *= alpha;
          mrun[rb] = mnew;
        }
      }
      // ---- probabilities (times the V scale) as the bf16 P^T operand
      bf16x8 pf[NRB][2];
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb) {
        const float mu = (mrun[rb] == -INFINITY) ? 0.0f : mrun[rb];
        float lsum = 0.0f;
        float pv[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float pe = fexp2(s[rb][v] - mu);
          lsum += pe;
          if constexpr (QUANT) {
            pv[v] = interior ? pe * sv[v] : (pe > 0.0f ? pe * sv[v] : 0.0f);
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
      // ---- O^T += V^T P^T
      const int nv = hi - (t0 + kb);          // keys of this lane's 16 inside the split
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          bf16x8 vf;
          if constexpr (VT) {
            uint32_t x[4];
            if constexpr (EB == 1) {
#pragma unroll
              for (int c2 = 0; c2 < 2; ++c2) {
                const int wi = 2 * kh + c2;
                x[c2] = interior ? r.v[tb][db * VTW + wi] : keep_bytes(r.v[tb][db * VTW + wi], 4 * wi, nv, 4);
              }
              vf = cvt8<KT>(x[0], x[1], 0u, 0u);
            } else {
#pragma unroll
              for (int c2 = 0; c2 < 4; ++c2) {
                const int wi = 4 * kh + c2;
                x[c2] = interior ? r.v[tb][db * VTW + wi] : keep_bytes(r.v[tb][db * VTW + wi], 2 * wi, nv, 2);
              }
              vf = cvt8<KT>(x[0], x[1], x[2], x[3]);
            }
          } else {
            const int wi = (EB == 1) ? (db >> 2) : (db >> 1);
            u32x4 rr;
#pragma unroll
            for (int u = 0; u < 4; ++u)
              rr[u] = vpair<KT>(r.v[tb][(8 * kh + 2 * u) * VPW + wi], r.v[tb][(8 * kh + 2 * u + 1) * VPW + wi], db);
            vf = __builtin_bit_cast(bf16x8, rr);
          }
#pragma unroll
          for (int rb = 0; rb < NRB; ++rb) acc[rb][db] = mfma(vf, pf[rb][kh], acc[rb][db]);
        }
      }
    }
  };

  const int ntiles = hi > lo ? (hi - lo + T - 1) / T : 0;
  if constexpr (PF) {
    int ti = w;
    Raw cur, nxt;
    Ids ids2;
    if (ti < ntiles) cur = load_raw(lo + ti * T, load_ids(lo + ti * T));
    if (ti + 4 < ntiles) ids2 = load_ids(lo + (ti + 4) * T);
    for (; ti < ntiles; ti += 4) {
      const int t0 = lo + ti * T;
      const bool has1 = ti + 4 < ntiles;
      const bool has2 = ti + 8 < ntiles;
      if (has1) nxt = load_raw(t0 + 4 * T, ids2);
      if (has2) ids2 = load_ids(t0 + 8 * T);
      compute(cur, t0);
      if (has1) cur = nxt;
    }
  } else {
    for (int ti = w; ti < ntiles; ti += 4) {
      const int t0 = lo + ti * T;
      const Raw cur = load_raw(t0, load_ids(t0));
      compute(cur, t0);
    }
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
  __syncthreads();
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
    case 256: return launch_v<KT, 256, 1>(p, stream, grid);
  }
  return SKV_ERR_SHAPE;
}

}  // namespace

bool mfma_supported(const Params& p) {
  if (p.q_dtype != SKV_BF16) return false;
  if (p.kv_dtype != SKV_BF16 && p.kv_dtype != SKV_INT8 && p.kv_dtype != SKV_FP8_E4M3) return false;
  if (p.D != 64 && p.D != 128 && p.D != 256) return false;
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
