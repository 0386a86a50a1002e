// Vector-ALU partial kernel: the general path (any Q and KV dtype, fp32 KV
// included) and the one used for few query rows per KV head.
//
// One wave (64 lanes) per (work item, KV head, chunk of up to 8 query rows).
// A work item is one split of one request, or the whole request in
// single-pass mode, where the record is finalized in place. The design record
// of tiny-llm #11 ("split-KV decode attention design record", section
// "Design") lays the partial kernel out over (head, split): each split finds
// its own key range from the visible length held on the device, with a chunk
// length of the visible keys divided by the split count, rounded up, and
// writes its own running maximum, sum and weighted values.
//
// Per 64-key tile: lane t owns key t for Q.K^T (its K row is read with
// 16-byte loads and dequantized in registers, Q comes from LDS as broadcasts);
// the tile's masked logits go through an exact online softmax with wave
// butterflies for the row max and sum; then lanes switch to owning d for
// P.V, walking the tile's keys with the probabilities (times the V scale)
// broadcast from LDS.

#include "skv_device.h"

namespace skv {

namespace {

constexpr int RC = kValuRows;   // query rows per wave

template <class QT>
__device__ __forceinline__ float load_q(const void* q, int64_t idx) {
  if constexpr (Storage<QT>::bytes == 4) {
    return reinterpret_cast<const float*>(q)[idx];
  } else if constexpr (__is_same(QT, F16)) {
    return (float)reinterpret_cast<const _Float16*>(q)[idx];
  } else {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q)[idx]);
  }
}

// 16 bytes of a K row -> VEC fp32 values (codes for quantized types).
template <class KT>
struct Vec {
  static constexpr int n = 16 / Storage<KT>::bytes;
};

template <class KT>
__device__ __forceinline__ void load16(const void* base, int64_t elem, float* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(base) +
                                                  elem * Storage<KT>::bytes);
  if constexpr (Storage<KT>::bytes == 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
  } else if constexpr (Storage<KT>::bytes == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else if constexpr (__is_same(KT, FP8)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx2 a = fp8x2_to_f32<false>(w[i]);
      floatx2 b = fp8x2_to_f32<true>(w[i]);
      out[4 * i] = a[0];
      out[4 * i + 1] = a[1];
      out[4 * i + 2] = b[0];
      out[4 * i + 3] = b[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * i + e] = i8_to_f32(w[i], e);
  }
}

template <class KT>
__device__ __forceinline__ float load1(const void* base, int64_t elem) {
  if constexpr (Storage<KT>::bytes == 4) {
    return reinterpret_cast<const float*>(base)[elem];
  } else if constexpr (Storage<KT>::bytes == 2) {
    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(base)[elem]);
  } else if constexpr (__is_same(KT, FP8)) {
    uint32_t c = reinterpret_cast<const uint8_t*>(base)[elem];
    return fp8x2_to_f32<false>(c)[0];
  } else {
    return (float)reinterpret_cast<const int8_t*>(base)[elem];
  }
}

}  // namespace

template <class QT, class KT, int D, bool VT>
__global__ __launch_bounds__(64) void partial_valu(Params p) {
  constexpr int DPL = D / 64;
  constexpr int VEC = Vec<KT>::n;
  constexpr bool QUANT = Storage<KT>::quant;
  __shared__ float q_s[RC][D];
  __shared__ floatx4 p_s[64][RC / 4];

  const int lane = threadIdx.x;
  const int nrc = (p.rho + RC - 1) / RC;
  int blk = blockIdx.x;
  const int rc = blk % nrc;
  blk /= nrc;
  const int g = blk % p.Hkv;
  const int item = blk / p.Hkv;
  Item it;
  if (!decode_item(p, item, &it)) return;
  const int b = it.b;
  const int ctx = clamp_ctx(p, b);
  int lo, hi;
  split_range(ctx, p.R, p.causal, p.window, it.S, it.s, &lo, &hi);
  const int r0 = rc * RC;

  for (int i = lane; i < RC * D; i += 64) {
    const int rr = i / D, d = i - (i / D) * D, r = r0 + rr;
    float x = 0.0f;
    if (r < p.rho) {
      int j, h;
      row_jh(p, g, r, &j, &h);
      x = load_q<QT>(p.q, qo_idx(p, b, j, h, d));
    }
    q_s[rr][d] = x;
  }
  int vlo[RC], vhi[RC];
  const uint64_t* tm[RC];                       // rows' verify mask words (with masks)
  const int dbase = p.tree_mask ? ctx - p.R : 0x7FFFFFFF;
#pragma unroll
  for (int rr = 0; rr < RC; ++rr) {
    vlo[rr] = 0;
    vhi[rr] = 0;
    tm[rr] = p.tree_mask;
    if (r0 + rr < p.rho) {
      row_range(ctx, p.R, p.causal, p.window, (r0 + rr) / p.G, &vlo[rr], &vhi[rr]);
      if (p.tree_mask) tm[rr] = p.tree_mask + ((int64_t)b * p.R + (r0 + rr) / p.G) * verify_words(p.R);
    }
  }
  float m[RC], l[RC], acc[RC][DPL];
#pragma unroll
  for (int rr = 0; rr < RC; ++rr) {
    m[rr] = -INFINITY;
    l[rr] = 0.0f;
#pragma unroll
    for (int k = 0; k < DPL; ++k) acc[rr][k] = 0.0f;
  }
  __syncthreads();

  for (int t0 = lo; t0 < hi; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < hi;
    const int tt = valid ? t : lo;            // never look past the request's pages
    const int page = page_of(p, b, tt);
    float sc[RC];
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) sc[rr] = 0.0f;
    const int64_t krow = k_row(p, page, b, g, tt);
#pragma unroll 2
    for (int d0 = 0; d0 < D; d0 += VEC) {
      float kv[VEC];
      load16<KT>(p.k, krow + d0, kv);
#pragma unroll
      for (int rr = 0; rr < RC; ++rr) {
#pragma unroll
        for (int e = 0; e < VEC; e += 4) {
          const floatx4 qv = *reinterpret_cast<const floatx4*>(&q_s[rr][d0 + e]);
          sc[rr] += qv[0] * kv[e] + qv[1] * kv[e + 1] + qv[2] * kv[e + 2] + qv[3] * kv[e + 3];
        }
      }
    }
    float ksc = 1.0f, vsc = 1.0f;
    if constexpr (QUANT) {
      const int64_t si = scale_idx(p, page, b, g, tt);
      ksc = p.ks[si];
      vsc = p.vs[si];
    }
    float pr[RC];
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) {
      float x = sc[rr] * ksc * p.scale_log2;
      const bool vis = valid && t >= vlo[rr] && t < vhi[rr] && tree_visible_mem(tm[rr], t, dbase);
      x = vis ? x : -INFINITY;
      const float mt = wave_max(x);
      const float mn = fmaxf(m[rr], mt);
      const float mu = (mn == -INFINITY) ? 0.0f : mn;
      const float alpha = fexp2(m[rr] - mu);
      const float pe = fexp2(x - mu);
      l[rr] = l[rr] * alpha + wave_sum(pe);
      m[rr] = mn;
#pragma unroll
      for (int k = 0; k < DPL; ++k) acc[rr][k] *= alpha;
      pr[rr] = vis ? pe * vsc : 0.0f;
    }
    p_s[lane][0] = floatx4{pr[0], pr[1], pr[2], pr[3]};
    p_s[lane][1] = floatx4{pr[4], pr[5], pr[6], pr[7]};
    __syncthreads();
    const int n = (hi - t0) < 64 ? (hi - t0) : 64;
    for (int i = 0; i < n; ++i) {
      const int tok = t0 + i;
      const int pg = __shfl(page, i, 64);
      const floatx4 pa = p_s[i][0];
      const floatx4 pb = p_s[i][1];
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        const int64_t vi = VT ? vt_idx(p, pg, b, g, d, tok) : k_row(p, pg, b, g, tok) + d;
        const float v = load1<KT>(p.v, vi);
        acc[0][k] += pa[0] * v;
        acc[1][k] += pa[1] * v;
        acc[2][k] += pa[2] * v;
        acc[3][k] += pa[3] * v;
        acc[4][k] += pb[0] * v;
        acc[5][k] += pb[1] * v;
        acc[6][k] += pb[2] * v;
        acc[7][k] += pb[3] * v;
      }
    }
    __syncthreads();
  }

  if (p.finalize || it.S == 1) {                 // one split: the output itself (combine skips it)
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) {
      const int r = r0 + rr;
      if (r >= p.rho) break;
      int j, h;
      row_jh(p, g, r, &j, &h);
      const float s2 = p.has_sink ? p.sinks[h] * kLog2e : 0.0f;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        store_o1(p, qo_idx(p, b, j, h, d), finalize_one(m[rr], l[rr], acc[rr][k], p.has_sink, s2));
      }
    }
  } else {
    const int64_t slot = (int64_t)it.slot_item * p.Hkv + g;
#pragma unroll
    for (int rr = 0; rr < RC; ++rr) {
      const int r = r0 + rr;
      if (r >= p.rho) break;
      const int64_t rec = slot * p.rho + r;
      if (lane == 0) {
        p.pm[rec] = m[rr];
        p.pl[rec] = l[rr];
      }
#pragma unroll
      for (int k = 0; k < DPL; ++k) store_rec1(p, rec * D + lane + 64 * k, acc[rr][k]);
    }
    if (p.counters) fused_merge_tail(p, it, g, 64);
  }
}

namespace {

template <class QT, class KT, int D>
int launch_vt(const Params& p, void* stream, int64_t grid) {
  if (p.v_layout == SKV_V_TRANSPOSED)
    hipLaunchKernelGGL((partial_valu<QT, KT, D, true>), dim3((unsigned)grid), dim3(64), 0,
                       (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL((partial_valu<QT, KT, D, false>), dim3((unsigned)grid), dim3(64), 0,
                       (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

template <class QT, class KT>
int launch_d(const Params& p, void* stream, int64_t grid) {
  switch (p.D) {
    case 64: return launch_vt<QT, KT, 64>(p, stream, grid);
    case 128: return launch_vt<QT, KT, 128>(p, stream, grid);
    case 256: return launch_vt<QT, KT, 256>(p, stream, grid);
  }
  return SKV_ERR_SHAPE;
}

template <class QT>
int launch_kv(const Params& p, void* stream, int64_t grid) {
  switch (p.kv_dtype) {
    case SKV_F32: return launch_d<QT, F32>(p, stream, grid);
    case SKV_BF16: return launch_d<QT, BF16>(p, stream, grid);
    case SKV_INT8: return launch_d<QT, I8>(p, stream, grid);
    case SKV_FP8_E4M3: return launch_d<QT, FP8>(p, stream, grid);
  }
  return SKV_ERR_DTYPE;
}

}  // namespace

int launch_partial_valu(Params p, void* stream) {
  const int nrc = (p.rho + RC - 1) / RC;
  p.row_groups = nrc;
  const int64_t grid = (int64_t)p.n_items * p.Hkv * nrc;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  if (p.q_dtype == SKV_F32) return launch_kv<F32>(p, stream, grid);
  if (p.q_dtype == SKV_F16) return launch_kv<F16>(p, stream, grid);
  return launch_kv<BF16>(p, stream, grid);
}

}  // namespace skv
