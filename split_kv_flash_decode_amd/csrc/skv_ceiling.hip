// Read-only gather with the memory pattern of the matrix-core partial kernel:
// a measurement of the bandwidth a paged split-KV read can reach on this GPU,
// not part of the attention path.
//
// The bytes that count are those of the bandwidth note of aiter #5628 "tune
// MTP work budgets and planned reduction" (Performance): the valid K and V
// codes and their per-token scales. This kernel reads exactly those, with the
// partial kernel's work decomposition (one workgroup per (work item, KV
// head), four key streams taking interleaved 32-key blocks of the item's
// split range), its page-table reads (scalar loads of the page ids of a
// block's two 16-key groups), its 16-byte-per-lane direct-to-LDS loads of
// whole K rows, V rows (or V^T runs) and one dword of scales per lane and its
// ring depth, and does no arithmetic on the data. It waits and synchronizes
// once per block with all but one stage in flight: of the partial kernel's
// two schedules (that one, and one barrier per two blocks after a full wait)
// the faster for a loop that computes nothing. Its time per launch is the
// floor the partial kernel's loads put under it; the partial kernel's own
// time over this one is the share of the memory ceiling it reaches.

#include "skv_device.h"

namespace skv {

namespace {

template <int EB, int D, bool VT, bool QUANT>
__global__ __launch_bounds__(256) void gather_ceiling_kernel(Params p, uint32_t* sink) {
  constexpr int RB = D * EB;                     // bytes of one key row
  constexpr int KIG = RB / 64;                   // 1 KiB loads per 16-key group, K and plain V
  constexpr int U = (D / 32) * EB;               // transposed V: 512-byte units per group
  constexpr int NVL = VT ? U / 2 : KIG;          // V loads per 16-key group
  constexpr int KSZ = 32 * RB;
  constexpr int VSZ = 32 * RB;
  constexpr int STAGE = KSZ + VSZ + (QUANT ? 256 : 0);
  constexpr int NS0 = (156 * 1024) / (4 * STAGE);
  constexpr int NS = NS0 > 4 ? 4 : (NS0 < 2 ? 2 : NS0);
  constexpr int LPB = 2 * KIG + 2 * NVL + (QUANT ? 1 : 0);   // loads per block and wave
  __shared__ __attribute__((aligned(16))) char smem[4 * NS * STAGE];

  const int lane = threadIdx.x & 63;
  const int sid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // key stream = wave
  const int g = blockIdx.x % p.Hkv;
  const int item = blockIdx.x / p.Hkv;
  Item it;
  if (!decode_item(p, item, &it)) return;
  const int b = it.b;
  const int ctx = clamp_ctx(p, b);
  int lo, hi;
  split_range(ctx, p.R, p.causal, p.window, it.S, it.s, &lo, &hi);
  char* ring = smem + sid * NS * STAGE;
  const int* trow = p.table + (int64_t)b * p.max_pages;
  const char* kbase = reinterpret_cast<const char*>(p.k);
  const char* vbase = reinterpret_cast<const char*>(p.v);
  const int i32 = lane & 31, hh = lane >> 5;
  const int dstride = (1 << p.bs_shift) * EB;

  // Row of the first key of 16-key group gp of the block at t0 (a group that
  // starts at or past hi reuses group 0, so no page past the context is read).
  auto grp_row = [&](int t0, int gp, int p0, int p1) __attribute__((always_inline)) {
    const int tg = (t0 + 16 * gp < hi) ? t0 + 16 * gp : t0;
    const int pg = (gp && p.bs_shift == 4 && t0 + 16 < hi) ? p1 : p0;
    return (((int64_t)pg * p.Hkv + g) << p.bs_shift) + (tg & ((1 << p.bs_shift) - 1));
  };
  auto issue = [&](int t0, int st) __attribute__((always_inline)) {
    const int p0 = cload(trow + (t0 >> p.bs_shift));
    const int p1 = (p.bs_shift == 4 && t0 + 16 < hi) ? cload(trow + (t0 >> 4) + 1) : p0;
    const uint32_t S = lds_addr(ring + st * STAGE);
    const int64_t R0 = grp_row(t0, 0, p0, p1), R1 = grp_row(t0, 1, p0, p1);
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      const char* kb = kbase + (gp ? R1 : R0) * RB;
#pragma unroll
      for (int n = 0; n < KIG; ++n) dma16s(kb, (uint32_t)(n * 1024 + lane * 16), S + (gp * KIG + n) * 1024);
    }
#pragma unroll
    for (int gp = 0; gp < 2; ++gp) {
      if constexpr (VT) {
        const int64_t R = gp ? R1 : R0;
        const int64_t pg_slot = R & ((1 << p.bs_shift) - 1);
        const int64_t base = ((R - pg_slot) * D << 0);   // (page, head) block start in elements of V^T
        const char* vb = vbase + (base + pg_slot) * EB;
#pragma unroll
        for (int n = 0; n < NVL; ++n) {
          const int u = 2 * n + (lane >> 5);
          const uint32_t off = (uint32_t)((32 * (u / EB) + i32) * dstride + (u % EB) * 16);
          dma16s(vb, off, S + KSZ + (gp * NVL + n) * 1024);
        }
      } else {
        const char* vb = vbase + (gp ? R1 : R0) * RB;
#pragma unroll
        for (int n = 0; n < NVL; ++n) dma16s(vb, (uint32_t)(n * 1024 + lane * 16), S + KSZ + (gp * NVL + n) * 1024);
      }
    }
    if constexpr (QUANT) {
      const int64_t r = ((i32 >= 16) ? R1 : R0) + (i32 & 15);
      dma4((hh ? p.vs : p.ks) + r, S + KSZ + VSZ);
    }
  };

  const int nblk = hi > lo ? (hi - lo + 31) / 32 : 0;
  const int mine = nblk > sid ? (nblk - 1 - sid) / 4 + 1 : 0;
  const int steps = (nblk + 3) / 4;
  auto t0_of = [&](int j) __attribute__((always_inline)) { return lo + (sid + 4 * j) * 32; };
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < mine) issue(t0_of(j), j);
  uint32_t acc = 0;
  for (int j = 0; j < steps; ++j) {
    const int r = mine - 1 - j;                  // own blocks issued after block j
    if (r >= NS - 2) wait_vm<(NS - 2) * LPB>();
    else if (r == 1) wait_vm<LPB>();
    else wait_vm<0>();
    __syncthreads();
    if (j < mine) acc ^= *reinterpret_cast<const uint32_t*>(ring + (j % NS) * STAGE + lane * 4);
    const int jn = j + NS - 1;
    if (jn < mine) issue(t0_of(jn), jn % NS);
  }
  wait_vm<0>();
  acc ^= __shfl_xor(acc, 32, 64);
  if (threadIdx.x == 0) sink[blockIdx.x] = acc;
}

template <int EB, int D, bool VT>
int launch_q(const Params& p, uint32_t* sink, void* stream, int64_t grid) {
  if (p.kv_dtype == SKV_INT8 || p.kv_dtype == SKV_FP8_E4M3)
    hipLaunchKernelGGL((gather_ceiling_kernel<EB, D, VT, true>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p, sink);
  else
    hipLaunchKernelGGL((gather_ceiling_kernel<EB, D, VT, false>), dim3((unsigned)grid), dim3(256), 0,
                       (hipStream_t)stream, p, sink);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

template <int EB, int D>
int launch_v(const Params& p, uint32_t* sink, void* stream, int64_t grid) {
  return p.v_layout == SKV_V_TRANSPOSED ? launch_q<EB, D, true>(p, sink, stream, grid)
                                        : launch_q<EB, D, false>(p, sink, stream, grid);
}

}  // namespace

int launch_gather_ceiling(Params p, uint32_t* sink, void* stream) {
  const int64_t grid = (int64_t)p.n_items * p.Hkv;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  const bool one = p.kv_dtype == SKV_INT8 || p.kv_dtype == SKV_FP8_E4M3;
  if (one) {
    switch (p.D) {
      case 64: return launch_v<1, 64>(p, sink, stream, grid);
      case 128: return launch_v<1, 128>(p, sink, stream, grid);
      case 256: return launch_v<1, 256>(p, sink, stream, grid);
    }
  } else if (p.kv_dtype == SKV_BF16) {
    switch (p.D) {
      case 64: return launch_v<2, 64>(p, sink, stream, grid);
      case 128: return launch_v<2, 128>(p, sink, stream, grid);
    }
  }
  return SKV_ERR_UNSUPPORTED;
}

}  // namespace skv
