// Combine kernel: merge the partial records of every split of a request into
// the output with the flash-decoding merge (tiny-llm #11 split-KV design
// record, "Design": a second kernel does the merge); the reducer visits only
// the partitions a request actually has (aiter #5628 "tune MTP work budgets
// and planned reduction", Changes).
//
// One 256-thread workgroup per (request, KV head, chunk of rows); four
// adjacent threads share one output (four consecutive d of one query row)
// and merge a quarter of the splits each, so record reads and output writes
// are 16-byte coalesced and a request with many splits is read by many
// lanes at once. The quarters are visited in a fixed order, which makes the
// result deterministic, and with one split bit-identical to the single-pass
// kernels (same operations as finalize_one); requests with one split are
// therefore finalized by the partial kernels themselves and skipped here.
// bf16 records are widened to fp32 as they are read; the arithmetic is the
// same.

#include "skv_device.h"

namespace skv {

constexpr int kCombineThreads = 256;

template <bool RBF>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(Params p) {
  const int tpr = p.D >> 2;            // outputs per row
  const int rpw = kCombineThreads / (4 * tpr);   // rows per workgroup
  const int nch = (p.rho + rpw - 1) / rpw;
  int blk = blockIdx.x;
  const int ch = blk % nch;
  blk /= nch;
  const int g = blk % p.Hkv;
  const int b = blk / p.Hkv;
  const int o = (int)threadIdx.x >> 2, q = (int)threadIdx.x & 3;
  const int r = ch * rpw + o / tpr;
  if (r >= p.rho) return;                        // (whole quads of lanes)
  const int d = (o % tpr) * 4;
  int S, slot0;
  if (p.plan) {
    S = p.plan[4 + b];
    slot0 = p.plan[4 + p.B + b];
  } else {
    S = p.num_splits;
    slot0 = b * S;
  }
  if (S == 1) return;                             // the partial kernel wrote it
  int j, h;
  row_jh(p, g, r, &j, &h);
  const floatx4 v = merge_splits4<RBF>(p, g, r, d, h, S, slot0, q);
  if (q == 0) store_o4(p, qo_idx(p, b, j, h, d), v);
}

int launch_combine(Params p, void* stream) {
  const int tpr = p.D >> 2;
  const int rpw = kCombineThreads / (4 * tpr);
  const int nch = (p.rho + rpw - 1) / rpw;
  const int64_t grid = (int64_t)p.B * p.Hkv * nch;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  if (p.rec_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(kCombineThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(kCombineThreads), 0, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

}  // namespace skv
