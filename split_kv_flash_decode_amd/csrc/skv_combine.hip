// Combine kernel: merge the partial records of every split of a request into
// the output with the flash-decoding merge (tiny-llm #11 split-KV design
// record, "Design": a second kernel does the merge); the reducer visits only
// the partitions a request actually has (aiter #5628 "tune MTP work budgets
// and planned reduction", Changes).
//
// The grid is the work list itself: K 256-thread workgroups per (work item,
// KV head). A request with S splits thus gets S * K workgroups, which share
// its rho * D / 4 output units (merge_part): a long request is merged by as
// many workgroups as it has splits, each thread loads about eight records,
// and lanes that share a unit combine their states by a fixed butterfly.
// The arithmetic depends only on (S, K, rho, D), so the result is
// deterministic. Requests with one split were finalized by the partial
// kernels themselves (same bits as the single-pass kernels) and are skipped;
// so are unused plan items. bf16 records are widened to fp32 as they are
// read; the arithmetic is the same.

#include "skv_device.h"

namespace skv {

template <bool RBF>
__global__ __launch_bounds__(kMergeThreads) void combine_kernel(Params p) {
  const int K = merge_wgs_per_item(p.rho, p.D);
  int blk = blockIdx.x;
  const int k = blk % K;
  blk /= K;
  const int g = blk % p.Hkv;
  const int item = blk / p.Hkv;
  Item it;
  if (!decode_item(p, item, &it)) return;        // unused plan item
  if (it.S == 1) return;                          // the partial kernel wrote it
  const int slot0 = it.slot_item - it.s;          // slot item of the request's split 0
  merge_part<RBF>(p, it.b, g, it.S, slot0, it.s * K + k, K, (int)threadIdx.x);
}

int launch_combine(Params p, void* stream) {
  const int K = merge_wgs_per_item(p.rho, p.D);
  const int64_t grid = (int64_t)p.n_items * p.Hkv * K;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  if (grid == 0) return SKV_OK;
  if (p.rec_bf16)
    hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)grid), dim3(kMergeThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)grid), dim3(kMergeThreads), 0, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

}  // namespace skv
