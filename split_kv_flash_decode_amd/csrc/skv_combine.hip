// Combine kernel: merge the partial records of every split of a request into
// the output ("combine kernel ... merged by the flash-decoding formula",
// tiny-llm #11 split-KV design record, "Design"; the reducer iterates only
// each request's actual partitions, aiter #5628 "tune MTP work budgets and
// planned reduction", Changes).
//
// One 256-thread workgroup per (request, KV head, chunk of rows); each thread
// owns four consecutive d of one query row, so record reads and output writes
// are 16-byte coalesced. Splits are visited in increasing s, which makes the
// result deterministic, and with one split bit-identical to the single-pass
// kernels (same operations as finalize_one).

#include "skv_device.h"

namespace skv {

__global__ __launch_bounds__(256) void combine_kernel(Params p) {
  const int tpr = p.D >> 2;            // threads per row
  const int rpw = 256 / tpr;           // rows per workgroup
  const int nch = (p.rho + rpw - 1) / rpw;
  int blk = blockIdx.x;
  const int ch = blk % nch;
  blk /= nch;
  const int g = blk % p.Hkv;
  const int b = blk / p.Hkv;
  const int r = ch * rpw + (int)threadIdx.x / tpr;
  if (r >= p.rho) return;
  const int d = ((int)threadIdx.x % tpr) * 4;
  int S, slot0;
  if (p.plan) {
    S = p.plan[4 + b];
    slot0 = p.plan[4 + p.B + b];
  } else {
    S = p.num_splits;
    slot0 = b * S;
  }
  int j, h;
  row_jh(p, g, r, &j, &h);
  store_o4(p, qo_idx(p, b, j, h, d), merge_splits4(p, g, r, d, h, S, slot0));
}

int launch_combine(Params p, void* stream) {
  const int tpr = p.D >> 2;
  const int rpw = 256 / tpr;
  const int nch = (p.rho + rpw - 1) / rpw;
  const int64_t grid = (int64_t)p.B * p.Hkv * nch;
  if (grid > 0x7FFFFFFF) return SKV_ERR_SHAPE;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, p);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

}  // namespace skv
