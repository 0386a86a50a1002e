// Device-side plan refresh: the split planner of skv_plan_fill run on the GPU
// from the device context lengths, so that a captured decode step re-plans
// on every replay without a host round trip (aiter #5628 "tune MTP work
// budgets and planned reduction", intro and Changes: per-request partition
// counts from the work, a fixed capacity that graph replay keeps).
//
// One workgroup of 1024 threads, batch <= SKV_PLAN_DEVICE_MAX_BATCH; all
// per-request state lives in LDS. The arithmetic is the host planner's, in
// the same integer widths, so the metadata block is bit-identical to
// skv_plan_fill's for the same context lengths:
//  1. counts: an explicit count, or the work floor ceil(span * R / work),
//     clamped to [1, min(max_partitions, tiles of the span)];
//  2. without an explicit count, a batch that does not fill the base budget
//     num_cus * ctas_per_cu / (Hkv * workgroups_per_head) raises each request
//     to its span share of it (at most span / min_tokens, at most the clamp);
//  3. counts above the capacity are scaled down (at least 1 each), then the
//     first largest is trimmed until the sum fits;
//  4. header, counts, exclusive prefix sums (record slots) and the work list:
//     items ordered by decreasing key count, ties in (request, split) order.
//     A request's splits are full chunks, at most one shorter split and then
//     empty ones, so its items form at most three runs of equal length, read
//     off the split geometry. The runs are sorted in LDS (bitonic, key:
//     length descending, then request, then run) and a prefix sum of their
//     item counts in that order gives each run's first rank.

#include "skv_device.h"

namespace skv {

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxB = SKV_PLAN_DEVICE_MAX_BATCH;

__device__ __forceinline__ int64_t span_keys(const PlanDev& h, int ctx) {
  int lo, hi;
  split_range(ctx, h.R, h.causal, h.window, 1, 0, &lo, &hi);
  return (int64_t)hi - lo;
}

// Sum over the workgroup (every thread gets the total).
__device__ int64_t block_sum(int64_t x, int64_t* red) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  __syncthreads();
  if ((tid & 63) == 0) red[tid >> 6] = x;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) t += red[w];
  return t;
}

// Runs of equal-length items of a request with p splits (k = 0: the first
// split and all as long; k = 1: one shorter non-empty split; k = 2: empty
// splits): item count, key count and first split.
// Inclusive prefix sum of buf[src][0, n) (double-buffered, every thread
// takes part); returns the buffer holding the result.
__device__ int inclusive_scan(int32_t (*buf)[4 * kMaxB], int src, int n) {
  int cur = src;
  for (int d = 1; d < n; d <<= 1) {
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) buf[cur ^ 1][i] = buf[cur][i] + (i >= d ? buf[cur][i - d] : 0);
    cur ^= 1;
  }
  __syncthreads();
  return cur;
}

__device__ __forceinline__ void run_info(const PlanDev& h, int ctx, int p, int k, int* cnt, int* len, int* s0) {
  *cnt = 0;
  *len = 0;
  *s0 = 0;
  if (ctx <= 0) {
    if (k == 0) *cnt = p;                         // every split empty
    return;
  }
  int u, chunk;
  split_geometry(ctx, h.R, h.causal, h.window, p, &u, &chunk);
  const int span = ctx - u;
  const int full = span / chunk < p ? span / chunk : p;   // splits of a whole chunk
  const int rem = full < p ? span - full * chunk : 0;      // the shorter split, if any
  const int c0 = full >= 1 ? full : 1;            // (no whole chunk: split 0 is the shorter one)
  const int c1 = full >= 1 && rem > 0 ? 1 : 0;
  if (k == 0) {
    *cnt = c0;
    *len = full >= 1 ? chunk : span;
  } else if (k == 1) {
    *cnt = c1;
    *len = rem;
    *s0 = c0;
  } else {
    *cnt = p - c0 - c1;
    *s0 = c0 + c1;
  }
}

__global__ __launch_bounds__(kThreads) void plan_kernel(PlanDev h, const int32_t* ctx, int32_t* meta) {
  constexpr int kRuns = 4 * kMaxB;                // power of two >= 3 runs per request
  __shared__ int32_t P_s[kMaxB];
  __shared__ int32_t ctx_s[kMaxB];
  __shared__ uint64_t key_s[kRuns];
  __shared__ int32_t scan_s[2][kRuns];
  __shared__ int64_t red_s[kThreads / 64];
  __shared__ int64_t sum_s;
  const int tid = threadIdx.x;
  const int B = h.B;

  // 1. counts from the work (or the explicit count)
  int64_t tot = 0, sum = 0;
  for (int b = tid; b < B; b += kThreads) {
    const int c = ctx[b];
    ctx_s[b] = c;
    const int64_t span = span_keys(h, c);
    const int64_t tiles = (span + kSplitAlign - 1) / kSplitAlign;
    const int64_t cap = max((int64_t)1, min((int64_t)h.maxp, tiles));
    const int64_t pb = h.explicit_p > 0 ? (int64_t)h.explicit_p : (span * h.R + h.work - 1) / h.work;
    const int p = (int)max((int64_t)1, min(pb, cap));
    P_s[b] = p;
    tot += span;
    sum += p;
  }
  tot = block_sum(tot, red_s);
  sum = block_sum(sum, red_s);

  // 2. raise to the base budget
  if (h.explicit_p <= 0 && tot > 0) {
    const int64_t budget = (int64_t)h.cus * h.ctas / ((int64_t)h.Hkv * h.wph);
    if (sum < budget) {
      int64_t s2 = 0;
      for (int b = tid; b < B; b += kThreads) {
        const int64_t span = span_keys(h, ctx_s[b]);
        const int64_t tiles = (span + kSplitAlign - 1) / kSplitAlign;
        const int64_t cap = max((int64_t)1, min((int64_t)h.maxp, tiles));
        int64_t share = budget * span / tot;
        const int64_t by_tokens = max((int64_t)1, span / h.min_tokens);
        share = min(share, by_tokens);
        const int p = (int)max((int64_t)P_s[b], min(share, cap));
        P_s[b] = p;
        s2 += p;
      }
      sum = block_sum(s2, red_s);
    }
  }

  // 3. keep the capacity
  if (sum > h.C) {
    int64_t s3 = 0;
    for (int b = tid; b < B; b += kThreads) {
      const int p = (int)max((int64_t)1, (int64_t)P_s[b] * h.C / sum);
      P_s[b] = p;
      s3 += p;
    }
    s3 = block_sum(s3, red_s);
    if (tid == 0) {
      // (terminates: the capacity is at least B, so a count above 1 remains)
      while (s3 > h.C) {
        int bm = 0;
        for (int b = 1; b < B; ++b)
          if (P_s[b] > P_s[bm]) bm = b;
        --P_s[bm];
        --s3;
      }
      sum_s = s3;
    }
    __syncthreads();
    sum = sum_s;
  }
  __syncthreads();

  // 4. header, counts, slot offsets (exclusive prefix sums), largest count
  int pmax = 0;
  {
    int x = 0;
    for (int b = tid; b < B; b += kThreads) x = max(x, P_s[b]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x = max(x, __shfl_xor(x, o, 64));
    __syncthreads();
    if ((tid & 63) == 0) red_s[tid >> 6] = x;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) pmax = max(pmax, (int)red_s[w]);
  }
  for (int b = tid; b < B; b += kThreads) scan_s[0][b] = P_s[b];
  int cur = inclusive_scan(scan_s, 0, B);
  if (tid == 0) {
    meta[0] = B;
    meta[1] = h.C;
    meta[2] = (int32_t)sum;
    meta[3] = pmax;
  }
  for (int b = tid; b < B; b += kThreads) {
    meta[4 + b] = P_s[b];
    meta[4 + B + b] = scan_s[cur][b] - P_s[b];
  }

  // 5. sort the runs: key = (length descending, request, run); empty runs last
  int n = 1;
  while (n < 3 * B) n <<= 1;
  for (int i = tid; i < n; i += kThreads) {
    uint64_t key = ~0ull;
    if (i < 3 * B) {
      const int b = i / 3, k = i - 3 * (i / 3);
      int cnt, len, s0;
      run_info(h, ctx_s[b], P_s[b], k, &cnt, &len, &s0);
      if (cnt > 0) key = ((uint64_t)(0x7FFFFFFFu - (uint32_t)len) << 32) | (uint32_t)i;
    }
    key_s[i] = key;
  }
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < n / 2; i += kThreads) {
        const int lo = 2 * i - (i & (stride - 1));   // element pair (lo, lo + stride)
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const uint64_t a = key_s[lo], c = key_s[hi];
        if ((a > c) == up) {
          key_s[lo] = c;
          key_s[hi] = a;
        }
      }
    }
  }
  __syncthreads();

  // 6. first rank of every run (prefix sum of counts in sorted order), work list
  for (int i = tid; i < n; i += kThreads) {
    int cnt = 0;
    const uint64_t key = key_s[i];
    if (key != ~0ull) {
      const int g = (int)(uint32_t)key, b = g / 3;
      int len, s0;
      run_info(h, ctx_s[b], P_s[b], g - 3 * b, &cnt, &len, &s0);
    }
    scan_s[0][i] = cnt;
  }
  cur = inclusive_scan(scan_s, 0, n);
  int32_t* work = meta + 4 + 2 * B;
  for (int i = tid; i < n; i += kThreads) {
    const uint64_t key = key_s[i];
    if (key == ~0ull) continue;
    const int g = (int)(uint32_t)key, b = g / 3;
    int cnt, len, s0;
    run_info(h, ctx_s[b], P_s[b], g - 3 * b, &cnt, &len, &s0);
    const int first = scan_s[cur][i] - cnt;
    for (int j = 0; j < cnt; ++j) work[first + j] = b * 256 + s0 + j;
  }
  for (int64_t i = sum + tid; i < h.C; i += kThreads) work[i] = -1;
}

}  // namespace

int launch_plan_device(const PlanDev& h, const int32_t* ctx, int32_t* meta, void* stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kThreads), 0, (hipStream_t)stream, h, ctx, meta);
  return hipGetLastError() == hipSuccess ? SKV_OK : SKV_ERR_LAUNCH;
}

}  // namespace skv
