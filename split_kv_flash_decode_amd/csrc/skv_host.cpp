// Host side of the C ABI: status strings, argument validation, partial-record
// sizing, the split planner, and the dispatch of the compute entry points.
//
// This file makes no HIP runtime call itself: validation, sizing and planning
// run on any host, with or without a GPU. The compute entry points validate
// first and only then hand a parameter block to the kernel launchers.

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "skv.h"
#include "skv_internal.h"

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

int64_t rho_of(const skv_desc* d) {
  return (int64_t)d->q_rows * (d->num_q_heads / d->num_kv_heads);
}

// Shape, dtype and layout checks of a descriptor (no pointers). paged < 0
// skips the KV-layout fields (the combine stage never reads KV).
int check_desc(const skv_desc* d, int paged) {
  if (!d) return SKV_ERR_NULL;
  if (d->batch < 1 || d->q_rows < 1 || d->num_kv_heads < 1 || d->num_q_heads < 1)
    return SKV_ERR_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return SKV_ERR_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256) return SKV_ERR_SHAPE;
  if (rho_of(d) > 4096) return SKV_ERR_SHAPE;
  if (d->window < 0) return SKV_ERR_SHAPE;
  if (d->causal != 0 && d->causal != 1) return SKV_ERR_SHAPE;
  if (!(d->scale == d->scale) || isinf(d->scale)) return SKV_ERR_SHAPE;
  if (d->q_dtype != SKV_F32 && d->q_dtype != SKV_BF16 && d->q_dtype != SKV_F16) return SKV_ERR_DTYPE;
  if (d->kv_dtype < SKV_F32 || d->kv_dtype > SKV_FP8_E4M3) return SKV_ERR_DTYPE;
  if (d->v_layout != SKV_V_PLAIN && d->v_layout != SKV_V_TRANSPOSED) return SKV_ERR_SHAPE;
  if (d->has_sink != 0 && d->has_sink != 1) return SKV_ERR_SHAPE;
  if (d->impl < SKV_IMPL_AUTO || d->impl > SKV_IMPL_MFMA) return SKV_ERR_UNSUPPORTED;
  if (d->record_dtype != SKV_F32 && d->record_dtype != SKV_BF16) return SKV_ERR_DTYPE;
  if (paged > 0) {
    if (!is_pow2(d->block_size) || d->block_size > 1024) return SKV_ERR_SHAPE;
    if (d->max_pages < 1) return SKV_ERR_SHAPE;
    if ((int64_t)d->max_pages * d->block_size > INT32_MAX) return SKV_ERR_SHAPE;
  } else if (paged == 0) {
    if (d->kv_capacity < 1) return SKV_ERR_SHAPE;
  }
  return SKV_OK;
}

int check_args(const skv_desc* d, const skv_args* a, int paged) {
  if (!a) return SKV_ERR_NULL;
  if (!a->q || !a->k || !a->v || !a->ctx_lens || !a->o) return SKV_ERR_NULL;
  if (paged && !a->page_table) return SKV_ERR_NULL;
  bool quant = d->kv_dtype == SKV_INT8 || d->kv_dtype == SKV_FP8_E4M3;
  if (quant && (!a->k_scale || !a->v_scale)) return SKV_ERR_NULL;
  if (d->has_sink && !a->sinks) return SKV_ERR_NULL;
  if (a->tree_mask && (d->causal != 1 || d->q_rows > SKV_MAX_VERIFY_ROWS)) return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

int check_partials(const skv_desc* d, const skv_partials* p, int64_t slots) {
  if (!p) return SKV_ERR_NULL;
  if (!p->m || !p->l || !p->acc) return SKV_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(p->acc) % 16 != 0) return SKV_ERR_ALIGN;
  if (p->capacity_slots < slots) return SKV_ERR_CAPACITY;
  return SKV_OK;
}

skv::Params make_params(const skv_desc* d, const skv_args* a, int paged, int num_splits,
                        const int32_t* plan, const skv_partials* p, int finalize) {
  skv::Params q;
  memset(&q, 0, sizeof(q));
  q.q = a->q;
  q.k = a->k;
  q.v = a->v;
  q.ks = a->k_scale;
  q.vs = a->v_scale;
  q.table = a->page_table;
  q.ctx = a->ctx_lens;
  q.sinks = d->has_sink ? a->sinks : nullptr;
  q.o = a->o;
  q.tree_mask = a->tree_mask;
  if (p) {
    q.pm = p->m;
    q.pl = p->l;
    q.pacc = p->acc;
  }
  q.plan = plan;
  q.B = d->batch;
  q.R = d->q_rows;
  q.Hq = d->num_q_heads;
  q.Hkv = d->num_kv_heads;
  q.D = d->head_dim;
  q.G = d->num_q_heads / d->num_kv_heads;
  q.rho = (int32_t)rho_of(d);
  q.causal = d->causal;
  q.window = d->window;
  q.scale_log2 = d->scale * skv::kLog2e;
  q.paged = paged > 0;
  if (paged > 0) {
    q.bs_shift = ilog2(d->block_size);
    q.max_pages = d->max_pages;
    q.cap = d->max_pages * d->block_size;
  } else {
    q.kv_cap = d->kv_capacity;
    q.cap = d->kv_capacity;
  }
  q.num_splits = num_splits;
  q.has_sink = d->has_sink;
  q.finalize = finalize;
  q.n_items = plan ? num_splits : d->batch * num_splits;
  q.q_dtype = d->q_dtype;
  q.kv_dtype = d->kv_dtype;
  q.v_layout = d->v_layout;
  q.block_size = paged > 0 ? d->block_size : 0;
  q.impl = d->impl;
  q.rec_bf16 = d->record_dtype == SKV_BF16;
  return q;
}

bool use_mfma(const skv::Params& p) {
  if (p.impl == SKV_IMPL_VALU) return false;
  return skv::mfma_supported(p);
}

int impl_check(const skv::Params& p) {
  if (p.impl == SKV_IMPL_MFMA && !skv::mfma_supported(p)) return SKV_ERR_UNSUPPORTED;
  return SKV_OK;
}

int run_partial(skv::Params p, void* stream) {
  int rc = impl_check(p);
  if (rc) return rc;
  return use_mfma(p) ? skv::launch_partial_mfma(p, stream) : skv::launch_partial_valu(p, stream);
}

// ---- planner ---------------------------------------------------------------

struct Hints {
  int B, R, Hkv, causal, window, cus, ctas, wph, explicit_p, maxp, work, min_tokens;
};

Hints resolve(const skv_plan_hints* h) {
  Hints r;
  r.B = h->batch;
  r.R = h->q_rows;
  r.Hkv = h->num_kv_heads;
  r.causal = h->causal;
  r.window = h->window;
  r.cus = h->num_cus > 0 ? h->num_cus : 256;
  r.ctas = h->ctas_per_cu > 0 ? h->ctas_per_cu : 2;
  r.wph = h->workgroups_per_head > 0 ? h->workgroups_per_head : 1;
  r.explicit_p = h->partitions_per_request;
  r.maxp = h->max_partitions > 0 ? std::min(h->max_partitions, SKV_MAX_SPLITS) : SKV_PLAN_DEFAULT_MAX_PARTITIONS;
  r.work = h->work_per_partition > 0 ? h->work_per_partition : 50000;
  r.min_tokens = h->min_tokens_per_partition > 0 ? h->min_tokens_per_partition : 256;
  return r;
}

int check_hints(const skv_plan_hints* h) {
  if (!h) return SKV_ERR_NULL;
  if (h->batch < 1 || h->q_rows < 1 || h->num_kv_heads < 1 || h->window < 0) return SKV_ERR_PLAN;
  if (h->partitions_per_request < 0 || h->max_partitions < 0 || h->num_cus < 0 ||
      h->ctas_per_cu < 0 || h->work_per_partition < 0 || h->min_tokens_per_partition < 0 ||
      h->workgroups_per_head < 0)
    return SKV_ERR_PLAN;
  if (h->batch > (1 << 23)) return SKV_ERR_PLAN;
  return SKV_OK;
}

// Keys of the visible union a request's splits cover (window-capped).
int64_t span_of(const Hints& h, int ctx) {
  int lo, hi;
  skv::split_range(ctx, h.R, h.causal, h.window, 1, 0, &lo, &hi);
  return hi - lo;
}

// Partition counts from host-known work ([PA] intro and Changes):
//  * explicit partitions_per_request take precedence (clamped to the tiles);
//  * otherwise a work floor ceil(span * R / work_per_partition), raised to the
//    request's share of the base budget num_cus * ctas_per_cu /
//    (Hkv * workgroups_per_head) items when the batch would not fill it, but
//    never below min_tokens keys per partition from that raise;
//  * every count lies in [1, min(max_partitions, tiles of the span)].
std::vector<int> partition_counts(const Hints& h, const std::vector<int>& ctx) {
  const int B = (int)ctx.size();
  std::vector<int64_t> span(B);
  int64_t total = 0;
  for (int b = 0; b < B; ++b) {
    span[b] = span_of(h, ctx[b]);
    total += span[b];
  }
  std::vector<int> P(B, 1);
  for (int b = 0; b < B; ++b) {
    int64_t tiles = (span[b] + skv::kSplitAlign - 1) / skv::kSplitAlign;
    int64_t cap = std::max<int64_t>(1, std::min<int64_t>(h.maxp, tiles));
    int64_t pb;
    if (h.explicit_p > 0) {
      pb = h.explicit_p;
    } else {
      pb = (span[b] * h.R + h.work - 1) / h.work;
    }
    P[b] = (int)std::max<int64_t>(1, std::min<int64_t>(pb, cap));
  }
  if (h.explicit_p <= 0 && total > 0) {
    int64_t budget = (int64_t)h.cus * h.ctas / ((int64_t)h.Hkv * h.wph);
    int64_t sum = 0;
    for (int b = 0; b < B; ++b) sum += P[b];
    if (sum < budget) {
      for (int b = 0; b < B; ++b) {
        int64_t tiles = (span[b] + skv::kSplitAlign - 1) / skv::kSplitAlign;
        int64_t cap = std::max<int64_t>(1, std::min<int64_t>(h.maxp, tiles));
        int64_t share = budget * span[b] / total;
        int64_t by_tokens = std::max<int64_t>(1, span[b] / h.min_tokens);
        share = std::min(share, by_tokens);
        P[b] = (int)std::max<int64_t>(P[b], std::min<int64_t>(share, cap));
      }
    }
  }
  return P;
}

}  // namespace

extern "C" {

int skv_abi_version(void) { return SKV_ABI_VERSION; }

const char* skv_status_str(int status) {
  switch (status) {
    case SKV_OK: return "ok";
    case SKV_ERR_NULL: return "a required pointer is NULL";
    case SKV_ERR_SHAPE: return "shape, stride or layout out of range";
    case SKV_ERR_DTYPE: return "unsupported dtype";
    case SKV_ERR_SPLITS: return "num_splits out of range [1, 256]";
    case SKV_ERR_CAPACITY: return "partial buffers or plan capacity too small";
    case SKV_ERR_UNSUPPORTED: return "unsupported combination for the requested kernel family";
    case SKV_ERR_LAUNCH: return "kernel launch failed";
    case SKV_ERR_PLAN: return "inconsistent plan hints or metadata";
    case SKV_ERR_ALIGN: return "partials.acc is not 16-byte aligned";
    case SKV_ERR_SCRATCH: return "the call needs more than the library's static scratch";
    default: return "unknown status";
  }
}

int skv_validate(const skv_desc* d, int32_t paged, int32_t num_splits, const skv_partials* p) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  if (num_splits < 0 || num_splits > SKV_MAX_SPLITS) return SKV_ERR_SPLITS;
  if (num_splits > 0) {
    rc = check_partials(d, p, skv_uniform_slots(d, num_splits));
    if (rc) return rc;
  }
  skv::Params q;
  memset(&q, 0, sizeof(q));
  skv_args dummy;
  memset(&dummy, 0, sizeof(dummy));
  q = make_params(d, &dummy, paged, num_splits > 0 ? num_splits : 1, nullptr, p, num_splits == 0);
  return impl_check(q);
}

int skv_workspace_size(const skv_desc* d, int64_t slots, size_t* m_bytes, size_t* l_bytes,
                       size_t* acc_bytes) {
  if (!d) return SKV_ERR_NULL;
  if (d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0 || d->q_rows < 1 ||
      d->head_dim < 1 || slots < 0)
    return SKV_ERR_SHAPE;
  size_t rows = (size_t)slots * (size_t)rho_of(d);
  if (m_bytes) *m_bytes = rows * sizeof(float);
  if (l_bytes) *l_bytes = rows * sizeof(float);
  if (d->record_dtype != SKV_F32 && d->record_dtype != SKV_BF16) return SKV_ERR_DTYPE;
  if (acc_bytes) *acc_bytes = rows * (size_t)d->head_dim * (d->record_dtype == SKV_BF16 ? 2 : 4);
  return SKV_OK;
}

int skv_splitkv_workspace_size(const skv_desc* d, int64_t slots, size_t* m_bytes, size_t* l_bytes,
                               size_t* acc_bytes) {
  return skv_workspace_size(d, slots, m_bytes, l_bytes, acc_bytes);
}

int64_t skv_uniform_slots(const skv_desc* d, int32_t num_splits) {
  if (!d || num_splits < 1) return 0;
  return (int64_t)d->batch * num_splits * d->num_kv_heads;
}

static int single_pass(const skv_desc* d, const skv_args* a, int paged, void* stream) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  rc = check_args(d, a, paged);
  if (rc) return rc;
  skv::Params p = make_params(d, a, paged, 1, nullptr, nullptr, 1);
  return run_partial(p, stream);
}

int skv_attention_decode(const skv_desc* d, const skv_args* a, void* stream) {
  return single_pass(d, a, 0, stream);
}

int skv_attention_decode_paged(const skv_desc* d, const skv_args* a, void* stream) {
  return single_pass(d, a, 1, stream);
}

}  // extern "C"

namespace skv {
int check_split_call(const skv_desc* d, const skv_args* a, int paged, int32_t num_splits) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  rc = check_args(d, a, paged);
  if (rc) return rc;
  if (num_splits < 1 || num_splits > SKV_MAX_SPLITS) return SKV_ERR_SPLITS;
  if ((int64_t)d->batch * num_splits * d->num_kv_heads * 64 > INT32_MAX) return SKV_ERR_SHAPE;
  skv_args none;
  memset(&none, 0, sizeof(none));
  return impl_check(make_params(d, &none, paged, num_splits, nullptr, nullptr, 0));
}
}  // namespace skv

extern "C" {

static int split_call(const skv_desc* d, const skv_args* a, int paged, int32_t num_splits,
                      const skv_partials* p, void* stream) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  rc = check_args(d, a, paged);
  if (rc) return rc;
  if (num_splits < 1 || num_splits > SKV_MAX_SPLITS) return SKV_ERR_SPLITS;
  rc = check_partials(d, p, skv_uniform_slots(d, num_splits));
  if (rc) return rc;
  if ((int64_t)d->batch * num_splits * d->num_kv_heads * 64 > INT32_MAX) return SKV_ERR_SHAPE;
  skv::Params prm = make_params(d, a, paged, num_splits, nullptr, p, 0);
  rc = impl_check(prm);
  if (rc) return rc;
  rc = run_partial(prm, stream);
  if (rc) return rc;
  return skv::launch_combine(prm, stream);
}

int skv_attention_decode_splitkv(const skv_desc* d, const skv_args* a, int32_t num_splits,
                                 const skv_partials* p, void* stream) {
  return split_call(d, a, 0, num_splits, p, stream);
}

int skv_attention_decode_paged_splitkv(const skv_desc* d, const skv_args* a, int32_t num_splits,
                                       const skv_partials* p, void* stream) {
  return split_call(d, a, 1, num_splits, p, stream);
}

int64_t skv_plan_meta_len(int32_t batch, int32_t capacity_items) {
  if (batch < 1 || capacity_items < 1) return 0;
  return 4 + 2 * (int64_t)batch + capacity_items;
}

int skv_plan_capacity(const skv_plan_hints* h, const int32_t* host_ctx, int32_t* capacity_items) {
  int rc = check_hints(h);
  if (rc) return rc;
  if (!capacity_items) return SKV_ERR_NULL;
  Hints r = resolve(h);
  std::vector<int> ctx(r.B);
  if (host_ctx) {
    for (int b = 0; b < r.B; ++b) ctx[b] = host_ctx[b];
  } else if (h->total_context_length > 0) {
    int64_t per = h->total_context_length / r.B;
    if (per > INT32_MAX) return SKV_ERR_PLAN;
    for (int b = 0; b < r.B; ++b) ctx[b] = (int)per;
  } else {
    return SKV_ERR_NULL;
  }
  std::vector<int> P = partition_counts(r, ctx);
  int64_t sum = 0;
  for (int x : P) sum += x;
  if (sum * r.Hkv > INT32_MAX / 64) return SKV_ERR_PLAN;
  *capacity_items = (int32_t)sum;
  return SKV_OK;
}

int skv_plan_fill(const skv_plan_hints* h, const int32_t* host_ctx, int32_t capacity_items,
                  int32_t* meta, int64_t meta_len, skv_plan_info* info) {
  int rc = check_hints(h);
  if (rc) return rc;
  if (!host_ctx || !meta) return SKV_ERR_NULL;
  Hints r = resolve(h);
  if (capacity_items < r.B) return SKV_ERR_CAPACITY;
  if (meta_len < skv_plan_meta_len(r.B, capacity_items)) return SKV_ERR_PLAN;
  std::vector<int> ctx(host_ctx, host_ctx + r.B);
  std::vector<int> P = partition_counts(r, ctx);
  int64_t sum = 0;
  for (int x : P) sum += x;
  if (sum > capacity_items) {
    // Keep the plan's capacity (graph replay): scale counts down, then trim the largest.
    for (int b = 0; b < r.B; ++b)
      P[b] = (int)std::max<int64_t>(1, (int64_t)P[b] * capacity_items / sum);
    sum = 0;
    for (int x : P) sum += x;
    while (sum > capacity_items) {
      int bm = (int)(std::max_element(P.begin(), P.end()) - P.begin());
      if (P[bm] <= 1) return SKV_ERR_CAPACITY;
      --P[bm];
      --sum;
    }
  }
  meta[0] = r.B;
  meta[1] = capacity_items;
  meta[2] = (int32_t)sum;
  int pmax = 0, pmin = INT32_MAX;
  int32_t off = 0;
  for (int b = 0; b < r.B; ++b) {
    meta[4 + b] = P[b];
    meta[4 + r.B + b] = off;
    off += P[b];
    pmax = std::max(pmax, P[b]);
    pmin = std::min(pmin, P[b]);
  }
  meta[3] = pmax;
  // Work list, longest items first (ties in request then split order).
  struct W {
    int64_t len;
    int b, s;
  };
  std::vector<W> items;
  items.reserve((size_t)sum);
  for (int b = 0; b < r.B; ++b) {
    for (int s = 0; s < P[b]; ++s) {
      int lo, hi;
      skv::split_range(ctx[b] < 0 ? 0 : ctx[b], r.R, r.causal, r.window, P[b], s, &lo, &hi);
      items.push_back({hi - lo, b, s});
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const W& x, const W& y) { return x.len > y.len; });
  int32_t* work = meta + 4 + 2 * r.B;
  for (int64_t i = 0; i < capacity_items; ++i)
    work[i] = i < (int64_t)items.size() ? items[i].b * 256 + items[i].s : -1;
  if (info) {
    info->num_items = (int32_t)sum;
    info->capacity_items = capacity_items;
    info->max_partitions = pmax;
    info->min_partitions = pmin;
    info->slots = (int64_t)capacity_items * r.Hkv;
  }
  return SKV_OK;
}

int skv_plan_make(const skv_plan_hints* h, skv_plan* plan) {
  int rc = check_hints(h);
  if (rc) return rc;
  if (!plan) return SKV_ERR_NULL;
  int32_t cap = plan->capacity_items;
  if (cap <= 0) {
    if (h->total_context_length <= 0) return SKV_ERR_PLAN;
    rc = skv_plan_capacity(h, nullptr, &cap);
    if (rc) return rc;
  }
  if (cap < h->batch) return SKV_ERR_CAPACITY;
  plan->hints = *h;
  plan->capacity_items = cap;
  plan->meta_len = skv_plan_meta_len(h->batch, cap);
  memset(&plan->info, 0, sizeof(plan->info));
  return SKV_OK;
}

int skv_plan_refresh(skv_plan* plan, const int32_t* host_ctx) {
  if (!plan) return SKV_ERR_NULL;
  return skv_plan_fill(&plan->hints, host_ctx, plan->capacity_items, plan->meta, plan->meta_len, &plan->info);
}

int skv_attention_decode_paged_planned(const skv_desc* d, const skv_args* a,
                                       const int32_t* plan_meta, int32_t capacity_items,
                                       const skv_partials* p, void* stream) {
  int rc = check_desc(d, 1);
  if (rc) return rc;
  rc = check_args(d, a, 1);
  if (rc) return rc;
  if (!plan_meta) return SKV_ERR_NULL;
  if (capacity_items < d->batch) return SKV_ERR_CAPACITY;
  if ((int64_t)capacity_items * d->num_kv_heads * 64 > INT32_MAX) return SKV_ERR_SHAPE;
  rc = check_partials(d, p, (int64_t)capacity_items * d->num_kv_heads);
  if (rc) return rc;
  skv::Params prm = make_params(d, a, 1, capacity_items, plan_meta, p, 0);
  rc = impl_check(prm);
  if (rc) return rc;
  rc = run_partial(prm, stream);
  if (rc) return rc;
  return skv::launch_combine(prm, stream);
}

int skv_attention_decode_paged_planned_host(const skv_desc* d, const skv_args* a,
                                            const int32_t* plan_meta_host, int32_t capacity_items,
                                            const skv_partials* p, void* stream) {
  int rc = check_desc(d, 1);
  if (rc) return rc;
  rc = check_args(d, a, 1);
  if (rc) return rc;
  if (!plan_meta_host) return SKV_ERR_NULL;
  if (capacity_items < d->batch) return SKV_ERR_CAPACITY;
  const int64_t n = skv_plan_meta_len(d->batch, capacity_items);
  if (n > SKV_PLAN_INLINE_MAX) return SKV_ERR_UNSUPPORTED;
  if (plan_meta_host[0] != d->batch || plan_meta_host[1] != capacity_items) return SKV_ERR_PLAN;
  rc = check_partials(d, p, (int64_t)capacity_items * d->num_kv_heads);
  if (rc) return rc;
  skv::Params prm = make_params(d, a, 1, capacity_items, nullptr, p, 0);
  prm.n_items = capacity_items;
  prm.plan_inline = 1;
  memcpy(prm.plan_blob, plan_meta_host, (size_t)n * sizeof(int32_t));
  rc = impl_check(prm);
  if (rc) return rc;
  rc = run_partial(prm, stream);
  if (rc) return rc;
  return skv::launch_combine(prm, stream);
}

int skv_splitkv_partial(const skv_desc* d, const skv_args* a, int32_t paged, int32_t num_splits,
                        const int32_t* plan_meta, const skv_partials* p, void* stream) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  rc = check_args(d, a, paged);
  if (rc) return rc;
  int64_t slots;
  if (plan_meta) {
    if (!paged) return SKV_ERR_UNSUPPORTED;
    if (num_splits < d->batch) return SKV_ERR_CAPACITY;
    slots = (int64_t)num_splits * d->num_kv_heads;
  } else {
    if (num_splits < 1 || num_splits > SKV_MAX_SPLITS) return SKV_ERR_SPLITS;
    slots = skv_uniform_slots(d, num_splits);
  }
  if (slots * 64 > INT32_MAX) return SKV_ERR_SHAPE;
  rc = check_partials(d, p, slots);
  if (rc) return rc;
  skv::Params prm = make_params(d, a, paged, num_splits, plan_meta, p, 0);
  return run_partial(prm, stream);
}

int skv_plan_hints_for_desc(const skv_desc* d, int32_t paged, skv_plan_hints* h) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  if (!h) return SKV_ERR_NULL;
  memset(h, 0, sizeof(*h));
  h->batch = d->batch;
  h->q_rows = d->q_rows;
  h->num_kv_heads = d->num_kv_heads;
  h->causal = d->causal;
  h->window = d->window;
  skv_args none;
  memset(&none, 0, sizeof(none));
  const skv::Params prm = make_params(d, &none, paged, 1, nullptr, nullptr, 0);
  const int rho = (int)rho_of(d);
  if (use_mfma(prm)) {
    // one workgroup per CU (its LDS ring), one per row group of a KV head
    const int rows = skv::mfma_group_rows(d->head_dim, rho);
    h->ctas_per_cu = 1;
    h->workgroups_per_head = (rho + rows - 1) / rows;
  } else {
    // one-wave workgroups, many per CU; a partition of one 64-key tile
    // still pays for itself
    h->ctas_per_cu = 16;
    h->workgroups_per_head = (rho + skv::kValuRows - 1) / skv::kValuRows;
    h->min_tokens_per_partition = skv::kSplitAlign;
  }
  return SKV_OK;
}

int skv_plan_refresh_device(const skv_plan_hints* h, const int32_t* ctx_dev, int32_t capacity_items,
                            int32_t* meta_dev, int64_t meta_len, void* stream) {
  int rc = check_hints(h);
  if (rc) return rc;
  if (!ctx_dev || !meta_dev) return SKV_ERR_NULL;
  Hints r = resolve(h);
  if (r.B > SKV_PLAN_DEVICE_MAX_BATCH) return SKV_ERR_UNSUPPORTED;
  if (capacity_items < r.B) return SKV_ERR_CAPACITY;
  if (meta_len < skv_plan_meta_len(r.B, capacity_items)) return SKV_ERR_PLAN;
  skv::PlanDev d;
  d.B = r.B;
  d.R = r.R;
  d.Hkv = r.Hkv;
  d.causal = r.causal;
  d.window = r.window;
  d.cus = r.cus;
  d.ctas = r.ctas;
  d.wph = r.wph;
  d.explicit_p = r.explicit_p;
  d.maxp = r.maxp;
  d.work = r.work;
  d.min_tokens = r.min_tokens;
  d.C = capacity_items;
  return skv::launch_plan_device(d, ctx_dev, meta_dev, stream);
}

int skv_splitkv_fused(const skv_desc* d, const skv_args* a, int32_t paged, int32_t num_splits,
                      const int32_t* plan_meta, const skv_partials* p, int32_t* counters, void* stream) {
  int rc = check_desc(d, paged);
  if (rc) return rc;
  rc = check_args(d, a, paged);
  if (rc) return rc;
  if (!counters) return SKV_ERR_NULL;
  int64_t slots;
  if (plan_meta) {
    if (!paged) return SKV_ERR_UNSUPPORTED;
    if (num_splits < d->batch) return SKV_ERR_CAPACITY;
    slots = (int64_t)num_splits * d->num_kv_heads;
  } else {
    if (num_splits < 1 || num_splits > SKV_MAX_SPLITS) return SKV_ERR_SPLITS;
    slots = skv_uniform_slots(d, num_splits);
  }
  if (slots * 64 > INT32_MAX) return SKV_ERR_SHAPE;
  rc = check_partials(d, p, slots);
  if (rc) return rc;
  skv::Params prm = make_params(d, a, paged, num_splits, plan_meta, p, 0);
  prm.counters = counters;
  return run_partial(prm, stream);
}

int skv_gather_ceiling(const skv_desc* d, const skv_args* a, int32_t num_splits, const int32_t* plan_meta,
                       uint32_t* sink, int64_t sink_len, void* stream) {
  int rc = check_desc(d, 1);
  if (rc) return rc;
  rc = check_args(d, a, 1);
  if (rc) return rc;
  if (!sink) return SKV_ERR_NULL;
  if (plan_meta) {
    if (num_splits < d->batch) return SKV_ERR_CAPACITY;
  } else if (num_splits < 1 || num_splits > SKV_MAX_SPLITS) {
    return SKV_ERR_SPLITS;
  }
  const int64_t items = plan_meta ? num_splits : (int64_t)d->batch * num_splits;
  if (items * d->num_kv_heads > INT32_MAX) return SKV_ERR_SHAPE;
  if (sink_len < items * d->num_kv_heads) return SKV_ERR_CAPACITY;
  const bool eight = d->kv_dtype == SKV_INT8 || d->kv_dtype == SKV_FP8_E4M3;
  if (d->block_size < 16 || !(eight || (d->kv_dtype == SKV_BF16 && d->head_dim <= 128)))
    return SKV_ERR_UNSUPPORTED;
  skv::Params prm = make_params(d, a, 1, num_splits, plan_meta, nullptr, 0);
  return skv::launch_gather_ceiling(prm, sink, stream);
}

int skv_splitkv_combine(const skv_desc* d, const skv_args* a, int32_t num_splits,
                        const int32_t* plan_meta, const skv_partials* p, void* stream) {
  int rc = check_desc(d, -1);
  if (rc) return rc;
  if (!a || !a->o || (d->has_sink && !a->sinks)) return SKV_ERR_NULL;
  int64_t slots;
  if (plan_meta) {
    if (num_splits < d->batch) return SKV_ERR_CAPACITY;
    slots = (int64_t)num_splits * d->num_kv_heads;
  } else {
    if (num_splits < 1 || num_splits > SKV_MAX_SPLITS) return SKV_ERR_SPLITS;
    slots = skv_uniform_slots(d, num_splits);
  }
  rc = check_partials(d, p, slots);
  if (rc) return rc;
  skv::Params prm = make_params(d, a, -1, num_splits, plan_meta, p, 0);
  return skv::launch_combine(prm, stream);
}

}  // extern "C"
