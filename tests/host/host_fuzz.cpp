// Host-only exercise of the library's C entry points under AddressSanitizer
// and UndefinedBehaviorSanitizer: the planner (capacity, fill, descriptor
// hints), validation and sizes over seeded random arguments, and the compute
// entry points with arguments they must reject. The kernel launchers are
// replaced by stubs that count calls (no GPU is involved); a call that reaches
// a launcher with invalid arguments is an error.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <random>
#include <vector>

#include "skv.h"
#include "skv_internal.h"

namespace skv {
static int g_launches = 0;
int launch_partial_valu(Params, void*) { ++g_launches; return SKV_OK; }
int launch_partial_mfma(Params, void*) { ++g_launches; return SKV_OK; }
int launch_combine(Params, void*) { ++g_launches; return SKV_OK; }
int launch_plan_device(const PlanDev&, const int32_t*, int32_t*, void*) { ++g_launches; return SKV_OK; }
int launch_gather_ceiling(Params, uint32_t*, void*) { ++g_launches; return SKV_OK; }
bool mfma_supported(const Params& p) { return p.q_dtype == SKV_BF16 && p.block_size >= 16; }
}  // namespace skv

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);  \
      return 1;                                                         \
    }                                                                   \
  } while (0)

// A valid descriptor, then (half the time) one field set to a random, often
// invalid, value.
static skv_desc random_desc(std::mt19937& rng) {
  auto pick = [&](std::initializer_list<int> v) { return *(v.begin() + rng() % v.size()); };
  skv_desc d;
  memset(&d, 0, sizeof(d));
  d.batch = pick({1, 3, 200});
  d.q_rows = pick({1, 4, 16, 64});
  d.num_kv_heads = pick({1, 2, 4, 8});
  d.num_q_heads = d.num_kv_heads * pick({1, 2, 7, 16});
  d.head_dim = pick({64, 128, 256});
  d.causal = pick({0, 1});
  d.window = pick({0, 0, 500});
  d.scale = 0.1f;
  d.q_dtype = pick({SKV_F32, SKV_BF16, SKV_F16});
  d.kv_dtype = pick({SKV_F32, SKV_BF16, SKV_INT8, SKV_FP8_E4M3});
  d.block_size = pick({1, 8, 16, 128});
  d.max_pages = pick({1, 100});
  d.kv_capacity = pick({64, 4096});
  d.v_layout = pick({0, 1});
  d.has_sink = pick({0, 1});
  d.impl = pick({0, 1, 2});
  d.record_dtype = pick({SKV_F32, SKV_BF16});
  if (rng() % 2) {
    const int bad = pick({-1, 0, 3, 7, 65, 96, 512, 1 << 22, 5000});
    switch (rng() % 12) {
      case 0: d.batch = bad; break;
      case 1: d.q_rows = bad; break;
      case 2: d.num_q_heads = bad; break;
      case 3: d.head_dim = bad; break;
      case 4: d.causal = bad; break;
      case 5: d.window = bad; break;
      case 6: d.q_dtype = bad; break;
      case 7: d.kv_dtype = bad; break;
      case 8: d.block_size = bad; break;
      case 9: d.max_pages = bad; break;
      case 10: d.impl = bad; break;
      default: d.record_dtype = bad; break;
    }
  }
  return d;
}

int main() {
  std::mt19937 rng(12345);
  // ---- planner over random hints and lengths
  for (int trial = 0; trial < 3000; ++trial) {
    skv_plan_hints h;
    memset(&h, 0, sizeof(h));
    const int B = 1 + (int)(rng() % (trial % 10 == 0 ? 3000 : 40));
    h.batch = B;
    h.q_rows = 1 + (int)(rng() % 16);
    h.num_kv_heads = 1 + (int)(rng() % 8);
    h.causal = (int)(rng() % 2);
    h.window = (rng() % 3 == 0) ? (int)(rng() % 5000) : 0;
    h.num_cus = (int)(rng() % 3) * 128;
    h.ctas_per_cu = (int)(rng() % 3);
    h.partitions_per_request = (rng() % 4 == 0) ? (int)(rng() % 300) : 0;
    h.max_partitions = (int)(rng() % 4) * 100;
    h.work_per_partition = (int)(rng() % 2) * 7000;
    h.min_tokens_per_partition = (int)(rng() % 3) * 300;
    h.workgroups_per_head = (int)(rng() % 4);
    std::vector<int32_t> ctx(B);
    for (auto& c : ctx) {
      const int k = (int)(rng() % 6);
      c = k == 0 ? 0 : k == 1 ? 1 : k == 2 ? (int)(rng() % 100) : k == 3 ? (int)(rng() % 20000) : (int)(rng() % 300000);
    }
    int32_t C = 0;
    CHECK(skv_plan_capacity(&h, ctx.data(), &C) == SKV_OK);
    CHECK(C >= B);
    // capacity as computed, and a tight one that forces trimming
    for (int32_t cap : {C, B + (C - B) / 3}) {
      const int64_t n = skv_plan_meta_len(B, cap);
      std::vector<int32_t> meta((size_t)n + 8, -12345);
      skv_plan_info info;
      CHECK(skv_plan_fill(&h, ctx.data(), cap, meta.data(), n, &info) == SKV_OK);
      CHECK(meta[n] == -12345 && meta[n + 7] == -12345);      // nothing past the block
      CHECK(meta[0] == B && meta[1] == cap && meta[2] == info.num_items && info.num_items <= cap);
      int64_t sum = 0;
      for (int b = 0; b < B; ++b) {
        CHECK(meta[4 + b] >= 1 && meta[4 + b] <= SKV_MAX_SPLITS);
        CHECK(meta[4 + B + b] == sum);
        sum += meta[4 + b];
      }
      CHECK(sum == info.num_items);
      std::vector<int> seen((size_t)B * 256, 0);
      for (int i = 0; i < cap; ++i) {
        const int w = meta[4 + 2 * B + i];
        if (i >= info.num_items) {
          CHECK(w == -1);
          continue;
        }
        const int b = w / 256, s = w % 256;
        CHECK(b >= 0 && b < B && s < meta[4 + b]);
        CHECK(seen[(size_t)b * 256 + s]++ == 0);
      }
      CHECK(skv_plan_fill(&h, ctx.data(), cap, meta.data(), n - 1, &info) != SKV_OK);   // short block
    }
    if (skv_plan_fill(&h, ctx.data(), B - 1, nullptr, 0, nullptr) == SKV_OK) return 1;
  }
  // ---- descriptors: validation, sizes, hints, and compute calls that must fail
  int accepted = 0;
  for (int trial = 0; trial < 20000; ++trial) {
    skv_desc d = random_desc(rng);
    const int paged = (int)(rng() % 2);
    const int v = skv_validate(&d, paged, (int)(rng() % 3), nullptr);
    size_t mb = 0, lb = 0, ab = 0;
    const int ws = skv_workspace_size(&d, (int64_t)(rng() % 1000), &mb, &lb, &ab);
    (void)ws;
    skv_plan_hints h;
    const int hr = skv_plan_hints_for_desc(&d, paged, &h);
    if (v == SKV_OK) {
      ++accepted;
      CHECK(hr == SKV_OK);
      CHECK(h.batch == d.batch && h.q_rows == d.q_rows && h.ctas_per_cu >= 1 && h.workgroups_per_head >= 1);
    }
    // compute calls with NULL arguments never launch
    skv_args a;
    memset(&a, 0, sizeof(a));
    const int before = skv::g_launches;
    CHECK(skv_attention_decode_paged(&d, &a, nullptr) != SKV_OK);
    CHECK(skv_attention_decode(&d, &a, nullptr) != SKV_OK);
    CHECK(skv_attention_decode_paged_splitkv(&d, &a, 4, nullptr, nullptr) != SKV_OK);
    CHECK(skv_splitkv_combine(&d, &a, 4, nullptr, nullptr, nullptr) != SKV_OK);
    CHECK(skv::g_launches == before);
  }
  CHECK(accepted > 100);
  printf("host fuzz ok: %d descriptors accepted\n", accepted);
  return 0;
}
