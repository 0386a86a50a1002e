/*
 * skv.h -- C ABI of the split-KV (flash-decoding) paged decode-attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * A few query rows per request (one decode token, a speculative-verify block,
 * or MTP rows) attend over a long KV cache that is contiguous or paged through
 * a page table. The split-KV calls partition each request's visible key range
 * into splits, run one workgroup per (split, KV head) that emits partial
 * softmax statistics, and merge the splits in a second kernel.
 *
 * Sources, by page title and section:
 *   [DR]  tiny-llm #11, "split-KV decode attention design record":
 *         "Design" (partial kernel over (head, split) with chunk =
 *         ceil(visible / splits) computed from a device visible length,
 *         (m_i, l_i, acc_i) records, a combine kernel; host num_splits,
 *         preallocated partial buffers, no allocation and no device-to-host
 *         copy so calls stay graph-capturable; the single-pass entry points
 *         keep num_splits = 1 semantics), "points for reviewer decision"
 *         (Q1 separate combine kernel, Q2 host num_splits, Q3/Q4 the
 *         single-split bitwise anchor exp(0) = 1 and 1/(l + 1e-9), Q5 the
 *         caller may fall back to one split).
 *   [VS]  hipfire #760, "split packed-Q8 verifier KV scans", Summary: the
 *         causal prefix of a multi-row verifier split over 2/4/8 workgroups,
 *         stable max-LSE merge; int8 ("Q8") KV; fail-closed admission.
 *   [PA]  aiter #5628, "tune MTP work budgets and planned reduction":
 *         intro and Changes (host work planner from host-known KV work,
 *         per-request partition counts, capacity fixed for graph replay,
 *         explicit budgets and caps take precedence, windowed work capped by
 *         the causal-window union and tile alignment, reducer that iterates
 *         only each request's actual partitions up to 256, sink
 *         normalization, masked fallback, window checks); Performance (BF16
 *         Q/O, FP8 KV with per-token FP32 scales, MTP4 causal rows, page
 *         sizes 16 and 128, plain and transposed V).
 *
 * Conventions shared by every call
 * --------------------------------
 *  * All pointers in skv_args and skv_partials are DEVICE pointers; the
 *    caller owns every buffer and the stream. No call allocates, frees,
 *    synchronizes or copies device-to-host; every compute call only enqueues
 *    kernels on `stream` (a hipStream_t passed as void*, NULL = the null
 *    stream), so all compute calls can be captured into a HIP graph.
 *  * Every call validates its host arguments before enqueuing anything and
 *    returns 0 on success or a negative SKV_ERR_* code; on error nothing was
 *    enqueued (fail closed, [VS] Summary).
 *  * Device values (context lengths, page-table entries) cannot be checked
 *    without a device-to-host copy. Kernels clamp each context length to
 *    [0, capacity] where capacity = max_pages * block_size (paged) or
 *    kv_capacity (contiguous), and read only page-table entries
 *    [0, ceil(ctx / block_size)) of a request. Entries there must be valid
 *    page indices of the pool; an invalid index is undefined behaviour.
 *
 * Shapes and layouts (row-major, innermost last)
 *   q, o          [B][R][Hq][D]   q_dtype (F32, BF16 or F16); o has q's
 *                                 dtype, 16-bit results are rounded to
 *                                 nearest even.
 *   paged k       [pages][Hkv][block_size][D]
 *   paged v       PLAIN: as k;  TRANSPOSED: [pages][Hkv][D][block_size]
 *   paged scales  [pages][Hkv][block_size] fp32 (INT8 / FP8 KV only; one
 *                 scale per token per KV head for K and one for V)
 *   contiguous k  [B][Hkv][kv_capacity][D]; v PLAIN as k, TRANSPOSED
 *                 [B][Hkv][D][kv_capacity]; scales [B][Hkv][kv_capacity]
 *   page_table    int32 [B][max_pages]: logical page i of request b is pool
 *                 page page_table[b * max_pages + i]
 *   ctx_lens      int32 [B] device visible lengths (the keys of a request,
 *                 its R query tokens included)
 *   sinks         fp32 [Hq] per-query-head sink logits (natural-log units)
 *   tree_mask     uint64 [B][R][ceil(R / 64)] verify masks (optional, see below)
 *
 * Semantics (readings of the pages where they leave a step open)
 *   Query head h uses KV head h / (Hq / Hkv). Causal row j of a request of
 *   length ctx sits at position p_j = ctx - R + j (non-causal rows: ctx - 1)
 *   and sees keys t in [0, ctx) with t <= p_j and, when window W > 0,
 *   t > p_j - W. The logit of key t is x_t = scale * k_scale_t * <q, code_t>.
 *   O = sum_t e^(x_t - M) v_t / (sum_t e^(x_t - M) [+ e^(sink_h - M)]).
 *   A row that sees no key outputs 0 (with or without a sink).
 *
 * Verify masks ([VS] Summary names tree-structured and independent-batch
 * verification beside the causal multi-row route without defining them; the
 * reading here): the R query tokens of a causal request are the draft tokens
 * at keys ctx - R .. ctx - 1, in an order where every token comes after its
 * ancestors. With args.tree_mask set, row j sees the committed prefix
 * t < ctx - R as before, and draft key ctx - R + i only when bit i % 64 of
 * word tree_mask[(b * R + j) * W + i / 64] is set, W = ceil(R / 64) (and
 * i <= j: a row never sees a later draft; a window still applies on top).
 * Causal verification is the mask with bits 0..j set; tree verification sets
 * the bits of the token's ancestors and itself; independent-batch
 * verification sets bit j alone. Requires causal = 1 and
 * R <= SKV_MAX_VERIFY_ROWS (SKV_ERR_UNSUPPORTED otherwise). Split ranges and
 * records are unchanged.
 *
 * Split ranges ([DR] Design; [PA] Changes). For a request with S splits the
 * split range is [u, ctx) where u = 0, or with a window the earliest row's
 * window start aligned down to SKV_SPLIT_ALIGN; chunk = ceil((ctx - u) / S)
 * rounded up to SKV_SPLIT_ALIGN; split s covers
 * [u + s * chunk, min(u + (s + 1) * chunk, ctx)), possibly empty.
 *
 * Partial records (caller-owned scratch, [DR] Design / Q4). A record holds,
 * for every one of the rho = R * Hq / Hkv query rows that share a KV head
 * (row index r = j * (Hq / Hkv) + (h mod (Hq / Hkv))), three fp32 values of
 * the split's visible keys T_s:
 *   m   a reference maximum in log2 units, l = sum_{t in T_s} 2^(x_t log2(e) - m),
 *   acc[D] = sum_{t in T_s} 2^(x_t log2(e) - m) v_t.
 * (m is at least the largest x_t log2(e) - 8, so l and acc stay finite.)
 * acc is stored as fp32, or as bf16 (round to nearest even) when the
 * descriptor's record_dtype is SKV_BF16: half the record bytes, the layout of
 * the planned-reduction page ([PA] Changes: bf16 partial output plus two fp32
 * per row; here the un-normalised acc with m and l). bf16 records are an
 * option, not the default: their rounding moves an output element by up to
 * 2^-8 * sum_t p_t |v_t| / sum_t p_t, so where values of opposite sign in
 * different splits cancel, the result can exceed atol = rtol = 5e-3 against
 * the exact merge (measured: |d| 0.021 at |O| 0.03 with queries scaled by 8).
 * fp32 records (the default) carry no such term.
 * An empty T_s gives m = -inf, l = 0, acc = 0. Record slot numbers:
 *   uniform splits:  slot = ((b * S) + s) * Hkv + g
 *   planned splits:  slot = (req_slot0[b] + s) * Hkv + g
 * and m[slot * rho + r], l[slot * rho + r], acc[(slot * rho + r) * D + d].
 * The merge ([DR] Design, Q3; [PA] Changes): M = max over splits with l > 0
 * (and the sink logit in log2 units); L = sum_s 2^(m_s - M) l_s
 * (+ 2^(sink log2(e) - M)); O = (sum_s 2^(m_s - M) acc_s) * (1 / (L + 1e-9)),
 * splits taken in increasing s. A merge of one record is exactly the
 * single-pass finalization, so a request with one split (num_splits = 1, or
 * P_b = 1 in a plan) gets its output from the partial stage directly, with
 * the same bits as the single-pass entry points, writes no record, and the
 * combine stage leaves it alone.
 */
#ifndef SKV_H_
#define SKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKV_ABI_VERSION 4
#define SKV_SPLIT_ALIGN 64    /* split boundaries are multiples of this many tokens */
#define SKV_PLAN_DEVICE_MAX_BATCH 2048   /* largest batch skv_plan_refresh_device plans */
#define SKV_MAX_SPLITS 256    /* per request ([PA] Changes: maximum of 256) */
#define SKV_MAX_VERIFY_ROWS 256   /* query rows per request with verify masks (four mask words) */
#define SKV_PLAN_INLINE_MAX 480   /* int32 of a plan block skv_attention_decode_paged_planned_host takes */
/* The planner's default cap on partitions per request (max_partitions = 0):
 * a merge visits every record of a request, so past this many partitions
 * the merge costs more than the extra partial workgroups save (measured on
 * one 100,000- or 200,000-key request with fifteen of 1,024). An explicit
 * max_partitions up to SKV_MAX_SPLITS still applies. */
#define SKV_PLAN_DEFAULT_MAX_PARTITIONS 160

/* Status codes. */
#define SKV_OK 0
#define SKV_ERR_NULL (-1)          /* a required pointer is NULL */
#define SKV_ERR_SHAPE (-2)         /* B, R, Hq, Hkv, D, block size or strides out of range */
#define SKV_ERR_DTYPE (-3)         /* unsupported dtype or dtype combination */
#define SKV_ERR_SPLITS (-4)        /* num_splits < 1 or > SKV_MAX_SPLITS */
#define SKV_ERR_CAPACITY (-5)      /* partial buffers hold too few records */
#define SKV_ERR_UNSUPPORTED (-6)   /* valid request this library does not implement */
#define SKV_ERR_LAUNCH (-7)        /* the HIP runtime rejected a kernel launch */
#define SKV_ERR_PLAN (-8)          /* inconsistent plan hints or metadata sizes */
#define SKV_ERR_ALIGN (-9)         /* partials.acc is not 16-byte aligned */
#define SKV_ERR_SCRATCH (-10)      /* the call needs more than the library's static scratch */

/* Bytes of the library's static device scratch (one copy per GPU it runs on,
 * held until the process ends): the partial records of the allocation-free
 * call live there. */
#define SKV_STATIC_SCRATCH_BYTES ((size_t)128 << 20)

typedef enum skv_dtype {
  SKV_F32 = 0,
  SKV_BF16 = 1,
  SKV_INT8 = 2,       /* KV only: symmetric int8 codes times an fp32 scale */
  SKV_FP8_E4M3 = 3,   /* KV only: OCP e4m3fn codes times an fp32 scale */
  SKV_F16 = 4         /* Q/O only: IEEE binary16 ([PA] Validation: FP16 coverage); O by RNE */
} skv_dtype;

typedef enum skv_v_layout { SKV_V_PLAIN = 0, SKV_V_TRANSPOSED = 1 } skv_v_layout;

/* Kernel family selection. AUTO picks the matrix-core kernel when q is BF16
 * and KV is BF16, INT8 or FP8, or q is F16 and KV is INT8 or FP8 (page size
 * >= 16; not BF16 KV at D 256), else the vector kernel; MFMA outside those
 * cases is SKV_ERR_UNSUPPORTED. */
typedef enum skv_impl { SKV_IMPL_AUTO = 0, SKV_IMPL_VALU = 1, SKV_IMPL_MFMA = 2 } skv_impl;

/* Host description of one call; fixed for the life of a captured graph. */
typedef struct skv_desc {
  int32_t batch;          /* B >= 1 */
  int32_t q_rows;         /* R >= 1 query rows per request */
  int32_t num_q_heads;    /* Hq, a multiple of Hkv */
  int32_t num_kv_heads;   /* Hkv >= 1 */
  int32_t head_dim;       /* D in {64, 128, 256} */
  int32_t causal;         /* 1: row j sits at ctx - R + j; 0: every row at ctx - 1 */
  int32_t window;         /* sliding window W in keys, 0 = none */
  float scale;            /* logit scale, usually 1/sqrt(D) */
  int32_t q_dtype;        /* SKV_F32, SKV_BF16 or SKV_F16 (o has the same dtype) */
  int32_t kv_dtype;       /* skv_dtype */
  int32_t block_size;     /* paged: tokens per page, power of two in [1, 1024] */
  int32_t max_pages;      /* paged: page-table row stride (>= 1) */
  int32_t kv_capacity;    /* contiguous: token stride per (request, KV head) */
  int32_t v_layout;       /* skv_v_layout */
  int32_t has_sink;       /* 1: args.sinks holds Hq fp32 logits */
  int32_t impl;           /* skv_impl */
  int32_t record_dtype;   /* partial-record acc: SKV_F32 (0) or SKV_BF16; else SKV_ERR_DTYPE */
} skv_desc;

/* Device pointers of one call (k_scale / v_scale only for INT8 / FP8 KV,
 * page_table only for paged calls, sinks only with has_sink, tree_mask
 * optional). */
typedef struct skv_args {
  const void* q;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const int32_t* page_table;
  const int32_t* ctx_lens;
  const float* sinks;
  void* o;
  const uint64_t* tree_mask;   /* NULL, or [B][R][ceil(R / 64)] verify masks (see above) */
} skv_args;

/* Caller-owned partial-record buffers (device memory), sized by
 * skv_workspace_size for `capacity_slots` records. `acc` holds fp32 or bf16
 * values (the descriptor's record_dtype) and must be 16-byte aligned (its
 * records are written and read as 4-element vectors); SKV_ERR_ALIGN
 * otherwise. */
typedef struct skv_partials {
  float* m;
  float* l;
  void* acc;
  int64_t capacity_slots;
} skv_partials;

/* ---- version, status ---------------------------------------------------- */

int skv_abi_version(void);
/* Static string naming a status code; never NULL. */
const char* skv_status_str(int status);

/* ---- host-only checks and sizes (no HIP call; usable without a GPU) ------ */

/* Validate a descriptor for a paged (paged = 1) or contiguous call with
 * num_splits splits (0 = a single-pass call) and optional partial buffers.
 * Returns SKV_OK or the error the corresponding compute call would return. */
int skv_validate(const skv_desc* d, int32_t paged, int32_t num_splits, const skv_partials* p);

/* Bytes of m, l and acc for `slots` partial records of descriptor d:
 * slots * rho * 4, slots * rho * 4 and slots * rho * D * (4, or 2 for bf16
 * records). Any output pointer may be NULL. */
int skv_workspace_size(const skv_desc* d, int64_t slots, size_t* m_bytes, size_t* l_bytes,
                       size_t* acc_bytes);

/* The same sizes under the split-KV name ([DR] Design: preallocated partial
 * buffers sized by the caller): identical to skv_workspace_size. */
int skv_splitkv_workspace_size(const skv_desc* d, int64_t slots, size_t* m_bytes, size_t* l_bytes,
                               size_t* acc_bytes);

/* Records needed by a uniform split call: B * num_splits * Hkv. */
int64_t skv_uniform_slots(const skv_desc* d, int32_t num_splits);

/* ---- single-pass entry points ([DR] Design: num_splits = 1 semantics) --- */

/* Contiguous KV, one pass per (request, KV head); writes o. */
int skv_attention_decode(const skv_desc* d, const skv_args* a, void* stream);
/* Paged KV, one pass per (request, KV head); writes o. */
int skv_attention_decode_paged(const skv_desc* d, const skv_args* a, void* stream);

/* ---- split-KV entry points ([DR] Design) ---------------------------------
 * num_splits is a host integer in [1, SKV_MAX_SPLITS], the same for every
 * request; partials must hold skv_uniform_slots(d, num_splits) records.
 * Enqueues the partial kernel and then the combine kernel. */
int skv_attention_decode_splitkv(const skv_desc* d, const skv_args* a, int32_t num_splits,
                                 const skv_partials* p, void* stream);
int skv_attention_decode_paged_splitkv(const skv_desc* d, const skv_args* a, int32_t num_splits,
                                       const skv_partials* p, void* stream);

/* ---- allocation-free split-KV call -----------------------------------------
 * For callers that cannot allocate device memory at all (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as skv_attention_decode_paged_splitkv, same kernels and results, with
 * the partial records in the library's static device scratch instead of
 * caller buffers. Nothing is allocated or freed. The records of B *
 * num_splits * Hkv slots (m, l and fp32 or bf16 acc, each region 256-byte
 * aligned) must fit in SKV_STATIC_SCRATCH_BYTES; SKV_ERR_SCRATCH otherwise,
 * before anything is enqueued. The first call on a device looks the scratch
 * up on that device (a HIP symbol query; SKV_ERR_LAUNCH if it fails). Every
 * call on one GPU shares that GPU's scratch: calls that overlap in time on
 * one GPU (other streams, other threads) race and are not allowed. No
 * scratch content needs to start at any value: every record a call's
 * combine reads is written by the same call's partial stage. */
int skv_attention_decode_paged_splitkv_noalloc(const skv_desc* d, const skv_args* a, int32_t num_splits,
                                               void* stream);

/* ---- host split planner ([PA] intro, Changes) -----------------------------
 * The planner turns host-known context lengths into per-request partition
 * counts P_b and a work list, written as an int32 metadata block that the
 * caller copies to the device (e.g. hipMemcpyAsync from pinned memory on the
 * compute stream) and passes to the planned call. Layout of the block:
 *   [0] B   [1] capacity_items C   [2] num_items = sum_b P_b   [3] max_b P_b
 *   [4, 4 + B)            P_b
 *   [4 + B, 4 + 2B)       req_slot0[b] = sum_{b' < b} P_b'
 *   [4 + 2B, 4 + 2B + C)  work item i: b * 256 + s, or -1 for an unused item
 * Items are ordered longest first. A plan's capacity is fixed when it is
 * made; refreshing it with new lengths keeps C (graph replay launches C
 * items) and lowers partition counts if they would exceed it.
 * Counts: an explicit partitions_per_request takes precedence; otherwise
 * ceil(span * R / work_per_partition), raised, when the batch does not fill
 * the base budget num_cus * ctas_per_cu / (Hkv * workgroups_per_head)
 * partitions, to the request's span share of it (never below
 * min_tokens_per_partition keys per partition); always within
 * [1, min(max_partitions, 64-key tiles of the span)].
 */
typedef struct skv_plan_hints {
  int32_t batch;                   /* B */
  int32_t q_rows;                  /* R, the query length */
  int32_t num_kv_heads;            /* Hkv */
  int32_t causal;
  int32_t window;                  /* 0 = none; work is capped by the causal-window union */
  int32_t num_cus;                 /* 0 = 256 */
  int32_t ctas_per_cu;             /* base occupancy budget per CU, 0 = 2 */
  int32_t partitions_per_request;  /* > 0: explicit P_b for every request (precedence) */
  int32_t max_partitions;          /* cap on P_b, 0 = SKV_PLAN_DEFAULT_MAX_PARTITIONS */
  int32_t work_per_partition;      /* target key-rows (keys * R) per partition, 0 = 50000 */
  int32_t min_tokens_per_partition;/* 0 = 256 */
  int32_t workgroups_per_head;     /* workgroups one partition of one KV head occupies, 0 = 1 */
  int64_t total_context_length;    /* optional work hint: sum of contexts to size capacity */
} skv_plan_hints;

typedef struct skv_plan_info {
  int32_t num_items;       /* sum_b P_b */
  int32_t capacity_items;  /* C */
  int32_t max_partitions;  /* max_b P_b */
  int32_t min_partitions;  /* min_b P_b */
  int64_t slots;           /* C * Hkv partial records the planned call needs */
} skv_plan_info;

/* int32 entries of a metadata block for B requests and capacity C. */
int64_t skv_plan_meta_len(int32_t batch, int32_t capacity_items);

/* Planner hints for calls with descriptor d (paged or contiguous): batch,
 * rows, heads, causal and window from d, and the budget of the kernel family
 * d selects. Matrix-core kernel: one workgroup per CU (ctas_per_cu 1) and
 * one per group of 32 or 64 query rows of a KV head (workgroups_per_head),
 * so the raise fills at most one round of the GPU. Vector kernel: one-wave
 * workgroups, 16 per CU, 8 rows each, partitions down to one 64-key tile.
 * Other fields 0 (defaults); the caller may override any of them. Host-only. */
int skv_plan_hints_for_desc(const skv_desc* d, int32_t paged, skv_plan_hints* h);

/* Capacity (items) a plan needs for these hints and host context lengths
 * (host_ctx may be NULL when hints->total_context_length sizes it). */
int skv_plan_capacity(const skv_plan_hints* h, const int32_t* host_ctx, int32_t* capacity_items);

/* Make or refresh a plan: fill the host metadata block `meta` of `meta_len`
 * int32 for capacity C from host context lengths. info may be NULL. */
int skv_plan_fill(const skv_plan_hints* h, const int32_t* host_ctx, int32_t capacity_items,
                  int32_t* meta, int64_t meta_len, skv_plan_info* info);

/* A plan as one caller-owned object ([PA] intro, Changes: the plan is made
 * once with a fixed capacity and refreshed per call from host-known lengths).
 * skv_plan_make copies the hints, fixes capacity_items and sets meta_len; the
 * caller then points `meta` at a host buffer of meta_len int32 (pinned memory
 * when it is copied to the device asynchronously) that it owns.
 * skv_plan_refresh fills that buffer and `info` from host context lengths,
 * keeping capacity_items. Host-only; no HIP call. */
typedef struct skv_plan {
  skv_plan_hints hints;      /* copied by skv_plan_make */
  int32_t capacity_items;    /* C, fixed by skv_plan_make */
  int64_t meta_len;          /* int32 entries the metadata block needs */
  int32_t* meta;             /* caller-owned host buffer of meta_len int32 */
  skv_plan_info info;        /* counts of the last refresh */
} skv_plan;

/* Make a plan. Capacity: plan->capacity_items when the caller set it > 0 on
 * entry (e.g. from skv_plan_capacity with the host lengths), else sized from
 * the work hint hints->total_context_length (SKV_ERR_PLAN with neither).
 * Sets hints, capacity_items and meta_len, zeroes info; meta is untouched. */
int skv_plan_make(const skv_plan_hints* h, skv_plan* plan);

/* Refresh a made plan from host context lengths (plan->meta must be set):
 * skv_plan_fill with the plan's hints and capacity. */
int skv_plan_refresh(skv_plan* plan, const int32_t* host_ctx);

/* Device-side refresh ([PA] intro, Changes; graph replay with changing
 * lengths): fill the DEVICE metadata block `meta_dev` (meta_len int32, for
 * capacity C) from the DEVICE context lengths `ctx_dev` [B] with one kernel
 * on `stream`; the block is bit-identical to what skv_plan_fill writes for
 * the same lengths. Nothing is copied to the host, so a captured step
 * (refresh, then the planned call) re-plans on every replay. Host checks as
 * skv_plan_fill; B <= SKV_PLAN_DEVICE_MAX_BATCH (SKV_ERR_UNSUPPORTED
 * otherwise). */
int skv_plan_refresh_device(const skv_plan_hints* h, const int32_t* ctx_dev, int32_t capacity_items,
                            int32_t* meta_dev, int64_t meta_len, void* stream);

/* Paged split-KV over a plan: plan_meta is the DEVICE copy of the block,
 * capacity_items its C (the grid size), partials hold C * Hkv records. */
int skv_attention_decode_paged_planned(const skv_desc* d, const skv_args* a,
                                       const int32_t* plan_meta, int32_t capacity_items,
                                       const skv_partials* p, void* stream);

/* The same call with the plan block in HOST memory (plan_meta_host, as
 * skv_plan_fill or skv_plan_refresh wrote it) instead of a device copy: the
 * block travels to the kernels by value, inside their argument block, so no
 * host-to-device copy precedes the call and the caller may refill the host
 * buffer as soon as the call returns. For plans of at most
 * SKV_PLAN_INLINE_MAX int32 (4 + 2 B + C; SKV_ERR_UNSUPPORTED above, e.g.
 * B200 x 200k with C = 3200 uses the device copy); the block's header must
 * say B and C (SKV_ERR_PLAN otherwise). Outputs are bit-identical to
 * skv_attention_decode_paged_planned with the same plan. */
int skv_attention_decode_paged_planned_host(const skv_desc* d, const skv_args* a,
                                            const int32_t* plan_meta_host, int32_t capacity_items,
                                            const skv_partials* p, void* stream);

/* ---- the two stages on their own -----------------------------------------
 * skv_splitkv_partial enqueues only the partial kernel, skv_splitkv_combine
 * only the combine kernel; a split-KV call is exactly the two in order. The
 * partial stage writes o for requests with one split (see the merge above).
 * plan_meta NULL selects uniform splits (num_splits); otherwise num_splits
 * must be the plan's capacity C. */
int skv_splitkv_partial(const skv_desc* d, const skv_args* a, int32_t paged, int32_t num_splits,
                        const int32_t* plan_meta, const skv_partials* p, void* stream);
int skv_splitkv_combine(const skv_desc* d, const skv_args* a, int32_t num_splits,
                        const int32_t* plan_meta, const skv_partials* p, void* stream);

/* ---- single-kernel split + merge ([DR] points for reviewer decision, Q1) ----
 * The partial stage alone, arguments as skv_splitkv_partial, where the last
 * workgroup to finish among those of a (request, KV head) also merges that
 * pair's records into o, in increasing split order with the arithmetic of
 * skv_splitkv_combine: o is bit-identical to the two-stage call, whichever
 * workgroup arrives last.
 * counters: DEVICE int32 [B * Hkv], all zero before the first call; each
 * call leaves them zero again, so the call can be captured and replayed.
 * Calls that overlap in time on one counters buffer race and are not
 * allowed; a call that fails validation touches nothing. SKV_ERR_NULL when
 * counters is NULL. */
int skv_splitkv_fused(const skv_desc* d, const skv_args* a, int32_t paged, int32_t num_splits,
                      const int32_t* plan_meta, const skv_partials* p, int32_t* counters, void* stream);

/* ---- measurement: the read ceiling of a paged layout -----------------------
 * Not part of the attention path. Reads exactly the K and V codes and scales
 * a paged split-KV call with these arguments reads (the effective bytes of
 * [PA] Performance, bandwidth note), with the matrix-core partial kernel's
 * memory pattern: one workgroup per (work item, KV head), four key streams of
 * 32-key blocks, page-table reads per 16-key group, 16-byte-per-lane
 * direct-to-LDS loads of whole rows, the same ring depth, one workgroup
 * barrier per block with all but one stage in flight (the faster of the
 * partial kernel's two load schedules when nothing is computed), and no
 * arithmetic. Its time is the floor those loads put under the partial
 * kernel. Work items as skv_splitkv_partial (plan_meta NULL:
 * uniform num_splits; else the device plan block, num_splits = its C).
 * sink: DEVICE uint32 [sink_len] >= items * Hkv (one value per workgroup,
 * overwritten). Paged calls with block_size >= 16 and 8-bit codes, or bf16
 * codes at D <= 128; SKV_ERR_UNSUPPORTED otherwise. */
int skv_gather_ceiling(const skv_desc* d, const skv_args* a, int32_t num_splits, const int32_t* plan_meta,
                       uint32_t* sink, int64_t sink_len, void* stream);

#ifdef __cplusplus
}  /* extern "C" */
#endif

#endif  /* SKV_H_ */
