/*
 * attn_decode.h -- C ABI of libsplitkv: split-KV paged decode attention for
 * MI355X (gfx950).
 *
 * The operation (aiter PR #4758, "[Gluon][MLA] Deeper async-copy pipeline in
 * the bh16 stage-1 decode loop": Motivation and Technical Details items 1-3):
 * every decode request's cached keys are cut into splits; a stage-1
 * workgroup per (request, KV head, split) gathers its keys through the page
 * table, scores them against all query rows that share the KV head (a GQA
 * group, or all heads of an MLA latent head), keeps the running max and sum
 * of the softmax and accumulates P.V, writing a normalised partial output and
 * its log-sum-exp; stage 2 merges the splits of each query row by
 * log-sum-exp.  For every (request b, query position j, query head h):
 *
 *     n      = ctx[b]                         (not causal)
 *            = ctx[b] - q_len + 1 + j         (causal, bottom-right aligned)
 *     s_t    = scale * <q[b,j,h,:], K_t[:Dk]>,     t in [0, n)
 *     out    = sum_t e^(s_t - m) V_t / sum_t e^(s_t - m),   m = max_t s_t
 *     lse    = m + ln sum_t e^(s_t - m)        (natural log; -inf if n = 0)
 *
 * with key t of request b stored at page page_table[b][t / P], slot t % P,
 * and query head h reading KV head h / (H_q / H_kv).
 *
 * Split rule (host and device agree; attn_decode_split_range exposes it):
 * chunk = A * ceil(ceil(ctx / S) / A) with A = split_align (64 keys); split s
 * covers [s*chunk, min((s+1)*chunk, ctx)).  The 64-key block is the block
 * the trip counts of the aiter PR's Test Result tables imply.  A plan with
 * split_chunk > 0 (attn_decode_plan_lens) uses chunk = split_chunk for every
 * request instead, and request b has n_b = ceil(host_len[b] / chunk) splits
 * (plan->split_start), so requests hold splits in proportion to their
 * lengths; its partials fill slots 0 .. n_b - 1 of the S (= plan->num_splits,
 * the largest n_b) slots per row, and the merge reads those slots only.
 *
 * Memory layouts (all device memory, caller-owned, element strides):
 *   q            [B, q_len, H_q, Dk]  contiguous, dtype
 *   k_cache      element (page, kvh, slot, d) at
 *                page*k_stride_page + kvh*k_stride_head + slot*k_stride_tok + d
 *   v_cache      same with v_strides; when v_aliases_k, V is K[..., :Dv] and
 *                v_cache must equal k_cache
 *   page_table   int32 [B, max_pages_per_req] row-major; entries past
 *                ceil(ctx/P) are never used (a single-request plan may read,
 *                and then ignore, entries up to ceil(max_context_len/P))
 *   context_lens int32 [B]
 *   out          [B, q_len, H_q, Dv] contiguous, dtype
 *   lse          float [B, q_len, H_q] (optional)
 *   workspace    float o_part [B, q_len, H_q, S, Dv] at o_part_offset and
 *                float lse_part [B, q_len, H_q, S] at lse_part_offset
 *                (attn_decode_workspace_layout), S = the run's split count;
 *                a plan made with ATTN_PLAN_FUSED_MERGE also keeps one
 *                uint32 counter per (request, KV head, head tile) at offset 0,
 *                before o_part
 *
 * Threading and ownership: the library allocates nothing and keeps no device
 * memory besides the static scratch of attn_decode_run_noalloc (below);
 * run/partials/merge only validate host-side arguments, enqueue
 * kernels on `stream` (a hipStream_t; NULL = the null stream) and return
 * without synchronising, so they may be captured into a HIP graph.  Device
 * data (page ids, context lengths) is not validated: page ids must lie in
 * [0, num_pages) and 0 <= ctx <= max_pages_per_req * P, or the kernels read
 * out of bounds.  With causal rows and ctx < q_len, the first q_len - ctx
 * rows see no key and return 0 / -inf (a varlen prefill batch right-aligns
 * each sequence this way).  The plan is a plain struct the caller owns and
 * may copy.
 *
 * Errors: every call returns an attn_status; the thread-local text of the
 * last failure is attn_decode_last_error().  No call aborts the process.
 */
#ifndef SPLITKV_ATTN_DECODE_H
#define SPLITKV_ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,        /* bad argument: null pointer, bad size or stride */
  ATTN_EUNSUPPORTED = 2,  /* no kernel is built for this dtype/dims/layout */
  ATTN_EWORKSPACE = 3,    /* num_splits above plan.max_splits, or workspace too small */
  ATTN_EHIP = 4           /* HIP runtime error; text in attn_decode_last_error() */
} attn_status;

typedef enum attn_dtype { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/* Plan flags. */
enum {
  ATTN_PLAN_POLICY_P2 = 1,          /* split count = max(1, 256 / batch), the policy the
                                       aiter PR's per-lever table was measured at */
  ATTN_PLAN_NO_XCD_REMAP = 2,       /* keep the plain (split-minor) workgroup order */
  ATTN_PLAN_FUSED_MERGE = 4,        /* run merges in stage 1 when 2 <= S <= 64: the workgroup
                                       that finishes a row group's last split merges the group,
                                       so no second launch waits on an idle part (aiter PR
                                       #4758, Motivation, batch-1 paragraph).  Matrix-core
                                       plans only; the workspace counters need
                                       attn_decode_workspace_init.  Off by default: on
                                       MI355X merging a whole group's partials on one CU
                                       (with the per-XCD L2 write-back of each release)
                                       takes longer than the launch it saves */
  ATTN_PLAN_PRIVATE_PAGES = 8,      /* performance hint: no KV page is shared between the
                                       batch's requests.  With 16-63 query rows per KV head
                                       the planner then takes the one-wave ring shape, which
                                       streams private pages faster, instead of four key
                                       streams, which compute four blocks at once and pay off
                                       when requests re-read shared prefix pages from the L2;
                                       and with fewer rows, one one-wave workgroup per CU
                                       instead of two at head dim 128 and two instead of four
                                       at 64 (more keep the CUs' work rate up when the L2
                                       serves shared pages).
                                       Results do not depend on it (either shape is exact) */
  ATTN_PLAN_SHARED_PASS = 16        /* shared-prefix plans only: run the shared pass where the
                                       planner would take the default plan
                                       (attn_decode_plan_prefix) */
};

/* Kernel families the planner picks from. */
enum {
  ATTN_VARIANT_VALU = 1,            /* vector-ALU stage 1 (fp32: head dims 64/64, 128/128) */
  ATTN_VARIANT_MFMA = 2             /* matrix-core stage 1 (bf16: head dims 64/64, 128/128,
                                       256/256, 576/512 with V = K[:512]) */
};

/* Requests a plan's split table covers (attn_decode_plan_lens). */
#define ATTN_MAX_SPLIT_TABLE 64

/* Shape and layout of one decode call; filled by the caller. */
typedef struct attn_decode_desc {
  int32_t batch;              /* B >= 1 requests */
  int32_t q_len;              /* query tokens per request (>= 1) */
  int32_t num_q_heads;        /* H_q, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* H_kv */
  int32_t head_dim_qk;        /* Dk */
  int32_t head_dim_v;         /* Dv (<= Dk when v_aliases_k) */
  int32_t page_size;          /* P keys per page, a power of two */
  int32_t max_pages_per_req;  /* page_table row length; max_pages_per_req * page_size <= 2^30 */
  int32_t dtype;              /* attn_dtype of q, K, V and out */
  int32_t causal;             /* 1: bottom-right causal among the q_len rows */
  int32_t v_aliases_k;        /* 1: V = K[..., :Dv] (MLA latent cache) */
  int32_t reserved;           /* must be 0 */
  int64_t num_pages;          /* pages in the pool */
  int64_t k_stride_page, k_stride_head, k_stride_tok;   /* elements */
  int64_t v_stride_page, v_stride_head, v_stride_tok;   /* elements */
} attn_decode_desc;

/* What attn_decode_plan decided.  Plain data; no device memory. */
typedef struct attn_decode_plan_t {
  attn_decode_desc desc;
  int32_t max_context_len;    /* largest ctx the plan was sized for */
  int32_t num_splits;         /* S used when run is called with num_splits = 0 */
  int32_t max_splits;         /* workspace is sized for up to this many splits */
  int32_t split_align;        /* A, keys (64) */
  int32_t variant;            /* ATTN_VARIANT_* */
  int32_t rows_per_wg;        /* query rows one stage-1 workgroup scores */
  int32_t head_tiles;         /* stage-1 workgroups per (request, KV head, split) */
  int32_t stage1_waves;       /* wavefronts per stage-1 workgroup */
  int32_t xcd_remap;          /* 1: split-major, XCD-contiguous workgroup order */
  int32_t flags;              /* ATTN_PLAN_* given to attn_decode_plan */
  int32_t split_chunk;        /* > 0: fixed split length in keys for every request (plans from
                                 attn_decode_plan_lens); 0: the split-count rule */
  int32_t live_splits;        /* with split_chunk > 0: stage-1 work items (request, split) in all,
                                 split_start[batch]; 0 otherwise */
  int64_t workspace_bytes;    /* bytes the caller must provide at max_splits */
  uint64_t key;               /* hash of every field a kernel specialisation depends on */
  int32_t split_start[ATTN_MAX_SPLIT_TABLE + 1];
                              /* with split_chunk > 0: request b owns work items
                                 [split_start[b], split_start[b+1]), its splits 0 .. n_b - 1 with
                                 n_b = ceil(host_context_lens[b] / split_chunk); unused entries 0 */
} attn_decode_plan_t;

/*
 * Plan a decode call.  Pure host function: checks the descriptor, picks the
 * kernel variant, the split count S (num_splits > 0 forces it; 0 lets the
 * policy choose so that about 256 CUs' worth of stage-1 workgroups exist,
 * aiter PR #4758, Motivation) and the workgroup order, and sizes the workspace for max(S, num_splits) splits.
 * Returns ATTN_EINVAL / ATTN_EUNSUPPORTED on a bad or unsupported shape.
 */
attn_status attn_decode_plan(const attn_decode_desc* desc, int32_t max_context_len,
                             int32_t num_splits, int32_t flags, attn_decode_plan_t* plan);

/*
 * Plan a decode call whose context lengths are known on the host:
 * host_context_lens holds `batch` lengths (host memory, read during the call
 * only).  Same as attn_decode_plan with max_context_len = their maximum,
 * except that the split policy (num_splits = 0, no ATTN_PLAN_POLICY_P2 or
 * ATTN_PLAN_FUSED_MERGE, batch <= ATTN_MAX_SPLIT_TABLE) may give every
 * request the same split length (plan->split_chunk keys, a multiple of 64)
 * instead of the same split count: request b then gets n_b =
 * ceil(host_context_lens[b] / split_chunk) splits, in proportion to its
 * length, and stage 1 runs one workgroup per (request, split) pair of that
 * flat work list (plan->split_start), so every workgroup walks about the
 * same number of keys and no workgroup is launched for a split that holds
 * none (aiter PR #4758, Motivation: the split count trades parallelism
 * against walk length).  It does so when that shortens the longest walk
 * while the work list still fits one round of workgroups on the 256 CUs.
 * Such a plan runs with its own split count (num_splits 0 or
 * plan->num_splits, ATTN_EINVAL otherwise).  Precondition for such a plan:
 * each device context_lens[b] <= host_context_lens[b] (a shorter one leaves
 * some of its splits empty; keys past n_b * split_chunk would be ignored).
 */
attn_status attn_decode_plan_lens(const attn_decode_desc* desc, const int32_t* host_context_lens,
                                  int32_t num_splits, int32_t flags, attn_decode_plan_t* plan);

/*
 * Full decode: stage 1 (partials into the workspace) then stage 2 (merge into
 * out and, when lse is non-null, lse), both enqueued on `stream`.  With one
 * split, stage 1 writes out and lse itself (the same bits a merge of one
 * split gives) and the workspace is not touched (its size is not checked).
 * num_splits = 0 uses plan->num_splits; any value in [1, plan->max_splits]
 * is allowed (results agree up to float rounding).  workspace_bytes must be
 * at least the size attn_decode_workspace_layout reports for that split
 * count.  With ATTN_PLAN_FUSED_MERGE and 2 <= S <= 64 the merge runs inside
 * the stage-1 launch (same results up to float rounding; the workspace must
 * have been through attn_decode_workspace_init); other split counts take the
 * two launches.  scale multiplies q.k before the softmax; it must be positive and
 * finite (with scale * log2(e) finite too), else ATTN_EINVAL.
 */
attn_status attn_decode_run(const attn_decode_plan_t* plan, const void* q,
                            const void* k_cache, const void* v_cache,
                            const int32_t* page_table, const int32_t* context_lens,
                            float scale, int32_t num_splits, void* out, float* lse,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* Stage 1 only: writes o_part / lse_part of every split into the workspace
 * (an empty split writes zeros and -inf; with a split table, request b's
 * slots n_b .. S - 1 are left untouched).  Same arguments as run. */
attn_status attn_decode_partials(const attn_decode_plan_t* plan, const void* q,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* page_table, const int32_t* context_lens,
                                 float scale, int32_t num_splits, void* workspace,
                                 int64_t workspace_bytes, void* stream);

/* Stage 2 only: log-sum-exp merge of the num_splits partials held in the
 * workspace (layout above) into out (plan dtype) and optional lse. */
attn_status attn_decode_merge(const attn_decode_plan_t* plan, int32_t num_splits,
                              const void* workspace, int64_t workspace_bytes,
                              void* out, float* lse, void* stream);

/* Byte offsets of o_part and lse_part inside the workspace and the total
 * bytes needed for num_splits splits (0 = plan->num_splits). */
attn_status attn_decode_workspace_layout(const attn_decode_plan_t* plan, int32_t num_splits,
                                         int64_t* o_part_offset, int64_t* lse_part_offset,
                                         int64_t* bytes);

/*
 * Makes a workspace ready for runs of this plan: with ATTN_PLAN_FUSED_MERGE,
 * enqueues on `stream` one small kernel that zeroes the row-group counters
 * at the start of the workspace (no memset, so it may be captured); for
 * other plans it does nothing.  Call it once after allocating a workspace
 * (or after using it with another plan): every fused run finds the counters
 * zero and leaves them zero.  A fused run on counters that are not zero
 * writes a wrong output without any error, and two runs that share a
 * workspace must not overlap in time (the same holds for the partials).
 * ATTN_EINVAL for a null or misaligned workspace, ATTN_EWORKSPACE if it is
 * smaller than the counters.
 */
attn_status attn_decode_workspace_init(const attn_decode_plan_t* plan, void* workspace,
                                       int64_t workspace_bytes, void* stream);

/* The split rule: [*begin, *end) of split `split` of `num_splits` (0 = the
 * plan's) for a request with context_len keys.  Pure host function. */
attn_status attn_decode_split_range(const attn_decode_plan_t* plan, int32_t context_len,
                                    int32_t num_splits, int32_t split, int32_t* begin,
                                    int32_t* end);

/*
 * Shared-prefix plans.  aiter PR #4758's MLA workload (Test Plan, workload
 * paragraph) has groups of 8 consecutive requests that share a 63,240-token
 * prefix (the same page ids); its kernel leaves the sharing to the L2
 * (Technical Details item 2: the programs of one split on one XCD).  A
 * caller that knows the groups can instead have the shared keys scored once
 * for all of a group's query rows.  Splits of a request's keys merged by the
 * log-sum-exp reduction give the unsplit result (Motivation; Technical
 * Details item 3), so splitting each row's keys into the shared ones and its
 * own changes nothing but float rounding:
 *   - the shared pass treats group g (requests gG .. gG + G - 1) as one
 *     request of G * q_len query rows (its members' rows, which follow one
 *     another in q and out) over keys [0, prefix_len), read through member
 *     gG's page-table row, in shared.num_splits splits by the split rule;
 *   - the own pass runs every request over keys [prefix_len, ctx[b]), in
 *     own.num_splits splits by the split rule applied to ctx[b] - prefix_len;
 *   - one stage-2 merge over both sets: row r's split slots are the shared
 *     pass's splits 0 .. shared.num_splits - 1, then the own pass's.
 * The workspace holds num_splits = shared.num_splits + own.num_splits slots
 * per row: o_part fp32 [B, q_len, H_q, num_splits, Dv] at offset 0, then
 * lse_part fp32 [B, q_len, H_q, num_splits] at the next multiple of 256
 * bytes; workspace_bytes is its size (rounded up to 256).  shared is unused
 * (all zero) when prefix_len is 0.
 */
#define ATTN_SHARED_PASS_MIN_ROWS 128

typedef struct attn_decode_prefix_plan_t {
  attn_decode_plan_t shared;  /* the groups' shared keys (virtual batch B / G, q_len G * q_len) */
  attn_decode_plan_t own;     /* every request's keys past the prefix */
  int32_t prefix_group;       /* G */
  int32_t prefix_len;         /* shared keys per group (0: no shared pass) */
  int32_t num_splits;         /* split slots per row */
  int32_t reserved;
  int64_t workspace_bytes;
  uint64_t key;               /* hash of both plans, G and prefix_len */
} attn_decode_prefix_plan_t;

/*
 * Plan a shared-prefix decode.  prefix_group G >= 1 must divide batch;
 * prefix_len must be a multiple of page_size with prefix_len + q_len - 1 <=
 * max_context_len; flags may hold ATTN_PLAN_NO_XCD_REMAP,
 * ATTN_PLAN_PRIVATE_PAGES and ATTN_PLAN_SHARED_PASS (the own pass is always
 * planned with ATTN_PLAN_PRIVATE_PAGES: its keys are private).
 * ATTN_EINVAL / ATTN_EUNSUPPORTED as attn_decode_plan.
 * Unless ATTN_PLAN_SHARED_PASS is set, the plan falls back to the default
 * plan over all keys where the shared pass did not pay on MI355X.  With R =
 * G * q_len * H_q / H_kv query rows per group and KV head, that is: G = 1;
 * R < 32; a single group (G = batch) with R < 64; and a default plan on the
 * four-key-stream shape (matrix cores, 16-63 query rows per KV head in a
 * batch that may share pages) with R < ATTN_SHARED_PASS_MIN_ROWS.  The
 * default plan's XCD-contiguous order then lets a group's requests share
 * the prefix through one XCD's L2.  The fallback plan has prefix_len and
 * shared zero and own equal to attn_decode_plan(desc, max_context_len, 0,
 * flags); attn_decode_run_prefix runs it with the same bits as
 * attn_decode_run.  Measured: MLA with 16 heads, the shared pass lost in
 * groups of 1, 2 and 4 requests and won from 8 (294 -> 199 us at batch
 * 48); GQA with 8 query heads per KV head lost in groups of 2, and in one
 * group of 4, and won in four groups of 4 and from groups of 8 (89.6 ->
 * 49.6 us at batch 16 in groups of 8).  Preconditions the
 * run cannot check: within a group the page-table rows hold the same page
 * ids in their first prefix_len / page_size entries, and every request has
 * ctx[b] >= prefix_len + q_len - 1 (each of its rows sees the whole prefix).
 * The shared pass reads member gG's first prefix_len / page_size page ids
 * whatever the members' ctx[b]: those entries must be valid page ids, or the
 * kernels read out of bounds; a request shorter than the prefix gets wrong
 * results, not an error.
 */
attn_status attn_decode_plan_prefix(const attn_decode_desc* desc, int32_t max_context_len,
                                    int32_t prefix_group, int32_t prefix_len, int32_t flags,
                                    attn_decode_prefix_plan_t* plan);

/*
 * Run a shared-prefix plan: the shared pass (when prefix_len > 0), the own
 * pass and the merge, enqueued on `stream` in that order.  Arguments as
 * attn_decode_run (always with the plan's split counts); workspace_bytes must
 * be at least plan->workspace_bytes (ATTN_EWORKSPACE otherwise).
 */
attn_status attn_decode_run_prefix(const attn_decode_prefix_plan_t* plan, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* page_table, const int32_t* context_lens,
                                   float scale, void* out, float* lse, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * decode as attn_decode_run (same kernels, same bits), with the workspace
 * taken from a static device array of ATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends, instead of a
 * caller buffer.  The caller still passes inputs and outputs.  No call
 * allocates or frees memory; the first call on a device looks the array's
 * address up (hipGetSymbolAddress) and keeps it, so make that first call
 * outside graph capture.  `stream` must belong to the current device
 * (ATTN_EINVAL otherwise).  ATTN_EWORKSPACE when more than one split is run
 * and the split count's workspace (attn_decode_workspace_layout) exceeds
 * the array (one split writes the output directly and needs none),
 * ATTN_EUNSUPPORTED for plans made with ATTN_PLAN_FUSED_MERGE.  Every call
 * on one GPU shares that GPU's array and leaves its partials there: calls
 * that overlap in time on one GPU (other streams, other threads) race and
 * give wrong outputs.  Nothing in the array needs to start at zero.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((int64_t)64 << 20)
attn_status attn_decode_run_noalloc(const attn_decode_plan_t* plan, const void* q,
                                    const void* k_cache, const void* v_cache,
                                    const int32_t* page_table, const int32_t* context_lens,
                                    float scale, int32_t num_splits, void* out, float* lse,
                                    void* stream);

/* Text of the calling thread's last error ("" if none).  Owned by the library;
 * valid until the thread's next failing call. */
const char* attn_decode_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLITKV_ATTN_DECODE_H */
