// Host side of libsplitkv: descriptor checks, the split policy, workspace
// layout, and the stage-1 / stage-2 launches on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn_decode.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";

attn_status fail(attn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

attn_status hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int kSplitAlign = 64;   // split granule in keys (the VALU kernel's block; two matrix-core blocks)
constexpr int kNumCu = 256;       // MI355X compute units
constexpr int kLdsPerCu = 160 * 1024;
constexpr int kMaxSplits = 4096;  // far above any useful split count; bounds the workspace

uint64_t fnv1a(const void* p, size_t n, uint64_t h = 1469598103934665603ull) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  for (size_t i = 0; i < n; ++i) {
    h ^= c[i];
    h *= 1099511628211ull;
  }
  return h;
}

int elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

attn_status check_desc(const attn_decode_desc* d) {
  if (!d) return fail(ATTN_EINVAL, "desc is null");
  if (d->batch < 1 || d->q_len < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1)
    return fail(ATTN_EINVAL, "batch, q_len and head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads)
    return fail(ATTN_EINVAL, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", d->num_q_heads,
                d->num_kv_heads);
  if (d->head_dim_qk < 1 || d->head_dim_v < 1 || d->page_size < 1 || d->max_pages_per_req < 1 ||
      d->num_pages < 1)
    return fail(ATTN_EINVAL, "head dims, page size, max_pages_per_req and num_pages must be >= 1");
  if (d->dtype != ATTN_F32 && d->dtype != ATTN_BF16) return fail(ATTN_EINVAL, "unknown dtype %d", d->dtype);
  if (d->page_size & (d->page_size - 1))
    return fail(ATTN_EUNSUPPORTED, "page_size %d is not a power of two", d->page_size);
  // Kernels divide context lengths and row indices as 31-bit values.
  if ((int64_t)d->max_pages_per_req * d->page_size > (int64_t(1) << 30))
    return fail(ATTN_EINVAL, "max_pages_per_req * page_size exceeds 2^30 keys");
  if ((int64_t)d->batch * d->q_len * d->num_q_heads * ((d->head_dim_v + 3) / 4) >= (int64_t(1) << 31))
    return fail(ATTN_EINVAL, "batch * q_len * num_q_heads * head_dim_v / 4 must stay below 2^31");
  if (d->causal != 0 && d->causal != 1) return fail(ATTN_EINVAL, "causal must be 0 or 1");
  if (d->v_aliases_k != 0 && d->v_aliases_k != 1) return fail(ATTN_EINVAL, "v_aliases_k must be 0 or 1");
  if (d->reserved != 0) return fail(ATTN_EINVAL, "reserved must be 0");
  if (d->v_aliases_k && d->head_dim_v > d->head_dim_qk)
    return fail(ATTN_EINVAL, "aliased V needs head_dim_v <= head_dim_qk");
  const int64_t es = elem_bytes(d->dtype);
  const int64_t ks[3] = {d->k_stride_page, d->k_stride_head, d->k_stride_tok};
  const int64_t vs[3] = {d->v_stride_page, d->v_stride_head, d->v_stride_tok};
  for (int i = 0; i < 3; ++i) {
    if (ks[i] < 0 || vs[i] < 0) return fail(ATTN_EINVAL, "strides must be >= 0");
    // Rows are read in 16-byte pieces (rocm-libraries PR #10102, Technical
    // Details: 16-byte reads need a 16-byte-aligned pitch), so every row
    // start must be 16-byte aligned.
    if ((ks[i] * es) % 16 || (vs[i] * es) % 16)
      return fail(ATTN_EUNSUPPORTED, "KV strides must be multiples of 16 bytes");
  }
  if (d->v_aliases_k && (vs[0] != ks[0] || vs[1] != ks[1] || vs[2] != ks[2]))
    return fail(ATTN_EINVAL, "aliased V must use the K strides");
  if (d->k_stride_tok < d->head_dim_qk || d->v_stride_tok < d->head_dim_v)
    return fail(ATTN_EINVAL, "token stride is shorter than the head dim");
  // Kernels address a row as a 32-bit count of 16-byte units from the head's
  // base (pools up to 64 GiB).
  const int64_t kmax = ((d->num_pages - 1) * ks[0] + (int64_t)(d->page_size - 1) * ks[2]) * es / 16;
  const int64_t vmax = ((d->num_pages - 1) * vs[0] + (int64_t)(d->page_size - 1) * vs[2]) * es / 16;
  if (kmax >= (int64_t(1) << 32) || vmax >= (int64_t(1) << 32))
    return fail(ATTN_EUNSUPPORTED, "KV pool spans more than 64 GiB");
  return ATTN_OK;
}

int pick_rows_per_wg(int dtype, int dk, int dv, int rows) {
  for (int rt : {4, 8, 16})
    if (rt >= rows && splitkv::stage1_valu_supported(dtype, dk, dv, rt)) return rt;
  int best = 0;
  for (int rt : {4, 8, 16})
    if (splitkv::stage1_valu_supported(dtype, dk, dv, rt)) best = rt;
  return best;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Row groups of the in-kernel merge: one counter per (request, KV head,
// head tile), i.e. per set of stage-1 workgroups that differ only in split.
int64_t counter_count(const attn_decode_plan_t* p) {
  if (!(p->flags & ATTN_PLAN_FUSED_MERGE)) return 0;
  return (int64_t)p->desc.batch * p->desc.num_kv_heads * p->head_tiles;
}

// [counters (fused plans)] [o_part] [lse_part], each 256-byte aligned; the
// counters come first so that their place does not depend on S.
void layout(const attn_decode_plan_t* p, int S, int64_t* o_off, int64_t* l_off, int64_t* bytes) {
  const attn_decode_desc& d = p->desc;
  const int64_t rows = (int64_t)d.batch * d.q_len * d.num_q_heads;
  const int64_t cb = align256(counter_count(p) * 4);
  const int64_t ob = align256(rows * S * d.head_dim_v * 4);
  if (o_off) *o_off = cb;
  if (l_off) *l_off = cb + ob;
  if (bytes) *bytes = cb + ob + align256(rows * S * 4);
}

attn_status resolve_splits(const attn_decode_plan_t* p, int32_t num_splits, int* S) {
  if (!p) return fail(ATTN_EINVAL, "plan is null");
  if (num_splits < 0) return fail(ATTN_EINVAL, "num_splits must be >= 0");
  *S = num_splits ? num_splits : p->num_splits;
  if (*S > p->max_splits)
    return fail(ATTN_EWORKSPACE, "num_splits %d exceeds the plan's max_splits %d", *S, p->max_splits);
  // With a fixed split length the plan's split count is the one that covers
  // its longest request; fewer would leave keys out.
  if (p->split_chunk > 0 && *S != p->num_splits)
    return fail(ATTN_EINVAL, "a plan with %d-key splits runs with its own %d splits (got %d)", p->split_chunk,
                p->num_splits, *S);
  return ATTN_OK;
}

// One stage-1 launch of a shared-prefix plan: which keys of each request it
// covers and where its splits go in the workspace.
struct PassOpts {
  int key_base = 0;      // first key (the page-table pointer moves by key_base / page_size entries)
  int fixed_ctx = 0;     // > 0: every (virtual) request has this many keys
  int slot_stride = 0;   // split slots per row in the workspace
  int slot_base = 0;     // first slot of this launch
  int pt_row_mult = 1;   // page-table rows per (virtual) request
};

attn_status enqueue_stage1(const attn_decode_plan_t* plan, int S, const void* q, const void* k,
                           const void* v, const int32_t* pt, const int32_t* ctx, float scale,
                           void* ws, int64_t ws_bytes, hipStream_t st, void* out = nullptr,
                           float* lse_out = nullptr, void* fin_out = nullptr, float* fin_lse = nullptr,
                           const PassOpts* po = nullptr) {
  const attn_decode_desc& d = plan->desc;
  if (!q || !k || !v || !pt || !ctx || !ws) return fail(ATTN_EINVAL, "a device pointer is null");
  if (d.v_aliases_k && v != k) return fail(ATTN_EINVAL, "aliased V: v_cache must equal k_cache");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v) % 16 || (uintptr_t)ws % 256)
    return fail(ATTN_EINVAL, "q/k/v must be 16-byte aligned and the workspace 256-byte aligned");
  // The kernels keep raw dot products and apply scale * log2(e) to the
  // block maximum and inside the weights' FMA, which needs a positive,
  // finite factor (a negative one would turn the maximum into a minimum,
  // zero would turn masked scores into NaN).
  const float scale_log2 = scale * 1.4426950408889634f;
  if (!(scale > 0.f) || !(scale_log2 <= 3.4028234663852886e38f))
    return fail(ATTN_EINVAL, "scale must be positive and finite (got %g)", (double)scale);
  const int slots = po ? po->slot_stride : S;
  int64_t o_off, l_off, need;
  layout(plan, slots, &o_off, &l_off, &need);
  // Direct output (one split) leaves the workspace untouched.
  if (!out && ws_bytes < need)
    return fail(ATTN_EWORKSPACE, "workspace of %lld bytes is below the %lld needed", (long long)ws_bytes,
                (long long)need);
  splitkv::Stage1Params p{};
  p.out = out;
  p.lse_out = lse_out;
  if (fin_out) {   // in-kernel merge: counters at the workspace's start
    p.counters = (uint32_t*)ws;
    p.fin_out = fin_out;
    p.fin_lse = fin_lse;
  }
  p.q = q;
  p.k = k;
  p.v = v;
  p.page_table = po ? pt + po->key_base / d.page_size : pt;
  p.ctx = ctx;
  p.key_base = po ? po->key_base : 0;
  p.fixed_ctx = po ? po->fixed_ctx : 0;
  p.o_part = (float*)((char*)ws + o_off);
  p.lse_part = (float*)((char*)ws + l_off);
  p.slot_stride = slots;
  p.slot_base = po ? po->slot_base : 0;
  p.scale_log2 = scale_log2;
  p.batch = d.batch;
  p.q_len = d.q_len;
  p.num_q_heads = d.num_q_heads;
  p.num_kv_heads = d.num_kv_heads;
  p.group = d.num_q_heads / d.num_kv_heads;
  p.page_size = d.page_size;
  p.page_shift = 0;
  while ((1 << p.page_shift) < d.page_size) ++p.page_shift;
  p.max_pages = d.max_pages_per_req * (po ? po->pt_row_mult : 1);
  p.causal = d.causal;
  p.num_splits = S;
  p.split_align = plan->split_align;
  p.split_chunk = plan->split_chunk;
  p.live_splits = plan->live_splits;
  for (int i = 0; i <= ATTN_MAX_SPLIT_TABLE; ++i) p.split_start[i] = plan->split_start[i];
  p.fd_live = splitkv::make_fastdiv((uint32_t)(plan->live_splits > 0 ? plan->live_splits : 1));
  p.align_shift = 0;
  while ((1 << p.align_shift) < p.split_align) ++p.align_shift;
  p.fd_tiles = splitkv::make_fastdiv((uint32_t)plan->head_tiles);
  p.fd_kvh = splitkv::make_fastdiv((uint32_t)d.num_kv_heads);
  p.fd_batch = splitkv::make_fastdiv((uint32_t)d.batch);
  p.fd_splits = splitkv::make_fastdiv((uint32_t)S);
  p.fd_group = splitkv::make_fastdiv((uint32_t)(d.num_q_heads / d.num_kv_heads));
  p.rows_total = p.group * d.q_len;
  // One request: its context is most likely the longest the plan was made
  // for.  Batches mix lengths, and a wrong guess costs more than it saves,
  // except under a split table: there a workgroup knows its split's start
  // without the context length, and its end whenever the split is not its
  // request's last (the kernels then guess min((s + 1) * chunk, max)).
  p.guess_ctx = d.batch == 1 || plan->live_splits > 0 ? plan->max_context_len : 0;
  p.rows_per_wg = plan->rows_per_wg;
  p.head_tiles = plan->head_tiles;
  p.xcd_remap = plan->xcd_remap;
  const int64_t nwg = (int64_t)(plan->live_splits > 0 ? plan->live_splits : (int64_t)S * d.batch) *
                     d.num_kv_heads * plan->head_tiles;
  if (nwg > 0x7fffffff) return fail(ATTN_EINVAL, "grid too large");
  p.num_wgs = (int32_t)nwg;
  p.ks_page = d.k_stride_page;
  p.ks_head = d.k_stride_head;
  p.ks_tok = d.k_stride_tok;
  p.vs_page = d.v_stride_page;
  p.vs_head = d.v_stride_head;
  p.vs_tok = d.v_stride_tok;
  const int rw = plan->rows_per_wg / 16;
  hipError_t e = plan->variant == ATTN_VARIANT_MFMA
                     ? splitkv::launch_stage1_mfma(p, d.head_dim_qk, d.head_dim_v, d.v_aliases_k != 0,
                                                   splitkv::MfmaShape{rw, plan->stage1_waves / rw}, st)
                     : splitkv::launch_stage1_valu(p, d.dtype, d.head_dim_qk, d.head_dim_v, st);
  if (e != hipSuccess) return hip_fail(e, "stage-1 launch");
  return ATTN_OK;
}

attn_status enqueue_stage2(const attn_decode_plan_t* plan, int S, const void* ws, int64_t ws_bytes,
                           void* out, float* lse, hipStream_t st) {
  const attn_decode_desc& d = plan->desc;
  if (!ws || !out) return fail(ATTN_EINVAL, "workspace or out is null");
  if ((uintptr_t)out % 16 || (uintptr_t)ws % 256 || (uintptr_t)lse % 4)
    return fail(ATTN_EINVAL, "out must be 16-byte aligned and the workspace 256-byte aligned");
  int64_t o_off, l_off, need;
  layout(plan, S, &o_off, &l_off, &need);
  if (ws_bytes < need)
    return fail(ATTN_EWORKSPACE, "workspace of %lld bytes is below the %lld needed", (long long)ws_bytes,
                (long long)need);
  splitkv::Stage2Params p{};
  p.o_part = (const float*)((const char*)ws + o_off);
  p.lse_part = (const float*)((const char*)ws + l_off);
  p.out = out;
  p.lse = lse;
  p.rows = d.batch * d.q_len * d.num_q_heads;
  p.num_splits = S;
  p.head_dim_v = d.head_dim_v;
  p.fd_cols = splitkv::make_fastdiv((uint32_t)(d.head_dim_v / 4));
  p.live_splits = plan->live_splits;
  for (int i = 0; i <= ATTN_MAX_SPLIT_TABLE; ++i) p.split_start[i] = plan->split_start[i];
  p.fd_req_rows = splitkv::make_fastdiv((uint32_t)(d.q_len * d.num_q_heads));
  hipError_t e = splitkv::launch_stage2(p, d.dtype, st);
  if (e != hipSuccess) return hip_fail(e, "stage-2 launch");
  return ATTN_OK;
}

// ---- Static scratch of the no-allocation entry point ----
// attn_decode_run_noalloc keeps a call's workspace (the partials of every
// split) in this device array instead of a caller buffer.  Every GPU the
// library runs on holds its own copy from the code object's load until the
// process ends.  In host code `scratch` names a host-side stand-in, never
// the device memory: kernels get the address hipGetSymbolAddress returns
// for the current device, looked up once per device and kept below.
constexpr int64_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Address of this device's scratch; `stream` must belong to the current
// device (the array's address differs from one device to the next).
attn_status device_scratch(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (stream) {
    hipDevice_t sdev = 0;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(ATTN_EINVAL, "the stream belongs to device %d but device %d is current", (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_EUNSUPPORTED, "device %d is beyond the %d devices the static scratch serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || (uintptr_t)p % 256) return fail(ATTN_EHIP, "static scratch is not 256-byte aligned");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_decode_last_error(void) { return g_err; }

}  // extern "C"

namespace {

// The key covers every field a kernel launch depends on (rocm-libraries
// PR #10102, Technical Details: a cache keyed on the kernel name alone
// missed the batch baked into the binary).
uint64_t plan_key(const attn_decode_plan_t& p) {
  uint64_t h = fnv1a(&p.desc, sizeof(p.desc));
  const int32_t fields[] = {p.max_context_len, p.num_splits, p.max_splits, p.split_align, p.variant,
                            p.rows_per_wg,     p.head_tiles, p.stage1_waves, p.xcd_remap, p.flags,
                            p.split_chunk, p.live_splits};
  h = fnv1a(fields, sizeof(fields), h);
  return fnv1a(p.split_start, sizeof(p.split_start), h);
}

// The planner behind attn_decode_plan and attn_decode_plan_lens; `lens`
// (batch entries, host memory) may be null.
attn_status plan_impl(const attn_decode_desc* desc, int32_t max_context_len, const int32_t* lens,
                      int32_t num_splits, int32_t flags, attn_decode_plan_t* plan) {
  if (!plan) return fail(ATTN_EINVAL, "plan is null");
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  if (max_context_len < 0) return fail(ATTN_EINVAL, "max_context_len must be >= 0");
  if ((int64_t)max_context_len > (int64_t)desc->max_pages_per_req * desc->page_size)
    return fail(ATTN_EINVAL, "max_context_len %d exceeds max_pages_per_req * page_size", max_context_len);
  if (num_splits < 0 || num_splits > kMaxSplits)
    return fail(ATTN_EINVAL, "num_splits must be in [0, %d]", kMaxSplits);
  if (flags & ~(ATTN_PLAN_POLICY_P2 | ATTN_PLAN_NO_XCD_REMAP | ATTN_PLAN_FUSED_MERGE | ATTN_PLAN_PRIVATE_PAGES))
    return fail(ATTN_EINVAL, "unknown plan flags 0x%x", flags);

  const attn_decode_desc& d = *desc;
  const int rows = (d.num_q_heads / d.num_kv_heads) * d.q_len;
  attn_decode_plan_t p{};
  p.desc = d;
  p.max_context_len = max_context_len;
  p.split_align = kSplitAlign;
  p.flags = flags;
  // XCD-contiguous order (each XCD one contiguous range of the split-major
  // order) keeps the programs that share KV on one XCD's L2 (aiter PR #4758,
  // Technical Details item 2, which applies it when batch > 1).  MLA batch
  // 48 with 8-request shared prefixes, stage 1 (us, A/B/B/A in one run):
  // contiguous 294.0 / 294.2, plain 573.8 / 572.7; L2 hit rate 78.6% against
  // 0.4%, L2 fetch 807 MB per launch against 3.77 GB.  With one request no
  // KV is shared and the order is neutral (64K GQA 16.14 / 15.85 against
  // 15.92 / 15.89), so batch 1 keeps the plain order as the PR does.  With
  // several query positions per request (causal drafts, prefill) a
  // request's work grows with its length, and whole requests per XCD leave
  // XCDs idle when the lengths differ; the plain order spreads every request
  // over all XCDs.  Measured (us per op, contiguous / plain): varlen prefill
  // 131 / 86 (head dim 64) and 197 / 124 (128); equal-length prefill 105 /
  // 118 and 151 / 180; drafts 19.3 / 18.6.  The plan does not see the
  // lengths, so q_len > 1 takes the plain order.
  p.xcd_remap = (flags & ATTN_PLAN_NO_XCD_REMAP) || d.q_len > 1 || d.batch == 1 ? 0 : 1;
  // bf16 runs on the matrix cores at every group size (a 16-row tile part
  // empty still costs a fraction of the vector-ALU work per key); fp32 runs
  // on the vector ALUs.  One request, or a batch whose requests share no
  // page (the caller's hint), takes a ring shape where a batch would take key
  // streams (16-63 rows): the streams' four waves compute four blocks at once
  // but load each block only when its wave is free, which pays when requests
  // re-read shared prefix pages from the L2.
  const bool streams = d.batch > 1 && !(flags & ATTN_PLAN_PRIVATE_PAGES);
  const splitkv::MfmaShape ms =
      splitkv::stage1_mfma_shape(d.dtype, d.head_dim_qk, d.head_dim_v, d.v_aliases_k != 0, rows, streams);
  int wgs_per_cu = 2;
  if (ms.rw > 0) {
    p.variant = ATTN_VARIANT_MFMA;
    p.rows_per_wg = 16 * ms.rw;
    p.stage1_waves = ms.rw * ms.kw;
    // Workgroups per CU: two where the LDS allows, else one; the one-wave
    // ring (1-15 rows per KV head) depends on the batch.
    //   * One request, or private pages (the hint): at head dim 128 one per
    //     CU, whose two 16 KB blocks in flight walk twice the keys at the
    //     same rate with half the partials to merge (64K GQA whole op
    //     18.73 -> 18.25 us, batch 4 / 8 52.3 -> 51.7 / 99.3 -> 98.0); at
    //     head dim 64 (8 KB blocks) two, one being far slower (stage 1 9.96
    //     -> 12.0 us).
    //   * A batch whose requests may share pages: two at head dim 128 and
    //     four at 64.  Once the L2 serves the shared blocks, each wave's own
    //     per-block work bounds the batch, and more waves per CU share it.
    //     61,440 of 65,536 keys shared (us per op): head dim 128, one / two
    //     per CU, batch 4 in one group 45.8 / 29.5, 8 in one group 84.6 /
    //     49.2, 16 in groups of 8 161.3 / 89.9; head dim 64, two / four,
    //     23.2 / 19.2, 39.3 / 28.6, 71.7 / 49.1.  On private pages planned
    //     without the hint the same choice costs at most 2%: head dim 128
    //     batch 2 / 4 / 8 30.4 / 51.3 / 97.4 against 30.1 / 51.7 / 99.4;
    //     head dim 64 18.2 / 29.9 / 52.0 against 18.5 / 30.0 / 52.1.
    const bool lone = ms.rw == 1 && ms.kw == 1;
    const bool may_share = d.batch > 1 && !(flags & ATTN_PLAN_PRIVATE_PAGES);
    if (lone && d.head_dim_qk == 128)
      wgs_per_cu = may_share ? 2 : 1;
    else if (lone && d.head_dim_qk == 64 && may_share)
      wgs_per_cu = 4;
    else
      wgs_per_cu = kLdsPerCu / ms.smem < 2 ? 1 : 2;
  } else {
    const int rt = pick_rows_per_wg(d.dtype, d.head_dim_qk, d.head_dim_v, rows);
    if (!rt)
      return fail(ATTN_EUNSUPPORTED, "no stage-1 kernel for dtype %d, head dims %d/%d", d.dtype, d.head_dim_qk,
                  d.head_dim_v);
    p.variant = ATTN_VARIANT_VALU;
    p.rows_per_wg = rt;
    p.stage1_waves = 4;
  }
  p.head_tiles = (rows + p.rows_per_wg - 1) / p.rows_per_wg;
  if ((flags & ATTN_PLAN_FUSED_MERGE) && p.variant != ATTN_VARIANT_MFMA)
    return fail(ATTN_EUNSUPPORTED, "the in-kernel merge needs the matrix-core stage 1 (bf16)");

  // Split count.  The aiter PR's launcher gives each request about 256 /
  // batch splits so that the 256 CUs stay busy (Motivation; Test Result
  // table 1).  The default counts every stage-1 workgroup a split creates
  // (KV heads and head tiles too) and never makes a split shorter than one
  // 64-key block.
  const int blocks = (max_context_len + kSplitAlign - 1) / kSplitAlign;
  int S;
  if (num_splits > 0) {
    S = num_splits;
  } else if (flags & ATTN_PLAN_POLICY_P2) {
    S = kNumCu / d.batch;
    if (S < 1) S = 1;
  } else {
    // One full round of workgroups at the workgroups per CU chosen above
    // (two where the LDS allows, one or two for the lone wave at head dim
    // 128 and two or four at 64).  Three lone waves per CU at head dim 128
    // were slower still for one request (64K GQA stage 1: 16.3 us against
    // 15.7 at two, 15.3 at one).
    const int per_split = d.batch * d.num_kv_heads * p.head_tiles;
    const int target = wgs_per_cu * kNumCu;
    S = target / per_split;
    if (S > blocks) S = blocks;
    if (S < 1) S = 1;
    // Drop the trailing splits that would hold no key even for the longest
    // context (the split rule rounds chunks up to 64 keys): they cost partial
    // writes and merge reads and change no chunk.  Drafts (longest 2,048 keys,
    // 10 -> 8 splits): 16.6 -> 16.3 us per op.
    int64_t chunk_u = kSplitAlign;   // the longest split walk under the split-count rule
    if (max_context_len > 0) {
      const int64_t per = (max_context_len + (int64_t)S - 1) / S;
      chunk_u = (per + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
      S = (int)((max_context_len + chunk_u - 1) / chunk_u);
    }
    // Known lengths (attn_decode_plan_lens): one split length for every
    // request, so that each request holds splits in proportion to its
    // length and every workgroup walks about the same number of keys.  The
    // shortest multiple of 64 keys whose live workgroups still fit one
    // round is taken when it shortens the longest walk of the rule above,
    // which gives every request the same split count.  Drafts (lengths 256
    // to 2,048): 64-key splits would need 384 workgroups; 128-key splits
    // need 192 and walk 128 keys where the split-count rule walks 256.
    // The work list holds one stage-1 workgroup per (request, split), so
    // no workgroup is launched for a split without keys (with one split
    // count for all, the short requests' empty splits each held a CU while
    // they wrote their zero partials, and delayed the long requests' late
    // splits).
    if (lens && max_context_len > 0 && d.batch <= ATTN_MAX_SPLIT_TABLE && !(flags & ATTN_PLAN_FUSED_MERGE)) {
      const int64_t per_req = (int64_t)d.num_kv_heads * p.head_tiles;
      for (int64_t c = kSplitAlign; c < chunk_u; c += kSplitAlign) {
        int64_t live = 0;
        for (int b = 0; b < d.batch; ++b) live += (lens[b] + c - 1) / c;
        if (live * per_req <= target && (max_context_len + c - 1) / c <= kMaxSplits) {
          p.split_chunk = (int32_t)c;
          S = (int)((max_context_len + c - 1) / c);
          int32_t at = 0;
          for (int b = 0; b < d.batch; ++b) {
            p.split_start[b] = at;
            at += (int32_t)((lens[b] + c - 1) / c);
          }
          p.split_start[d.batch] = at;
          p.live_splits = at;
          break;
        }
      }
    }
  }
  if (S > kMaxSplits) S = kMaxSplits;
  p.num_splits = S;
  p.max_splits = S;
  if (!splitkv::stage2_supported(d.dtype, d.head_dim_v))
    return fail(ATTN_EUNSUPPORTED, "no stage-2 kernel for head_dim_v %d", d.head_dim_v);
  int64_t bytes;
  layout(&p, p.max_splits, nullptr, nullptr, &bytes);
  p.workspace_bytes = bytes;
  p.key = plan_key(p);
  *plan = p;
  g_err[0] = 0;
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_decode_plan(const attn_decode_desc* desc, int32_t max_context_len, int32_t num_splits,
                             int32_t flags, attn_decode_plan_t* plan) {
  return plan_impl(desc, max_context_len, nullptr, num_splits, flags, plan);
}

attn_status attn_decode_plan_lens(const attn_decode_desc* desc, const int32_t* host_context_lens,
                                  int32_t num_splits, int32_t flags, attn_decode_plan_t* plan) {
  if (!desc) return fail(ATTN_EINVAL, "desc is null");
  if (!host_context_lens) return fail(ATTN_EINVAL, "host_context_lens is null");
  if (desc->batch < 1) return fail(ATTN_EINVAL, "batch, q_len and head counts must be >= 1");
  int32_t mx = 0;
  for (int b = 0; b < desc->batch; ++b) {
    if (host_context_lens[b] < 0) return fail(ATTN_EINVAL, "host_context_lens[%d] is negative", b);
    if (host_context_lens[b] > mx) mx = host_context_lens[b];
  }
  return plan_impl(desc, mx, host_context_lens, num_splits, flags, plan);
}

attn_status attn_decode_workspace_layout(const attn_decode_plan_t* plan, int32_t num_splits,
                                         int64_t* o_part_offset, int64_t* lse_part_offset, int64_t* bytes) {
  int S;
  attn_status st = resolve_splits(plan, num_splits, &S);
  if (st != ATTN_OK) return st;
  layout(plan, S, o_part_offset, lse_part_offset, bytes);
  return ATTN_OK;
}

attn_status attn_decode_workspace_init(const attn_decode_plan_t* plan, void* workspace, int64_t workspace_bytes,
                                       void* stream) {
  if (!plan) return fail(ATTN_EINVAL, "plan is null");
  const int64_t n = counter_count(plan);
  if (n == 0) return ATTN_OK;
  if (!workspace || (uintptr_t)workspace % 256) return fail(ATTN_EINVAL, "workspace must be 256-byte aligned");
  if (workspace_bytes < n * 4)
    return fail(ATTN_EWORKSPACE, "workspace of %lld bytes is below the %lld counter bytes", (long long)workspace_bytes,
                (long long)(n * 4));
  hipError_t e = splitkv::launch_zero_u32((uint32_t*)workspace, n, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "counter fill launch");
  return ATTN_OK;
}

attn_status attn_decode_split_range(const attn_decode_plan_t* plan, int32_t context_len, int32_t num_splits,
                                    int32_t split, int32_t* begin, int32_t* end) {
  if (!begin || !end) return fail(ATTN_EINVAL, "begin/end is null");
  if (!plan) return fail(ATTN_EINVAL, "plan is null");
  if (num_splits < 0) return fail(ATTN_EINVAL, "num_splits must be >= 0");
  const int S = num_splits ? num_splits : plan->num_splits;
  if (context_len < 0) return fail(ATTN_EINVAL, "context_len must be >= 0");
  if (split < 0 || split >= S) return fail(ATTN_EINVAL, "split %d outside [0, %d)", split, S);
  if (plan->split_chunk > 0 && S != plan->num_splits)
    return fail(ATTN_EINVAL, "a plan with %d-key splits has %d splits (got %d)", plan->split_chunk,
                plan->num_splits, S);
  const int64_t A = plan->split_align;
  const int64_t per = (context_len + (int64_t)S - 1) / S;
  int64_t chunk = (per + A - 1) / A * A;
  if (chunk <= 0) chunk = A;
  if (plan->split_chunk > 0) chunk = plan->split_chunk;
  const int64_t b = (int64_t)split * chunk, e = b + chunk;
  *begin = (int32_t)(b < context_len ? b : context_len);
  *end = (int32_t)(e < context_len ? e : context_len);
  return ATTN_OK;
}

attn_status attn_decode_partials(const attn_decode_plan_t* plan, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* page_table, const int32_t* context_lens,
                                 float scale, int32_t num_splits, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  int S;
  attn_status st = resolve_splits(plan, num_splits, &S);
  if (st != ATTN_OK) return st;
  return enqueue_stage1(plan, S, q, k_cache, v_cache, page_table, context_lens, scale, workspace,
                        workspace_bytes, (hipStream_t)stream);
}

attn_status attn_decode_merge(const attn_decode_plan_t* plan, int32_t num_splits, const void* workspace,
                              int64_t workspace_bytes, void* out, float* lse, void* stream) {
  int S;
  attn_status st = resolve_splits(plan, num_splits, &S);
  if (st != ATTN_OK) return st;
  return enqueue_stage2(plan, S, workspace, workspace_bytes, out, lse, (hipStream_t)stream);
}

attn_status attn_decode_run(const attn_decode_plan_t* plan, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* page_table, const int32_t* context_lens,
                            float scale, int32_t num_splits, void* out, float* lse, void* workspace,
                            int64_t workspace_bytes, void* stream) {
  int S;
  attn_status st = resolve_splits(plan, num_splits, &S);
  if (st != ATTN_OK) return st;
  if (!out) return fail(ATTN_EINVAL, "out is null");
  if ((uintptr_t)out % 16 || (uintptr_t)lse % 4) return fail(ATTN_EINVAL, "out must be 16-byte aligned");
  if (S == 1)  // one split: stage 1 writes the final output itself
    return enqueue_stage1(plan, S, q, k_cache, v_cache, page_table, context_lens, scale, workspace,
                          workspace_bytes, (hipStream_t)stream, out, lse);
  if ((plan->flags & ATTN_PLAN_FUSED_MERGE) && S <= splitkv::kFusedMaxSplits)
    return enqueue_stage1(plan, S, q, k_cache, v_cache, page_table, context_lens, scale, workspace,
                          workspace_bytes, (hipStream_t)stream, nullptr, nullptr, out, lse);
  st = enqueue_stage1(plan, S, q, k_cache, v_cache, page_table, context_lens, scale, workspace,
                      workspace_bytes, (hipStream_t)stream);
  if (st != ATTN_OK) return st;
  return enqueue_stage2(plan, S, workspace, workspace_bytes, out, lse, (hipStream_t)stream);
}

attn_status attn_decode_plan_prefix(const attn_decode_desc* desc, int32_t max_context_len, int32_t prefix_group,
                                    int32_t prefix_len, int32_t flags, attn_decode_prefix_plan_t* plan) {
  if (!plan) return fail(ATTN_EINVAL, "plan is null");
  attn_status st = check_desc(desc);
  if (st != ATTN_OK) return st;
  const attn_decode_desc& d = *desc;
  if (prefix_group < 1 || d.batch % prefix_group)
    return fail(ATTN_EINVAL, "prefix_group must be >= 1 and divide batch %d (got %d)", d.batch, prefix_group);
  if ((int64_t)d.max_pages_per_req * prefix_group > 0x7fffffff || (int64_t)d.q_len * prefix_group > 0x7fffffff)
    return fail(ATTN_EINVAL, "prefix_group %d too large for the page-table rows", prefix_group);
  if (prefix_len < 0 || prefix_len % d.page_size)
    return fail(ATTN_EINVAL, "prefix_len must be a non-negative multiple of page_size (got %d)", prefix_len);
  if ((int64_t)prefix_len + d.q_len - 1 > max_context_len)
    return fail(ATTN_EINVAL, "prefix_len + q_len - 1 (%lld) exceeds max_context_len %d",
                (long long)prefix_len + d.q_len - 1, max_context_len);
  if (flags & ~(ATTN_PLAN_NO_XCD_REMAP | ATTN_PLAN_PRIVATE_PAGES | ATTN_PLAN_SHARED_PASS))
    return fail(ATTN_EINVAL, "unknown or unsupported plan flags 0x%x for a shared-prefix plan", flags);
  attn_decode_prefix_plan_t pp{};
  pp.prefix_group = prefix_group;
  // When the shared pass does not pay, the default plan is taken:
  //   * groups of one request: nothing is shared;
  //   * fewer than 32 rows per group and KV head: a shared block then feeds
  //     at most two 16-row tiles' worth of rows, which the default plan's
  //     XCD-contiguous order also serves from one XCD's L2;
  //   * one group, fewer than 64 rows: the shared pass is then a single
  //     virtual request, cut into as many splits as fill the CUs (partials
  //     that weigh as much as the keys) and run in the plain order;
  //   * a default plan on four key streams per 16-row tile (16-63 rows per
  //     KV head in a batch that may share pages), fewer than
  //     ATTN_SHARED_PASS_MIN_ROWS rows: its streams already take a split's
  //     prefix blocks from the L2 four at a time.
  // Measured (us per op, shared-prefix plan / default plan; 61,440 of
  // 65,536 or 63,240 of 68,000 keys shared):
  //   MLA, 16 heads (key streams): groups of 1, 2, 4 requests 36.5 / 25.2,
  //   43.1 / 36.3, 60.3 / 48.7; of 8 at batch 8, 16, 48 61.1 / 73.3,
  //   81.1 / 114.4, 198.6 / 294.0;
  //   GQA, 8 query heads per KV head (one-wave ring, two workgroups per CU):
  //   groups of 2 at batch 2, 8 and 16 24.0 / 20.3, 62.2 / 58.9 and
  //   108.9 / 110.1; of 4 at batch 4, 8 and 16 32.9 / 29.6, 44.6 / 51.4 and
  //   75.8 / 95.3; of 8 at batch 8 and 16 34.8 / 49.0 and 49.6 / 89.6; of 16
  //   at batch 16 51.6 / 89.0.
  if (prefix_len > 0 && !(flags & ATTN_PLAN_SHARED_PASS)) {
    attn_decode_plan_t def{};
    st = plan_impl(&d, max_context_len, nullptr, 0, flags, &def);
    if (st != ATTN_OK) return st;
    const int64_t group_rows = (int64_t)prefix_group * d.q_len * (d.num_q_heads / d.num_kv_heads);
    const bool key_streams = def.variant == ATTN_VARIANT_MFMA && def.stage1_waves * 16 > def.rows_per_wg;
    const bool one_group = prefix_group == d.batch;
    if (prefix_group == 1 || group_rows < 32 || (one_group && group_rows < 64) ||
        (key_streams && group_rows < ATTN_SHARED_PASS_MIN_ROWS)) {
      pp.own = def;
      pp.num_splits = def.num_splits;
      pp.workspace_bytes = def.workspace_bytes;
      const uint64_t parts[] = {def.key, (uint64_t)prefix_group, 0};
      pp.key = fnv1a(parts, sizeof(parts));
      *plan = pp;
      g_err[0] = 0;
      return ATTN_OK;
    }
  }
  pp.prefix_len = prefix_len;
  if (prefix_len > 0) {
    // The groups' shared keys: group g is one request whose q_len * G rows
    // are its members' rows (consecutive in q and out), all of which see
    // every shared key.  Every such request has exactly prefix_len keys, so
    // the XCD-contiguous order suits it whatever q_len is: the head tiles of
    // one (group, split) then read each block on the same XCD.
    attn_decode_desc sd = d;
    sd.batch = d.batch / prefix_group;
    sd.q_len = d.q_len * prefix_group;
    sd.causal = 0;
    st = plan_impl(&sd, prefix_len, nullptr, 0, flags & ATTN_PLAN_NO_XCD_REMAP, &pp.shared);
    if (st != ATTN_OK) return st;
    pp.shared.xcd_remap = (flags & ATTN_PLAN_NO_XCD_REMAP) || sd.batch == 1 ? 0 : 1;
    pp.shared.key = plan_key(pp.shared);
  }
  // Every request's own keys, which no other request reads.
  st = plan_impl(&d, max_context_len - prefix_len, nullptr, 0,
                 (flags & ATTN_PLAN_NO_XCD_REMAP) | ATTN_PLAN_PRIVATE_PAGES, &pp.own);
  if (st != ATTN_OK) return st;
  pp.num_splits = pp.shared.num_splits + pp.own.num_splits;
  int64_t bytes;
  layout(&pp.own, pp.num_splits, nullptr, nullptr, &bytes);
  pp.workspace_bytes = bytes;
  const uint64_t parts[] = {pp.shared.key, pp.own.key, (uint64_t)prefix_group, (uint64_t)prefix_len};
  pp.key = fnv1a(parts, sizeof(parts));
  *plan = pp;
  g_err[0] = 0;
  return ATTN_OK;
}

attn_status attn_decode_run_prefix(const attn_decode_prefix_plan_t* plan, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* page_table, const int32_t* context_lens,
                                   float scale, void* out, float* lse, void* workspace, int64_t workspace_bytes,
                                   void* stream) {
  if (!plan) return fail(ATTN_EINVAL, "plan is null");
  if (!out) return fail(ATTN_EINVAL, "out is null");
  if ((uintptr_t)out % 16 || (uintptr_t)lse % 4) return fail(ATTN_EINVAL, "out must be 16-byte aligned");
  const int S = plan->num_splits, Sp = plan->prefix_len > 0 ? plan->shared.num_splits : 0;
  if (S != Sp + plan->own.num_splits || S < 1) return fail(ATTN_EINVAL, "inconsistent shared-prefix plan");
  hipStream_t st_ = (hipStream_t)stream;
  attn_status st;
  if (Sp > 0) {
    PassOpts po;
    po.fixed_ctx = plan->prefix_len;
    po.slot_stride = S;
    po.pt_row_mult = plan->prefix_group;
    st = enqueue_stage1(&plan->shared, Sp, q, k_cache, v_cache, page_table, context_lens, scale, workspace,
                        workspace_bytes, st_, nullptr, nullptr, nullptr, nullptr, &po);
    if (st != ATTN_OK) return st;
  }
  PassOpts po;
  po.key_base = plan->prefix_len;
  po.slot_stride = S;
  po.slot_base = Sp;
  st = enqueue_stage1(&plan->own, plan->own.num_splits, q, k_cache, v_cache, page_table, context_lens, scale,
                      workspace, workspace_bytes, st_, nullptr, nullptr, nullptr, nullptr, &po);
  if (st != ATTN_OK) return st;
  return enqueue_stage2(&plan->own, S, workspace, workspace_bytes, out, lse, st_);
}

attn_status attn_decode_run_noalloc(const attn_decode_plan_t* plan, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* page_table, const int32_t* context_lens,
                                    float scale, int32_t num_splits, void* out, float* lse, void* stream) {
  int S;
  attn_status st = resolve_splits(plan, num_splits, &S);
  if (st != ATTN_OK) return st;
  if (plan->flags & ATTN_PLAN_FUSED_MERGE)
    return fail(ATTN_EUNSUPPORTED, "the no-allocation call does not take ATTN_PLAN_FUSED_MERGE plans");
  int64_t need;
  layout(plan, S, nullptr, nullptr, &need);
  if (S > 1 && need > kScratchBytes)   // one split writes the output directly, no partials
    return fail(ATTN_EWORKSPACE, "%d splits need a %lld-byte workspace, above the %lld-byte static scratch", S,
                (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  st = device_scratch((hipStream_t)stream, &ws);
  if (st != ATTN_OK) return st;
  return attn_decode_run(plan, q, k_cache, v_cache, page_table, context_lens, scale, S, out, lse, ws,
                         kScratchBytes, stream);
}

}  // extern "C"
