// Internal launch parameters shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_decode.h"
#include "fastdiv.h"

namespace splitkv {

// Field order follows first use: a workgroup's start reads the first three
// 64-byte lines (its coordinates, split bounds and page-table pointer), so
// the argument reads that precede its first memory request touch few lines.
struct Stage1Params {
  // ---- workgroup coordinates ----
  int32_t xcd_remap;
  int32_t num_wgs;        // stage-1 workgroups
  int32_t causal;
  int32_t live_splits;    // > 0: the split table below enumerates the work
  int32_t batch, num_kv_heads, head_tiles, num_splits;
  // Divisors of the workgroup-id decomposition, the split rule and the row
  // index (see fastdiv.h).
  FastDiv fd_tiles, fd_kvh, fd_batch, fd_splits;
  FastDiv fd_live, fd_group;
  // ---- split bounds, rows, page walk ----
  int32_t split_chunk;    // > 0: every split is this many keys long (else the split-count rule)
  int32_t align_shift;    // split_align = 1 << align_shift
  int32_t guess_ctx;      // > 0: likely context length (early page-table reads)
  int32_t rows_total;     // query rows per KV head = group * q_len
  int32_t q_len, group, num_q_heads, rows_per_wg;
  int32_t page_shift;     // log2(page_size)
  int32_t page_size, max_pages, split_align;
  const int32_t* page_table;
  const int32_t* ctx;
  // A launch may cover part of each request's keys (shared-prefix plans):
  // request b's keys here are ctx[b] - key_base, from key_base on (the
  // page-table pointer already points past the first key_base / page_size
  // entries), or fixed_ctx > 0 keys for every request.
  int32_t key_base, fixed_ctx;
  // Split table (live_splits > 0): request b owns work items
  // [split_start[b], split_start[b+1]).
  int32_t split_start[ATTN_MAX_SPLIT_TABLE + 1];
  float scale_log2;       // scale * log2(e): scores are kept in base-2 units
  const void* q;
  const void* k;
  const void* v;
  int64_t ks_page, ks_head, ks_tok;   // elements
  int64_t vs_page, vs_head, vs_tok;
  float* o_part;          // [B, q_len, Hq, slot_stride, Dv]
  float* lse_part;        // [B, q_len, Hq, slot_stride]
  int32_t slot_stride;    // split slots per row in the workspace (num_splits unless the plan has several launches)
  int32_t slot_base;      // this launch's split s goes to slot slot_base + s
  // Single split: write the final output (q dtype) and log-sum-exp directly
  // instead of partials (identical bits to merging one split).
  void* out;              // null: write partials
  float* lse_out;         // optional with out
  // In-kernel merge (matrix-core kernel, 2 <= num_splits <= kFusedMaxSplits):
  // non-null counters, one per (request, KV head, head tile), zero on entry
  // and left zero, make the workgroup that writes a row group's last split
  // merge the group's partials into fin_out (bf16) and fin_lse (optional).
  uint32_t* counters;
  void* fin_out;
  float* fin_lse;
};

constexpr int kFusedMaxSplits = 64;   // one split per lane in the merge's weight pass

struct Stage2Params {
  int32_t rows;           // B * q_len * Hq
  int32_t num_splits;
  int32_t head_dim_v;
  int32_t live_splits;    // > 0: row r of request b = r / (q_len * Hq) merges
                          // split_start[b+1] - split_start[b] slots only
  FastDiv fd_cols;        // head_dim_v / 4 (output pair -> row, column)
  FastDiv fd_req_rows;
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse;             // may be null
  int32_t split_start[ATTN_MAX_SPLIT_TABLE + 1];
};

// Zeroes n 32-bit words with a small fill kernel (no memset node in a graph).
hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t s);

// Stage-1 launchers; return false when no kernel exists for the shape.
bool stage1_valu_supported(int dtype, int dk, int dv, int rows_per_wg);
hipError_t launch_stage1_valu(const Stage1Params& p, int dtype, int dk, int dv, hipStream_t s);

// Matrix-core workgroup shape: rw 16-row tiles x kw key streams and its LDS
// bytes ({0, 0, 0}: no matrix-core kernel for this dtype and head dims).
struct MfmaShape {
  int rw, kw, smem;
};
// streams = false: no key-stream shape (kw > 1); the ring shapes serve the rows.
MfmaShape stage1_mfma_shape(int dtype, int dk, int dv, bool v_aliases_k, int rows, bool streams = true);
hipError_t launch_stage1_mfma(const Stage1Params& p, int dk, int dv, bool v_aliases_k, MfmaShape shape,
                              hipStream_t s);

bool stage2_supported(int dtype, int dv);
// Lanes per output pair (query row, 4 dims) the merge uses.
int stage2_lanes(int64_t pairs, int num_splits);
hipError_t launch_stage2(const Stage2Params& p, int dtype, hipStream_t s);

}  // namespace splitkv
