// Internal launch parameters shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

namespace splitkv {

struct Stage1Params {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* page_table;
  const int32_t* ctx;
  float* o_part;          // [B, q_len, Hq, S, Dv]
  float* lse_part;        // [B, q_len, Hq, S]
  float scale_log2;       // scale * log2(e): scores are kept in base-2 units
  int32_t batch, q_len, num_q_heads, num_kv_heads, group;
  int32_t page_size, max_pages, causal;
  int32_t page_shift;     // log2(page_size)
  int32_t num_splits, split_align;
  int32_t rows_total;     // query rows per KV head = group * q_len
  int32_t rows_per_wg, head_tiles;
  int32_t xcd_remap;
  int32_t num_wgs;        // S * B * Hkv * head_tiles
  int64_t ks_page, ks_head, ks_tok;   // elements
  int64_t vs_page, vs_head, vs_tok;
  // Single split: write the final output (q dtype) and log-sum-exp directly
  // instead of partials (identical bits to merging one split).
  void* out;              // null: write partials
  float* lse_out;         // optional with out
  // Divisors of the workgroup-id decomposition, the split rule and the row
  // index (see fastdiv.h); split_align = 1 << align_shift.
  FastDiv fd_tiles, fd_kvh, fd_batch, fd_splits, fd_group;
  int32_t align_shift;
  int32_t guess_ctx;      // > 0: likely context length of every request (early page-table reads)
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
  const float* o_part;
  const float* lse_part;
  void* out;
  float* lse;             // may be null
  int32_t rows;           // B * q_len * Hq
  int32_t num_splits;
  int32_t head_dim_v;
  FastDiv fd_cols;        // head_dim_v / 4 (output pair -> row, column)
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
MfmaShape stage1_mfma_shape(int dtype, int dk, int dv, bool v_aliases_k, int rows);
hipError_t launch_stage1_mfma(const Stage1Params& p, int dk, int dv, bool v_aliases_k, MfmaShape shape,
                              hipStream_t s);

bool stage2_supported(int dtype, int dv);
// Lanes per output pair (query row, 4 dims) the merge uses.
int stage2_lanes(int64_t pairs, int num_splits);
hipError_t launch_stage2(const Stage2Params& p, int dtype, hipStream_t s);

}  // namespace splitkv
