// Device helpers for the gfx950 kernels: wave64 cross-lane reductions through
// DPP, bf16 packing, the split rule and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"
#include "launch.h"

namespace splitkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));


constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;

// DPP controls (GFX9 encoding).
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowNewBcast0 = 0x150;  // row_newbcast:n = 0x150 + n (gfx90a and later)

// Every DPP pattern used here reads a valid lane for every lane, so the
// "old" operand is never observed: mov_dpp leaves it undefined and saves the
// zero-initialising move update_dpp would need.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int x) {
  return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}

// Value of lane N of this lane's 16-lane row, for every lane of the row.
template <int N>
__device__ __forceinline__ float row_bcast_f32(float x) {
  return dpp_f32<kDppRowNewBcast0 + N>(x);
}
template <int N>
__device__ __forceinline__ int row_bcast_i32(int x) {
  return dpp_i32<kDppRowNewBcast0 + N>(x);
}

// Max / sum over the 16 lanes of a DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<kDppQuadSwap1>(x);
  x += dpp_f32<kDppQuadSwap2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  x += dpp_f32<kDppRowMirror>(x);
  return x;
}

// Max / sum of x over lanes l and l ^ 16 (l ^ 32) with the gfx950 lane
// swaps, no LDS round trip.  v_permlane16_swap a, b (a = b = x on entry)
// leaves a = x[l], b = x[l+16] on even 16-lane rows and a = x[l-16], b = x[l]
// on odd rows; v_permlane32_swap does the same across the two 32-lane
// halves.  Both lanes of a pair see both values (max and a two-term sum are
// symmetric, so the pair gets the same bits).  Written as assembly: the
// compiler's builtin folds max(a, b) / a + b of the pair as if a == b.  The
// s_nop covers the wait states a VALU write needs before a permlane reads it.
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float max_xor16(float x) {
  float a = x, b = x;
  swap16(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float max_xor32(float x) {
  float a = x, b = x;
  swap32(a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_xor16(float x) {
  float a = x, b = x;
  swap16(a, b);
  return a + b;
}
__device__ __forceinline__ float sum_xor32(float x) {
  float a = x, b = x;
  swap32(a, b);
  return a + b;
}

// fp32 -> bf16, nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// 2^x; exact at 0, 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land
// at lds + 16 * i (the LDS base is wave-uniform; it goes through M0).
__device__ __forceinline__ void lds_dma16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (GFX9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | (((N >> 4) & 3) << 14));
}

// Four consecutive outputs in the output dtype (0: fp32, 1: bf16 nearest-even).
__device__ __forceinline__ void store_out4(void* out, int dtype, int64_t off, float4 o) {
  if (dtype == 0) {
    *(float4*)((float*)out + off) = o;
  } else {
    uint2 pk;
    pk.x = pack_bf16x2(o.x, o.y);
    pk.y = pack_bf16x2(o.z, o.w);
    *(uint2*)((uint16_t*)out + off) = pk;
  }
}

// Split rule: split s of S over ctx keys, chunk = A * ceil(ceil(ctx / S) / A),
// or the plan's fixed split length when fixed_chunk > 0.
__device__ __forceinline__ void split_range(int ctx, int S, FastDiv fd_S, int align_shift, int fixed_chunk, int s,
                                            int& beg, int& end) {
  const int per = (int)fdiv((uint32_t)(ctx + S - 1), fd_S);
  int chunk = ((per + (1 << align_shift) - 1) >> align_shift) << align_shift;
  if (chunk <= 0) chunk = 1 << align_shift;
  if (fixed_chunk > 0) chunk = fixed_chunk;
  long long b = (long long)s * chunk;
  long long e = b + chunk;
  beg = (int)(b < ctx ? b : ctx);
  end = (int)(e < ctx ? e : ctx);
}

// Workgroup id -> (head tile, KV head, request, split), fastest first.
struct WgCoord {
  int tile, kvh, b, s;
};
__device__ __forceinline__ WgCoord wg_coord(uint32_t lid, FastDiv fd_tiles, int tiles, FastDiv fd_kvh, int kvhs,
                                            FastDiv fd_batch, int batch) {
  const uint32_t q1 = fdiv(lid, fd_tiles), q2 = fdiv(q1, fd_kvh), q3 = fdiv(q2, fd_batch);
  return WgCoord{(int)(lid - q1 * tiles), (int)(q1 - q2 * kvhs), (int)(q2 - q3 * batch), (int)q3};
}

// Causal plans: the head tile is the slowest index instead, so the tiles
// with the latest query positions (the most keys) of every request and KV
// head are dispatched before any shorter tile.  With the tile fastest, each
// run of `tiles` workgroups went from longest to shortest for one request
// and KV head, and the long tiles of the later requests started only when
// the first round of workgroups drained, leaving a long tail.
__device__ __forceinline__ WgCoord wg_coord_tiles_last(uint32_t lid, FastDiv fd_kvh, int kvhs, FastDiv fd_batch,
                                                       int batch, FastDiv fd_splits, int splits) {
  const uint32_t q1 = fdiv(lid, fd_kvh), q2 = fdiv(q1, fd_batch), q3 = fdiv(q2, fd_splits);
  return WgCoord{(int)q3, (int)(lid - q1 * kvhs), (int)(q1 - q2 * batch), (int)(q2 - q3 * splits)};
}

// Split-table lookups.  The table sits in the kernel arguments; its first
// entries are read at constant offsets (loaded together with the other
// arguments, no dependent load per step) and only batches beyond them scan
// further.  Request of work item f: the number of requests past the first
// whose items start at or before f (a request with no item is skipped).
constexpr int kTableFast = 16;
__device__ __forceinline__ int table_request(const int32_t* start, int batch, int f) {
  int b = 0;
#pragma unroll
  for (int i = 1; i <= kTableFast; ++i) b += (i < batch && f >= start[i]) ? 1 : 0;
  for (int i = kTableFast + 1; i < batch; ++i) b += f >= start[i] ? 1 : 0;
  return b;
}
// start[b] for a b that may differ across lanes.
__device__ __forceinline__ int table_entry(const int32_t* start, int b) {
  int v = 0;
#pragma unroll
  for (int i = 0; i <= kTableFast; ++i) v = b == i ? start[i] : v;
  return b > kTableFast ? start[b] : v;
}

// The stage-1 arguments a workgroup reads before its first memory request
// (coordinates, split bounds, page-table and context pointers, the split
// table's first entries), all in the
// parameters' first lines, read at kernel entry in one round: left alone,
// the compiler reads each argument where it is first used, after branches
// on earlier ones, and the reads become a chain of dependent round trips
// (workgroup coordinates known 0.72 us after entry, 0.32 us with the
// arguments reordered by first use).  The empty statement only holds the
// values in scalar registers at this point.
__device__ __forceinline__ void read_stage1_start_args(const Stage1Params& p) {
  // One statement, so that every read is issued before the first wait.
  asm volatile("" ::"s"(p.xcd_remap), "s"(p.num_wgs), "s"(p.causal), "s"(p.live_splits), "s"(p.batch),
               "s"(p.num_kv_heads), "s"(p.head_tiles), "s"(p.num_splits), "s"(p.fd_tiles.mul),
               "s"(p.fd_tiles.shift), "s"(p.fd_kvh.mul), "s"(p.fd_kvh.shift), "s"(p.fd_batch.mul),
               "s"(p.fd_batch.shift), "s"(p.fd_splits.mul), "s"(p.fd_splits.shift), "s"(p.fd_live.mul),
               "s"(p.fd_live.shift), "s"(p.fd_group.mul), "s"(p.fd_group.shift), "s"(p.split_chunk),
               "s"(p.align_shift), "s"(p.guess_ctx), "s"(p.rows_total), "s"(p.q_len), "s"(p.page_shift),
               "s"(p.max_pages), "s"(p.page_table), "s"(p.ctx), "s"(p.key_base), "s"(p.fixed_ctx));
  // The split table's first entries (the lookup's fast path).
  asm volatile("" ::"s"(p.split_start[0]), "s"(p.split_start[1]), "s"(p.split_start[2]), "s"(p.split_start[3]),
               "s"(p.split_start[4]), "s"(p.split_start[5]), "s"(p.split_start[6]), "s"(p.split_start[7]),
               "s"(p.split_start[8]), "s"(p.split_start[9]), "s"(p.split_start[10]), "s"(p.split_start[11]),
               "s"(p.split_start[12]), "s"(p.split_start[13]), "s"(p.split_start[14]), "s"(p.split_start[15]),
               "s"(p.split_start[16]));
}

// Keys of request b this launch covers (see Stage1Params::key_base).
__device__ __forceinline__ int launch_ctx(const Stage1Params& p, int b) {
  if (p.fixed_ctx > 0) return p.fixed_ctx;
  const int L = p.ctx[b] - p.key_base;
  return L > 0 ? L : 0;
}

// Workspace slot of split s of query row `row`.
__device__ __forceinline__ int64_t part_slot(const Stage1Params& p, int64_t row, int s) {
  return row * p.slot_stride + p.slot_base + s;
}

// Stage-1 workgroup -> (head tile, KV head, request, split).  Without a
// split table, lid enumerates (tile, KV head, request, split) fastest first
// (causal plans: the tile slowest).  With one, the (request, split) pairs of
// the plan's work list take the place of (request, split): item f belongs to
// the request b with split_start[b] <= f < split_start[b+1], as its split
// f - split_start[b].  The table sits in the kernel arguments, so the scan
// reads no device memory.
__device__ __forceinline__ WgCoord stage1_coord(const Stage1Params& p, uint32_t lid) {
  if (p.live_splits <= 0)
    return p.causal ? wg_coord_tiles_last(lid, p.fd_kvh, p.num_kv_heads, p.fd_batch, p.batch, p.fd_splits,
                                          p.num_splits)
                    : wg_coord(lid, p.fd_tiles, p.head_tiles, p.fd_kvh, p.num_kv_heads, p.fd_batch, p.batch);
  const FastDiv one{1u, 0u};   // division by 1
  WgCoord c = p.causal ? wg_coord_tiles_last(lid, p.fd_kvh, p.num_kv_heads, one, 1, p.fd_live, p.live_splits)
                       : wg_coord(lid, p.fd_tiles, p.head_tiles, p.fd_kvh, p.num_kv_heads, one, 1);
  const int f = c.s;
  const int b = table_request(p.split_start, p.batch, f);
  c.b = b;
  c.s = f - table_entry(p.split_start, b);
  return c;
}

// Workgroup order.  The dispatcher hands workgroup p to XCD p % 8; with the
// remap on, XCD x receives one contiguous range of the logical (split-major)
// order, so all requests' programs for one split land on one XCD's L2.  The
// mapping is a bijection for any n (the first n % 8 XCDs take one extra).
__device__ __forceinline__ int logical_wg(int p, int n, int remap) {
  if (!remap) return p;
  int q = n / kNumXcd, r = n % kNumXcd;
  int x = p % kNumXcd, k = p / kNumXcd;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

}  // namespace splitkv
