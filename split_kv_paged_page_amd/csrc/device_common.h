// Device helpers for the gfx950 kernels: wave64 cross-lane reductions through
// DPP, bf16 packing, the split rule and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastdiv.h"

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

// Split rule: split s of S over ctx keys, chunk = A * ceil(ceil(ctx / S) / A).
__device__ __forceinline__ void split_range(int ctx, int S, FastDiv fd_S, int align_shift, int s, int& beg,
                                            int& end) {
  const int per = (int)fdiv((uint32_t)(ctx + S - 1), fd_S);
  int chunk = ((per + (1 << align_shift) - 1) >> align_shift) << align_shift;
  if (chunk <= 0) chunk = 1 << align_shift;
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
