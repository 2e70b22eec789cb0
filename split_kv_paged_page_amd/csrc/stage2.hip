// Stage 2 of split-KV paged decode: log-sum-exp merge of the per-split
// partials (aiter PR #4758, "[Gluon][MLA] Deeper async-copy pipeline in the
// bh16 stage-1 decode loop", Technical Details item 3).
//
// Two kernels, chosen by the split count alone, so a given S always merges
// in the same order (same bits for every tiling and launch shape):
//
// * S <= kRowSplits (many rows, few splits: MLA batches, wide GQA): one
//   thread per (query row, 4 dims) walks the splits in order; no LDS, no
//   barrier, every load issued up front.
// * larger S (batch-1 decode): one workgroup per (query row, Dv slice).  With
//   few query rows the host cuts the head dim into up to 8 slices so more
//   CUs work; each slice re-derives the row's max and weight sum on its own,
//   so slices never talk to each other.  256 threads = SL split lanes x
//   (256 / SL) four-float columns, SL = the largest power of two <= min(S,
//   16); split lane sl sums splits sl, sl + SL, ... and the lanes are then
//   added in lane order.  Every summation order depends on the split count
//   only, never on the slicing.  The partial-output loads are issued before
//   the weights are known, so the merge costs one memory round trip.
#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;
constexpr int kMaxSplitsLds = 4096;
constexpr int kChunk = 16;                  // splits per split lane held in registers

// LDS-only workgroup barrier: wait for this wave's LDS traffic, then meet.
// Global loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
  __builtin_amdgcn_s_barrier();
}

template <int DTYPE>
__global__ __launch_bounds__(kThreads) void stage2_kernel(Stage2Params p) {
  __shared__ float w_lds[kMaxSplitsLds];
  __shared__ float red[kThreads / 64];
  __shared__ __align__(16) float4 part[kThreads];

  const int row = blockIdx.x / p.tiles;
  const int tile = blockIdx.x % p.tiles;
  const int S = p.num_splits;
  const int Dv = p.head_dim_v;
  const int dvt = Dv / p.tiles;  // slice width, a multiple of 4
  const int cols = dvt / 4;      // float4 columns in the slice
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int kSL = 1;
  while (kSL < 16 && kSL * 2 <= S) kSL *= 2;
  const int kColSlots = kThreads / kSL;
  const int cs = tid % kColSlots, sl = tid / kColSlots;

  const float* lse_row = p.lse_part + (int64_t)row * S;
  const float* base = p.o_part + (int64_t)row * S * Dv + tile * dvt;

  float4 ov[kChunk];
  auto load_chunk = [&](int c0, int s0) {
    const int col = c0 + cs;
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const int s = s0 + sl + k * kSL;
      ov[k] = (col < cols && s < S) ? *(const float4*)(base + (int64_t)s * Dv + col * 4)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  load_chunk(0, 0);

  // Row max of the split log-sum-exps.
  float mx = kNegInf;
  for (int s = tid; s < S; s += kThreads) mx = fmaxf(mx, lse_row[s]);
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  if (lane == 0) red[wave] = mx;
  lds_barrier();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red[w]);
  lds_barrier();

  // Weights exp(lse_s - M) into LDS; their sum by a fixed-order tree.
  float dl = 0.f;
  for (int s = tid; s < S; s += kThreads) {
    const float wgt = M == kNegInf ? 0.f : fast_exp2((lse_row[s] - M) * kLog2e);
    w_lds[s] = wgt;
    dl += wgt;
  }
  for (int o = 32; o > 0; o >>= 1) dl += __shfl_xor(dl, o);
  if (lane == 0) red[wave] = dl;
  lds_barrier();
  float den = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) den += red[w];

  for (int c0 = 0; c0 < cols; c0 += kColSlots) {
    const int col = c0 + cs;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < S; s0 += kSL * kChunk) {
      if (c0 != 0 || s0 != 0) load_chunk(c0, s0);
#pragma unroll
      for (int k = 0; k < kChunk; ++k) {
        const int s = s0 + sl + k * kSL;
        const float wgt = s < S ? w_lds[s] : 0.f;
        a.x = fmaf(wgt, ov[k].x, a.x);
        a.y = fmaf(wgt, ov[k].y, a.y);
        a.z = fmaf(wgt, ov[k].z, a.z);
        a.w = fmaf(wgt, ov[k].w, a.w);
      }
    }
    part[tid] = a;
    lds_barrier();
    if (sl == 0 && col < cols) {
      float4 t = part[cs];
      for (int k = 1; k < kSL; ++k) {
        const float4 u = part[k * kColSlots + cs];
        t.x += u.x; t.y += u.y; t.z += u.z; t.w += u.w;
      }
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (M != kNegInf) {
        const float inv = 1.f / den;
        o = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
      }
      store_out4(p.out, DTYPE, (int64_t)row * Dv + tile * dvt + col * 4, o);
    }
    lds_barrier();
  }
  if (p.lse && tile == 0 && tid == 0) p.lse[row] = M == kNegInf ? kNegInf : M + __logf(den);
}

constexpr int kRowSplits = 16;

template <int DTYPE>
__global__ __launch_bounds__(kThreads) void stage2_rows_kernel(Stage2Params p) {
  const int Dv = p.head_dim_v;
  const int cols = Dv / 4;
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;   // rows * cols < 2^31 (host-checked)
  const uint32_t rq = fdiv(idx, p.fd_cols);
  if ((int)rq >= p.rows) return;
  const int64_t row = rq;
  const int c = (int)(idx - rq * cols);
  const int S = p.num_splits;
  const float* lse_row = p.lse_part + row * S;
  const float* base = p.o_part + row * S * Dv + c * 4;
  float4 ov[kRowSplits];
  float ls[kRowSplits];
#pragma unroll
  for (int s = 0; s < kRowSplits; ++s) {
    if (s < S) {
      ov[s] = *(const float4*)(base + (int64_t)s * Dv);
      ls[s] = lse_row[s];
    }
  }
  float M = kNegInf;
#pragma unroll
  for (int s = 0; s < kRowSplits; ++s)
    if (s < S) M = fmaxf(M, ls[s]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float den = 0.f;
  if (M != kNegInf) {
    float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < kRowSplits; ++s) {
      if (s < S) {
        const float wgt = fast_exp2((ls[s] - M) * kLog2e);
        den += wgt;
        t.x = fmaf(wgt, ov[s].x, t.x);
        t.y = fmaf(wgt, ov[s].y, t.y);
        t.z = fmaf(wgt, ov[s].z, t.z);
        t.w = fmaf(wgt, ov[s].w, t.w);
      }
    }
    const float inv = 1.f / den;
    o = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
  }
  store_out4(p.out, DTYPE, row * Dv + c * 4, o);
  if (p.lse && c == 0) p.lse[row] = M == kNegInf ? kNegInf : M + __logf(den);
}

}  // namespace

bool stage2_supported(int dtype, int dv, int tiles) {
  if (dtype != 0 && dtype != 1) return false;
  if (tiles < 1 || dv % tiles) return false;
  const int dvt = dv / tiles;
  return dvt % 4 == 0;
}

hipError_t launch_stage2(const Stage2Params& p, int dtype, hipStream_t st) {
  if (p.num_splits > kMaxSplitsLds) return hipErrorInvalidValue;
  if (p.num_splits <= kRowSplits) {
    const int64_t threads = (int64_t)p.rows * (p.head_dim_v / 4);
    const dim3 grid((unsigned)((threads + kThreads - 1) / kThreads));
    if (dtype == 0)
      hipLaunchKernelGGL(stage2_rows_kernel<0>, grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL(stage2_rows_kernel<1>, grid, dim3(kThreads), 0, st, p);
    return hipGetLastError();
  }
  const dim3 grid(p.rows * p.tiles);
  if (dtype == 0)
    hipLaunchKernelGGL(stage2_kernel<0>, grid, dim3(kThreads), 0, st, p);
  else
    hipLaunchKernelGGL(stage2_kernel<1>, grid, dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace splitkv
