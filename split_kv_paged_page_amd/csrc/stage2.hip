// Stage 2 of split-KV paged decode: log-sum-exp merge of the per-split
// partials (aiter PR #4758, "[Gluon][MLA] Deeper async-copy pipeline in the
// bh16 stage-1 decode loop", Technical Details item 3).
//
// Two kernels; the split count and the output size pick the kernel and its
// lane count, so one plan always merges in the same order (same bits on
// every run):
//
// * S <= kRowSplits (many rows, few splits: MLA batches, wide GQA): one
//   thread per (query row, 4 dims) walks the splits in order; every load is
//   issued up front.
// * larger S (batch-1 decode): LP = 16, 32 or 64 lanes per (query row, 4
//   dims) in one-wave workgroups (16 unless the merge has few rows).  Lane
//   sl holds splits sl, sl + LP, ... (256 / LP at a time in registers, all
//   loads issued before the first use), forms its own max, weight sum and weighted
//   sum in split order, and the LP lanes are combined by a fixed butterfly
//   (DPP quad swaps and row mirrors, then the 16- and 32-lane swaps), which
//   leaves the same bits in every lane.  No LDS and no barriers: the merge
//   is one memory round trip plus a few cross-lane steps.  One-wave
//   workgroups spread the loads over many CUs' memory pipelines.
#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;   // rows kernel

template <int LP>
__device__ __forceinline__ float lanes_max(float x) {
  x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  if constexpr (LP >= 16) x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  if constexpr (LP >= 32) x = max_xor16(x);
  if constexpr (LP == 64) x = max_xor32(x);
  return x;
}
template <int LP>
__device__ __forceinline__ float lanes_sum(float x) {
  x += dpp_f32<kDppQuadSwap1>(x);
  x += dpp_f32<kDppQuadSwap2>(x);
  x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (LP >= 16) x += dpp_f32<kDppRowMirror>(x);
  if constexpr (LP >= 32) x = sum_xor16(x);
  if constexpr (LP == 64) x = sum_xor32(x);
  return x;
}

template <int DTYPE, int LP>
__global__ __launch_bounds__(64) void stage2_lanes_kernel(Stage2Params p) {
  constexpr int kPer = 256 / LP;   // splits per lane held in registers at a time
  const int Dv = p.head_dim_v;
  const int cols = Dv / 4;
  const int sl = threadIdx.x & (LP - 1);
  // (row, column) pair of this lane group; rows * cols < 2^31 (host-checked).
  const uint32_t pair = blockIdx.x * (64 / LP) + threadIdx.x / LP;
  const uint32_t rq = fdiv(pair, p.fd_cols);
  if ((int)rq >= p.rows) return;   // the LP lanes of a pair leave together
  const int64_t row = rq;
  const int c = (int)(pair - rq * cols);
  const int S = p.num_splits;
  const float* lse_row = p.lse_part + row * S;
  const float* base = p.o_part + row * S * Dv + c * 4;

  float ls[kPer];
  float4 ov[kPer];
  auto load = [&](int s0) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int s = s0 + sl + k * LP;
      if (s < S) {
        ls[k] = lse_row[s];
        ov[k] = *(const float4*)(base + (int64_t)s * Dv);
      } else {
        ls[k] = kNegInf;
        ov[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  load(0);
  float M = kNegInf;
#pragma unroll
  for (int k = 0; k < kPer; ++k) M = fmaxf(M, ls[k]);
  for (int s = LP * kPer + sl; s < S; s += LP) M = fmaxf(M, lse_row[s]);
  M = lanes_max<LP>(M);

  float den = 0.f;
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != kNegInf) {   // uniform over the pair's lanes
    for (int s0 = 0; s0 < S; s0 += LP * kPer) {
      if (s0 != 0) load(s0);
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const float wgt = fast_exp2((ls[k] - M) * kLog2e);   // 0 for an empty split or a lane past S
        den += wgt;
        t.x = fmaf(wgt, ov[k].x, t.x);
        t.y = fmaf(wgt, ov[k].y, t.y);
        t.z = fmaf(wgt, ov[k].z, t.z);
        t.w = fmaf(wgt, ov[k].w, t.w);
      }
    }
  }
  den = lanes_sum<LP>(den);
  t.x = lanes_sum<LP>(t.x);
  t.y = lanes_sum<LP>(t.y);
  t.z = lanes_sum<LP>(t.z);
  t.w = lanes_sum<LP>(t.w);
  if (sl == 0) {
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != kNegInf) {
      const float inv = 1.f / den;
      o = make_float4(t.x * inv, t.y * inv, t.z * inv, t.w * inv);
    }
    store_out4(p.out, DTYPE, row * Dv + c * 4, o);
    if (p.lse && c == 0) p.lse[row] = M == kNegInf ? kNegInf : M + __logf(den);
  }
}

template <int DTYPE, int LP>
void launch_lanes_lp(const Stage2Params& p, int64_t pairs, hipStream_t st) {
  constexpr int per_wg = 64 / LP;
  hipLaunchKernelGGL((stage2_lanes_kernel<DTYPE, LP>), dim3((unsigned)((pairs + per_wg - 1) / per_wg)), dim3(64),
                     0, st, p);
}

template <int DTYPE>
void launch_lanes(const Stage2Params& p, int64_t pairs, hipStream_t st) {
  // 16 lanes per pair once that gives 128 or more one-wave workgroups;
  // fewer pairs take more lanes.  Measured on the 64K GQA merge (512 pairs,
  // 256 splits): 16 lanes in 128 one-wave workgroups 3.0 us per op; 16 lanes
  // in 256-thread workgroups 4.2; 8 lanes 3.8; 32 lanes 3.5; 64 lanes 4.7.
  if (pairs >= 512)
    launch_lanes_lp<DTYPE, 16>(p, pairs, st);
  else if (pairs >= 256)
    launch_lanes_lp<DTYPE, 32>(p, pairs, st);
  else
    launch_lanes_lp<DTYPE, 64>(p, pairs, st);
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

bool stage2_supported(int dtype, int dv) {
  return (dtype == 0 || dtype == 1) && dv > 0 && dv % 4 == 0;
}

hipError_t launch_stage2(const Stage2Params& p, int dtype, hipStream_t st) {
  const int64_t pairs = (int64_t)p.rows * (p.head_dim_v / 4);
  if (p.num_splits <= kRowSplits) {
    const dim3 grid((unsigned)((pairs + kThreads - 1) / kThreads));
    if (dtype == 0)
      hipLaunchKernelGGL(stage2_rows_kernel<0>, grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL(stage2_rows_kernel<1>, grid, dim3(kThreads), 0, st, p);
  } else if (dtype == 0) {
    launch_lanes<0>(p, pairs, st);
  } else {
    launch_lanes<1>(p, pairs, st);
  }
  return hipGetLastError();
}

}  // namespace splitkv
