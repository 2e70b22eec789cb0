// Stage 2 of split-KV paged decode: log-sum-exp merge of the per-split
// partials (aiter PR #4758, "[Gluon][MLA] Deeper async-copy pipeline in the
// bh16 stage-1 decode loop", Technical Details item 3).
//
// Two kernels, chosen by the split count alone, so a given S always merges
// in the same order:
//
// * S <= kRowSplits (many rows, few splits: MLA batches, wide GQA): one
//   thread per (query row, 4 dims) walks the splits in order; every load is
//   issued up front.
// * larger S (batch-1 decode): one 16-lane DPP row per (query row, 4 dims).
//   Lane sl holds splits sl, sl + 16, ... (16 at a time in registers, all
//   loads issued before the first use), forms its own max, weight sum and
//   weighted sum in split order, and the 16 lanes are combined by a fixed
//   butterfly (quad swaps, half-row and row mirrors), which leaves the same
//   bits in every lane.  No LDS and no barriers: the merge is one memory
//   round trip plus a few cross-lane steps.
#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kThreads = 256;
constexpr int kLanes = 16;   // split lanes per (row, 4 dims): one DPP row
constexpr int kPer = 16;     // splits per lane held in registers at a time

template <int DTYPE>
__global__ __launch_bounds__(kThreads) void stage2_lanes_kernel(Stage2Params p) {
  const int Dv = p.head_dim_v;
  const int cols = Dv / 4;
  const int sl = threadIdx.x & (kLanes - 1);
  // (row, column) pair of this DPP row; rows * cols < 2^31 (host-checked).
  const uint32_t pair = blockIdx.x * (kThreads / kLanes) + threadIdx.x / kLanes;
  const uint32_t rq = fdiv(pair, p.fd_cols);
  if ((int)rq >= p.rows) return;   // the 16 lanes of a pair leave together
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
      const int s = s0 + sl + k * kLanes;
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
  for (int s = kLanes * kPer + sl; s < S; s += kLanes) M = fmaxf(M, lse_row[s]);
  M = row16_max(M);

  float den = 0.f;
  float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
  if (M != kNegInf) {   // uniform over the pair's 16 lanes
    for (int s0 = 0; s0 < S; s0 += kLanes * kPer) {
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
  den = row16_sum(den);
  t.x = row16_sum(t.x);
  t.y = row16_sum(t.y);
  t.z = row16_sum(t.z);
  t.w = row16_sum(t.w);
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
  } else {
    constexpr int per_wg = kThreads / kLanes;
    const dim3 grid((unsigned)((pairs + per_wg - 1) / per_wg));
    if (dtype == 0)
      hipLaunchKernelGGL(stage2_lanes_kernel<0>, grid, dim3(kThreads), 0, st, p);
    else
      hipLaunchKernelGGL(stage2_lanes_kernel<1>, grid, dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace splitkv
