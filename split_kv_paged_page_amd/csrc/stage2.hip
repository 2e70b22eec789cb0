// Stage 2 of split-KV paged decode: log-sum-exp merge of the per-split
// partials (aiter PR #4758, "[Gluon][MLA] Deeper async-copy pipeline in the
// bh16 stage-1 decode loop", Technical Details item 3).
//
// One kernel family: LP = 1, 2, ..., 64 lanes per output pair (query row, 4
// dims), one-wave workgroups.  Lane sl holds splits sl, sl + LP, ... (16 at
// a time in registers, every load of a pass issued before the first use),
// forms its own max, weight sum and weighted sum in split order, and the LP
// lanes are combined by a fixed butterfly (DPP quad swaps and row mirrors,
// then the 16- and 32-lane swaps), which leaves the same bits in every lane.
// No LDS and no barriers: a merge of up to 16 * LP splits is one memory
// round trip plus a few cross-lane steps.
//
// LP is the smallest power of two that keeps a lane at 16 splits or fewer
// (8 when there are at most 16), doubled while the merge would have fewer
// than 128 waves.  The split count
// and the output size alone pick it, so one plan always merges in the same
// order (same bits on every run).  Measured on the 64K GQA merge (512 pairs,
// 256 splits): 16 lanes in 128 one-wave workgroups 3.0 us per op; the same
// in 256-thread workgroups 4.2; 8 lanes 3.8; 32 lanes 3.5; 64 lanes 4.7.
// At 8 rather than 16 splits per lane the drafts' merge (up to 16 splits
// per row) takes 2 lanes: whole op 14.64 -> 14.45 us (at 4, 14.84); one
// MLA request's 213 splits at 8 per lane (32 lanes) took 26.7 us per op
// against 24.9 at 16 (16 lanes).
#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr int kPer = 16;        // splits per lane held in registers per pass
constexpr int kFewSplits = 16;  // up to this many splits, a lane takes at most half of them
constexpr int kMinWaves = 128;  // below this, more lanes per pair

template <int LP>
__device__ __forceinline__ float lanes_max(float x) {
  if constexpr (LP >= 2) x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  if constexpr (LP >= 4) x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  if constexpr (LP >= 8) x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  if constexpr (LP >= 16) x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  if constexpr (LP >= 32) x = max_xor16(x);
  if constexpr (LP == 64) x = max_xor32(x);
  return x;
}
template <int LP>
__device__ __forceinline__ float lanes_sum(float x) {
  if constexpr (LP >= 2) x += dpp_f32<kDppQuadSwap1>(x);
  if constexpr (LP >= 4) x += dpp_f32<kDppQuadSwap2>(x);
  if constexpr (LP >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (LP >= 16) x += dpp_f32<kDppRowMirror>(x);
  if constexpr (LP >= 32) x = sum_xor16(x);
  if constexpr (LP == 64) x = sum_xor32(x);
  return x;
}

template <int DTYPE, int LP>
__global__ __launch_bounds__(64) void stage2_kernel(Stage2Params p) {
  // Every argument read in one round at entry (the empty statements only
  // hold the values in scalar registers), instead of a chain of reads after
  // branches on earlier ones.
  asm volatile("" ::"s"(p.rows), "s"(p.num_splits), "s"(p.head_dim_v), "s"(p.live_splits), "s"(p.fd_cols.mul),
               "s"(p.fd_cols.shift), "s"(p.fd_req_rows.mul), "s"(p.fd_req_rows.shift), "s"(p.o_part),
               "s"(p.lse_part), "s"(p.out), "s"(p.lse));
  asm volatile("" ::"s"(p.split_start[0]), "s"(p.split_start[1]), "s"(p.split_start[2]), "s"(p.split_start[3]),
               "s"(p.split_start[4]), "s"(p.split_start[5]), "s"(p.split_start[6]), "s"(p.split_start[7]),
               "s"(p.split_start[8]), "s"(p.split_start[9]), "s"(p.split_start[10]), "s"(p.split_start[11]),
               "s"(p.split_start[12]), "s"(p.split_start[13]), "s"(p.split_start[14]), "s"(p.split_start[15]),
               "s"(p.split_start[16]));
  const int Dv = p.head_dim_v;
  const int cols = Dv / 4;
  const int sl = threadIdx.x & (LP - 1);
  // Output pair of this lane group; rows * cols < 2^31 (host-checked).
  const uint32_t pair = blockIdx.x * (64 / LP) + threadIdx.x / LP;
  const uint32_t rq = fdiv(pair, p.fd_cols);
  if ((int)rq >= p.rows) return;   // the LP lanes of a pair leave together
  const int64_t row = rq;
  const int c = (int)(pair - rq * cols);
  const int SS = p.num_splits;   // slots per row
  // Splits this row merges: all slots, or under a split table its
  // request's count (the later slots are not written).
  int S = SS;
  if (p.live_splits > 0) {
    const int b = (int)fdiv(rq, p.fd_req_rows);
    S = table_entry(p.split_start, b + 1) - table_entry(p.split_start, b);
  }
  const float* lse_row = p.lse_part + row * SS;
  const float* base = p.o_part + row * SS * Dv + c * 4;

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
void launch_lp(const Stage2Params& p, int64_t pairs, hipStream_t st) {
  constexpr int per_wg = 64 / LP;
  hipLaunchKernelGGL((stage2_kernel<DTYPE, LP>), dim3((unsigned)((pairs + per_wg - 1) / per_wg)), dim3(64), 0,
                     st, p);
}

template <int DTYPE>
void launch(const Stage2Params& p, int64_t pairs, int lp, hipStream_t st) {
  switch (lp) {
    case 1: launch_lp<DTYPE, 1>(p, pairs, st); break;
    case 2: launch_lp<DTYPE, 2>(p, pairs, st); break;
    case 4: launch_lp<DTYPE, 4>(p, pairs, st); break;
    case 8: launch_lp<DTYPE, 8>(p, pairs, st); break;
    case 16: launch_lp<DTYPE, 16>(p, pairs, st); break;
    case 32: launch_lp<DTYPE, 32>(p, pairs, st); break;
    default: launch_lp<DTYPE, 64>(p, pairs, st); break;
  }
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_u32(uint32_t* p, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

int stage2_lanes(int64_t pairs, int num_splits) {
  int lp = 1;
  const int per = num_splits <= kFewSplits ? kPer / 2 : kPer;
  while (lp < 64 && (int64_t)lp * per < num_splits) lp *= 2;
  while (lp < 64 && pairs * lp < (int64_t)kMinWaves * 64) lp *= 2;
  return lp;
}

bool stage2_supported(int dtype, int dv) {
  return (dtype == 0 || dtype == 1) && dv > 0 && dv % 4 == 0;
}

hipError_t launch_stage2(const Stage2Params& p, int dtype, hipStream_t st) {
  const int64_t pairs = (int64_t)p.rows * (p.head_dim_v / 4);
  const int lp = stage2_lanes(pairs, p.num_splits);
  if (dtype == 0)
    launch<0>(p, pairs, lp, st);
  else
    launch<1>(p, pairs, lp, st);
  return hipGetLastError();
}

}  // namespace splitkv
