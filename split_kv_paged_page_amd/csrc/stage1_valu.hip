// Stage 1 of split-KV paged decode on the vector ALUs (gfx950, wave64).
//
// One workgroup scores one split of one request's keys against RT query rows
// that share a KV head (aiter PR #4758, "[Gluon][MLA] Deeper async-copy
// pipeline in the bh16 stage-1 decode loop", Motivation: each stage-1
// program walks its split's KV blocks).  Rows per KV head below 16 are too
// few for a dense matrix-core contraction, so this kernel stays on the VALU.
//
// Work split inside a workgroup: NW waves take 64-key blocks of the split in
// turn, each with its own running max / sum / accumulator, merged at the end.
// Inside a wave:
//   * Q.K: lane t owns key t of the block and forms all RT dot products
//     against the query rows held in LDS (every lane reads the same q chunk,
//     an LDS broadcast);
//   * softmax: each 16-lane DPP row keeps its own running max per query row
//     (max over the row by DPP, TensorFold PR #1932's fold-by-DPP approach on
//     wave64's 16-lane rows), so no cross-row traffic happens in the loop;
//   * P.V: the 16 lanes of row g accumulate keys 16g..16g+15 of the block;
//     lane x owns a contiguous slice of the head dim, so every V row is read
//     as one coalesced 256-byte (or wider) segment, and the weight of key i
//     reaches the row's lanes through row_newbcast:i.
#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();

template <int DTYPE, int DK, int DV, int RT, int NW>
__global__ __launch_bounds__(64 * NW) void stage1_valu_kernel(Stage1Params p) {
  constexpr int ES = DTYPE == 0 ? 4 : 2;  // element bytes
  constexpr int KRB = DK * ES;            // bytes of one K row
  constexpr int VRB = DV * ES;            // bytes of one V row
  constexpr int KCH = KRB / 16;           // 16-byte chunks of a K row
  constexpr int VU4 = VRB / 256;          // 16-byte loads per lane per V row
  constexpr int VE = VU4 * 16 / ES;       // V elements a lane owns
  static_assert(VRB % 256 == 0 && KRB % 16 == 0, "row sizes");
  static_assert(RT * VE <= 128, "accumulator budget");

  __shared__ __align__(16) uint8_t q_lds[RT * KRB];
  __shared__ float comb_m[NW][RT];
  __shared__ float comb_l[NW][RT];
  __shared__ __align__(16) float comb_acc[NW][RT][DV];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int x = lane & 15;

  int lid = logical_wg(blockIdx.x, p.num_wgs, p.xcd_remap);
  const int tile = lid % p.head_tiles;
  lid /= p.head_tiles;
  const int kvh = lid % p.num_kv_heads;
  lid /= p.num_kv_heads;
  const int b = lid % p.batch;
  const int s = lid / p.batch;

  const int L = p.ctx[b];
  int sb, se;
  split_range(L, p.num_splits, p.split_align, s, sb, se);

  int row_end[RT];
  int end_max = sb;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int gr = tile * RT + r;
    int e = sb;
    if (gr < p.rows_total) {
      const int j = gr / p.group;
      const int n = p.causal ? L - p.q_len + 1 + j : L;
      e = n < se ? n : se;
      if (e < sb) e = sb;
    }
    row_end[r] = e;
    end_max = e > end_max ? e : end_max;
  }

  // Query rows of this tile into LDS (zeros for rows past the group).
  for (int c = threadIdx.x; c < RT * KCH; c += 64 * NW) {
    const int r = c / KCH, cc = c % KCH;
    const int gr = tile * RT + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (gr < p.rows_total) {
      const int j = gr / p.group, h = kvh * p.group + gr % p.group;
      const uint8_t* src = (const uint8_t*)p.q +
                           ((((int64_t)b * p.q_len + j) * p.num_q_heads + h) * DK) * ES + cc * 16;
      val = *(const uint4*)src;
    }
    *(uint4*)(q_lds + r * KRB + cc * 16) = val;
  }
  __syncthreads();

  float m[RT], l[RT], acc[RT][VE];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[r][e] = 0.f;
  }

  const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)kvh * p.ks_head * ES;
  const uint8_t* vbase = (const uint8_t*)p.v + (int64_t)kvh * p.vs_head * ES + x * (VU4 * 16);
  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int P = p.page_size;

  for (int blk = sb + wave * 64; blk < end_max; blk += NW * 64) {
    const int t = blk + lane;
    const bool tv = t < end_max;
    const int pg_idx = t / P;
    const int page = tv ? pt[pg_idx] : 0;
    const int slot = t - pg_idx * P;

    // ---- Q.K for key t ----
    float sc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) sc[r] = 0.f;
    if (tv) {
      const uint8_t* krow = kbase + ((int64_t)page * p.ks_page + (int64_t)slot * p.ks_tok) * ES;
#pragma unroll 8
      for (int c = 0; c < KCH; ++c) {
        const uint4 kc = *(const uint4*)(krow + c * 16);
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const uint4 qc = *(const uint4*)(q_lds + r * KRB + c * 16);
          if constexpr (DTYPE == 0) {
            sc[r] = fmaf(__builtin_bit_cast(float, qc.x), __builtin_bit_cast(float, kc.x), sc[r]);
            sc[r] = fmaf(__builtin_bit_cast(float, qc.y), __builtin_bit_cast(float, kc.y), sc[r]);
            sc[r] = fmaf(__builtin_bit_cast(float, qc.z), __builtin_bit_cast(float, kc.z), sc[r]);
            sc[r] = fmaf(__builtin_bit_cast(float, qc.w), __builtin_bit_cast(float, kc.w), sc[r]);
          } else {
            sc[r] = dot2_bf16(qc.x, kc.x, sc[r]);
            sc[r] = dot2_bf16(qc.y, kc.y, sc[r]);
            sc[r] = dot2_bf16(qc.z, kc.z, sc[r]);
            sc[r] = dot2_bf16(qc.w, kc.w, sc[r]);
          }
        }
      }
    }

    // ---- online softmax, per 16-lane row ----
    float pr[RT], al[RT];
    bool changed = false;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      sc[r] = t < row_end[r] ? sc[r] * p.scale_log2 : kNegInf;
      const float bm = row16_max(sc[r]);
      const float mn = fmaxf(m[r], bm);
      al[r] = mn == kNegInf ? 1.f : fast_exp2(m[r] - mn);
      changed |= al[r] != 1.f;
      pr[r] = sc[r] == kNegInf ? 0.f : fast_exp2(sc[r] - mn);
      l[r] = l[r] * al[r] + pr[r];
      m[r] = mn;
    }
    if (__any(changed)) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[r][e] *= al[r];
    }

    // ---- P.V: row g accumulates keys blk + 16g + i ----
    const int tg = blk + 16 * g;
    auto pv_step = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const int page_i = row_bcast_i32<i>(page);
      const int slot_i = row_bcast_i32<i>(slot);
      float pw[RT];
#pragma unroll
      for (int r = 0; r < RT; ++r) pw[r] = row_bcast_f32<i>(pr[r]);
      if (tg + i < end_max) {
        const uint8_t* vrow = vbase + ((int64_t)page_i * p.vs_page + (int64_t)slot_i * p.vs_tok) * ES;
#pragma unroll
        for (int u = 0; u < VU4; ++u) {
          const uint4 vv = *(const uint4*)(vrow + u * 16);
          float vf[16 / ES];
          if constexpr (DTYPE == 0) {
            vf[0] = __builtin_bit_cast(float, vv.x);
            vf[1] = __builtin_bit_cast(float, vv.y);
            vf[2] = __builtin_bit_cast(float, vv.z);
            vf[3] = __builtin_bit_cast(float, vv.w);
          } else {
            vf[0] = bf16_lo(vv.x); vf[1] = bf16_hi(vv.x);
            vf[2] = bf16_lo(vv.y); vf[3] = bf16_hi(vv.y);
            vf[4] = bf16_lo(vv.z); vf[5] = bf16_hi(vv.z);
            vf[6] = bf16_lo(vv.w); vf[7] = bf16_hi(vv.w);
          }
#pragma unroll
          for (int r = 0; r < RT; ++r)
#pragma unroll
            for (int e = 0; e < 16 / ES; ++e)
              acc[r][u * (16 / ES) + e] = fmaf(pw[r], vf[e], acc[r][u * (16 / ES) + e]);
        }
      }
    };
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (pv_step(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, 16>{});
  }

  // ---- merge the four 16-lane rows of the wave, then the waves ----
  float mw[RT], lw[RT];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    float lt = row16_sum(l[r]);
    float mx = fmaxf(m[r], __shfl_xor(m[r], 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float f = mx == kNegInf ? 0.f : fast_exp2(m[r] - mx);
    lt *= f;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float a = acc[r][e] * f;
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      acc[r][e] = a;
    }
    mw[r] = mx;
    lw[r] = lt;
  }
  if (g == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int e = 0; e < VE; ++e) comb_acc[wave][r][x * VE + e] = acc[r][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      comb_m[wave][r] = mw[r];
      comb_l[wave][r] = lw[r];
    }
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < RT * DV; idx += 64 * NW) {
    const int r = idx / DV, d = idx % DV;
    const int gr = tile * RT + r;
    if (gr >= p.rows_total) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, comb_m[w][r]);
    float o = 0.f, lse = kNegInf;
    if (M != kNegInf) {
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2(comb_m[w][r] - M);
        den += f * comb_l[w][r];
        num += f * comb_acc[w][r][d];
      }
      o = num / den;
      lse = (M + __log2f(den)) * kLn2;
    }
    const int j = gr / p.group, h = kvh * p.group + gr % p.group;
    const int64_t row = ((int64_t)b * p.q_len + j) * p.num_q_heads + h;
    p.o_part[(row * p.num_splits + s) * DV + d] = o;
    if (d == 0) p.lse_part[row * p.num_splits + s] = lse;
  }
}

template <int DTYPE, int DK, int DV, int RT>
constexpr auto kernel_ptr() {
  return &stage1_valu_kernel<DTYPE, DK, DV, RT, 4>;
}

struct Entry {
  int dtype, dk, dv, rt;
  void (*fn)(Stage1Params);
};

constexpr Entry kTable[] = {
    {0, 64, 64, 4, kernel_ptr<0, 64, 64, 4>()},
    {0, 64, 64, 8, kernel_ptr<0, 64, 64, 8>()},
    {0, 64, 64, 16, kernel_ptr<0, 64, 64, 16>()},
    {0, 128, 128, 4, kernel_ptr<0, 128, 128, 4>()},
    {0, 128, 128, 8, kernel_ptr<0, 128, 128, 8>()},
    {0, 128, 128, 16, kernel_ptr<0, 128, 128, 16>()},
    {1, 128, 128, 4, kernel_ptr<1, 128, 128, 4>()},
    {1, 128, 128, 8, kernel_ptr<1, 128, 128, 8>()},
    {1, 128, 128, 16, kernel_ptr<1, 128, 128, 16>()},
    {1, 256, 256, 4, kernel_ptr<1, 256, 256, 4>()},
    {1, 256, 256, 8, kernel_ptr<1, 256, 256, 8>()},
    {1, 576, 512, 4, kernel_ptr<1, 576, 512, 4>()},
};

const Entry* find(int dtype, int dk, int dv, int rt) {
  for (const Entry& e : kTable)
    if (e.dtype == dtype && e.dk == dk && e.dv == dv && e.rt == rt) return &e;
  return nullptr;
}

}  // namespace

bool stage1_valu_supported(int dtype, int dk, int dv, int rows_per_wg) {
  return find(dtype, dk, dv, rows_per_wg) != nullptr;
}

hipError_t launch_stage1_valu(const Stage1Params& p, int dtype, int dk, int dv, hipStream_t st) {
  const Entry* e = find(dtype, dk, dv, p.rows_per_wg);
  if (!e) return hipErrorInvalidValue;
  hipLaunchKernelGGL(e->fn, dim3(p.num_wgs), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace splitkv
