// Stage 1 of split-KV paged decode on the matrix cores (gfx950), for KV heads
// shared by 16 or more query rows: an MLA latent head (aiter PR #4758,
// "[Gluon][MLA] Deeper async-copy pipeline in the bh16 stage-1 decode loop",
// bh16 / bh64 regimes) or a wide GQA group with draft tokens.
//
// Each wave owns 16 query rows and walks 32-key blocks of its split; NW waves
// of a workgroup take the blocks in turn with their own running max / sum /
// accumulators and merge at the end.  Per block:
//   * page walk: lane k < 32 looks up key k's page; keys past the visible end
//     clamp to the last visible key (weight 0 later);
//   * the block's K rows (and V rows when V is a separate cache) go straight
//     into the wave's LDS tile with global_load_lds_dwordx4; one instruction
//     moves 64 contiguous bytes of each of 16 keys;
//   * S^T = K Q^T with v_mfma_f32_16x16x32_bf16: A = K rows read from the
//     tile (16 B per lane), B = the wave's query rows held in VGPRs for the
//     whole kernel.  Lane l ends with the scores of keys 4g+i and 16+4g+i
//     (g = l/16, i < 4) for query row l%16;
//   * online softmax per query row (the lane's 8 scores, then the 4 lane
//     groups through two cross-lane steps);
//   * O^T += V^T P^T: B = the lane's 8 weights packed to bf16 (exactly the
//     operand layout), A = V^T gathered by two ds_read_b64_tr_b16 per
//     instruction (each 16-lane group transposes a 4-key x 16-dim block).
//     The MFMA's key slots follow the score layout, so no shuffle is needed.
// Tile layout (16-byte units, 32 keys): chunk c of key k sits at
//   (c/4)*128 + k*4 + ((c%4) ^ ((k/4)%4)).
// The XOR keeps both read patterns at the LDS bank floor: the 16-byte Q.K
// reads hit each bank 4 times per wave, the 8-byte transpose reads twice
// (rocm-libraries PR #10102, Motivation bank table: 4 lanes per bank is the
// ds_read_b128 floor on gfx950).
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int DK, int DV, bool VALIAS, int NW>
struct MCfg {
  static constexpr int KCH = DK * 2 / 16;          // 16-byte chunks of a K row
  static constexpr int VCH = DV * 2 / 16;          // 16-byte chunks of a V row
  static constexpr int KK = DK / 32;               // Q.K MFMA steps
  static constexpr int DT = DV / 16;               // P.V output tiles
  static constexpr int KINS = KCH / 2;             // DMA instructions for the K tile (32 keys)
  static constexpr int VINS = VALIAS ? 0 : VCH / 2;
  static constexpr int KTILE = KCH * 32 * 16;      // bytes
  static constexpr int VTILE = VALIAS ? 0 : VCH * 32 * 16;
  static constexpr int TILE = KTILE + VTILE;
  static constexpr int PART = 16 * DV * 4 + 2 * 16 * 4;  // merge state: acc [16][DV], m[16], l[16]
  static constexpr int WAVE_B = ((TILE > PART ? TILE : PART) + 255) / 256 * 256;
  static constexpr int SMEM = NW * WAVE_B;
  static_assert(KCH % 4 == 0 && VCH % 4 == 0, "row sizes");
  static_assert(!VALIAS || DV <= DK, "aliased V");
};

// 16-byte slot of chunk c of key k (k < 32) in a tile.
__device__ __forceinline__ int tile_slot(int k, int c) { return (c >> 2) * 128 + k * 4 + ((c & 3) ^ ((k >> 2) & 3)); }

template <int DK, int DV, bool VALIAS, int NW>
__global__ __launch_bounds__(64 * NW) void stage1_mfma_kernel(Stage1Params p) {
  using C = MCfg<DK, DV, VALIAS, NW>;
  __shared__ __align__(256) uint8_t smem[C::SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // lane group
  const int n = lane & 15;   // query row of this lane in the MFMA output
  uint8_t* ktile = smem + wave * C::WAVE_B;
  uint8_t* vtile = VALIAS ? ktile : ktile + C::KTILE;

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

  // This lane's query row (of the tile's 16) and its visible end.
  const int gr = tile * 16 + n;
  const bool row_ok = gr < p.rows_total;
  int row_end = sb;
  if (row_ok) {
    const int j = gr / p.group;
    const int nv = p.causal ? L - p.q_len + 1 + j : L;
    row_end = nv < se ? nv : se;
    if (row_end < sb) row_end = sb;
  }
  // The workgroup's last visible key: the largest row end over the tile
  // (rows of one tile differ only with causal drafts).
  int end_max = row_end;
  for (int o = 8; o > 0; o >>= 1) end_max = max(end_max, __shfl_xor(end_max, o));
  end_max = __builtin_amdgcn_readfirstlane(end_max);

  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int psh = p.page_shift, P = p.page_size;
  const int blk0 = sb + wave * 32;
  auto page_of = [&](int blk) {
    const int t = blk + (lane & 31);
    const int tc = t < end_max ? t : end_max - 1;
    return pt[tc >> psh];
  };
  int page_next = blk0 < end_max ? page_of(blk0) : 0;

  // Query rows as the B operand of S^T = K Q^T: lane l holds
  // q[row n][kk*32 + g*8 .. +7] for every kk (rows past the group read row 0).
  bf16x8_t qb[C::KK];
  {
    const int qr = row_ok ? gr : tile * 16;
    const int j = qr / p.group, h = kvh * p.group + qr % p.group;
    const uint4* qrow = (const uint4*)((const uint16_t*)p.q + (((int64_t)b * p.q_len + j) * p.num_q_heads + h) * DK);
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) qb[kk] = __builtin_bit_cast(bf16x8_t, qrow[kk * 4 + g]);
  }

  f32x4_t acc[C::DT];
#pragma unroll
  for (int d = 0; d < C::DT; ++d) acc[d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, l = 0.f;

  const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)kvh * p.ks_head * 2;
  const uint8_t* vbase = (const uint8_t*)p.v + (int64_t)kvh * p.vs_head * 2;
  const int64_t ks_page16 = p.ks_page * 2 / 16, ks_tok16 = p.ks_tok * 2 / 16;
  const int64_t vs_page16 = p.vs_page * 2 / 16, vs_tok16 = p.vs_tok * 2 / 16;

  // DMA lane mapping: instruction i moves key (i%2)*16 + lane/4, the 4 chunks
  // (i/2)*4 + ((lane%4) ^ ((key/4)%4)); its LDS slot is i*64 + lane.
  const int dkey0 = lane >> 2, dkey1 = 16 + (lane >> 2);
  const int dsw0 = (lane & 3) ^ ((dkey0 >> 2) & 3), dsw1 = (lane & 3) ^ ((dkey1 >> 2) & 3);

  for (int blk = blk0; blk < end_max; blk += NW * 32) {
    // ---- page walk: offsets of keys blk + (lane & 31) ----
    const int t = blk + (lane & 31);
    const int tc = t < end_max ? t : end_max - 1;
    const int page = page_next;
    const int slot = tc & (P - 1);
    const uint32_t koff = (uint32_t)(page * ks_page16 + slot * ks_tok16);
    const uint32_t voff = (uint32_t)(page * vs_page16 + slot * vs_tok16);
    if (blk + NW * 32 < end_max) page_next = page_of(blk + NW * 32);

    // ---- K (and V) rows into the tile ----
    {
      const uint32_t k0 = (uint32_t)__shfl((int)koff, dkey0), k1 = (uint32_t)__shfl((int)koff, dkey1);
#pragma unroll
      for (int i = 0; i < C::KINS; ++i) {
        const uint32_t ko = (i & 1) ? k1 : k0;
        const int ch = (i >> 1) * 4 + ((i & 1) ? dsw1 : dsw0);
        lds_dma16(kbase + (uint64_t)ko * 16 + ch * 16, ktile + i * 1024);
      }
      if constexpr (!VALIAS) {
        const uint32_t v0 = (uint32_t)__shfl((int)voff, dkey0), v1 = (uint32_t)__shfl((int)voff, dkey1);
#pragma unroll
        for (int i = 0; i < C::VINS; ++i) {
          const uint32_t vo = (i & 1) ? v1 : v0;
          const int ch = (i >> 1) * 4 + ((i & 1) ? dsw1 : dsw0);
          lds_dma16(vbase + (uint64_t)vo * 16 + ch * 16, vtile + i * 1024);
        }
      }
    }
    wait_vmcnt<0>();
    __builtin_amdgcn_wave_barrier();

    // ---- S^T = K Q^T, two 16-key halves ----
    f32x4_t st0 = {0.f, 0.f, 0.f, 0.f}, st1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < C::KK; ++kk) {
      const int c = kk * 4 + g;
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(ktile + tile_slot(n, c) * 16));
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, *(const uint4*)(ktile + tile_slot(16 + n, c) * 16));
      st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qb[kk], st0, 0, 0, 0);
      st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qb[kk], st1, 0, 0, 0);
    }

    // ---- online softmax for query row n over keys 4g+i, 16+4g+i ----
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = blk + 4 * g + i, k1 = blk + 16 + 4 * g + i;
      sc[i] = k0 < row_end ? st0[i] * p.scale_log2 : kNegInf;
      sc[4 + i] = k1 < row_end ? st1[i] * p.scale_log2 : kNegInf;
    }
    float bm = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sc[e]);
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const float al = mn == kNegInf ? 1.f : fast_exp2(m - mn);
    float pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e] = sc[e] == kNegInf ? 0.f : fast_exp2(sc[e] - mn);
    if (__any(al != 1.f && m != kNegInf)) {
      l *= al;
#pragma unroll
      for (int d = 0; d < C::DT; ++d) acc[d] *= al;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) l += pw[e];
    m = mn;
    uint4 pk;
    pk.x = pack_bf16x2(pw[0], pw[1]);
    pk.y = pack_bf16x2(pw[2], pw[3]);
    pk.z = pack_bf16x2(pw[4], pw[5]);
    pk.w = pack_bf16x2(pw[6], pw[7]);
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);

    // ---- O^T += V^T P^T ----
    // Transpose reads: lane 16g + s addresses 4 dims (s%4) of key 4g + s/4
    // (first read) or 16 + 4g + s/4 (second read).
    const int rk0 = 4 * g + (lane & 15) / 4, rk1 = 16 + rk0;
    const int q4 = lane & 3;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt) {
      const int c = 2 * dt + (q4 >> 1), half = (q4 & 1) * 8;
      typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
      const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)((__attribute__((address_space(3))) uint8_t*)vtile + tile_slot(rk0, c) * 16 + half));
      const i16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)((__attribute__((address_space(3))) uint8_t*)vtile + tile_slot(rk1, c) * 16 + half));
      const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[dt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- wave state into LDS: acc^T [16 rows][DV], m[16], l[16] ----
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  float* pacc = (float*)(smem + wave * C::WAVE_B);
  float* pml = pacc + 16 * DV;
  // Lane l holds O^T[dims dt*16 + 4g + i][row n].
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
    *(float4*)(pacc + n * DV + dt * 16 + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
  if (g == 0) {
    pml[n] = m;
    pml[16 + n] = l;
  }
  __syncthreads();

  // ---- merge the NW waves: thread -> (row, 4 dims) ----
  for (int idx = threadIdx.x; idx < 16 * DV / 4; idx += 64 * NW) {
    const int r = idx / (DV / 4), d = (idx % (DV / 4)) * 4;
    const int grr = tile * 16 + r;
    if (grr >= p.rows_total) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, ((const float*)(smem + w * C::WAVE_B))[16 * DV + r]);
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = kNegInf;
    if (M != kNegInf) {
      float den = 0.f;
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float* base = (const float*)(smem + w * C::WAVE_B);
        const float f = fast_exp2(base[16 * DV + r] - M);
        den += f * base[16 * DV + 16 + r];
        const float4 a = *(const float4*)(base + r * DV + d);
        num.x += f * a.x;
        num.y += f * a.y;
        num.z += f * a.z;
        num.w += f * a.w;
      }
      const float inv = 1.f / den;
      o = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
      lse = (M + __log2f(den)) * kLn2;
    }
    const int j = grr / p.group, h = kvh * p.group + grr % p.group;
    const int64_t row = ((int64_t)b * p.q_len + j) * p.num_q_heads + h;
    if (p.out) {
      store_out4(p.out, 1, row * DV + d, o);
      if (d == 0 && p.lse_out) p.lse_out[row] = lse;
    } else {
      *(float4*)(p.o_part + (row * p.num_splits + s) * DV + d) = o;
      if (d == 0) p.lse_part[row * p.num_splits + s] = lse;
    }
  }
}

struct Entry {
  int dk, dv;
  bool valias;
  void (*fn)(Stage1Params);
};

constexpr Entry kTable[] = {
    {576, 512, true, &stage1_mfma_kernel<576, 512, true, 4>},
    {256, 256, false, &stage1_mfma_kernel<256, 256, false, 4>},
    {128, 128, false, &stage1_mfma_kernel<128, 128, false, 4>},
};

const Entry* find(int dk, int dv, bool valias) {
  for (const Entry& e : kTable)
    if (e.dk == dk && e.dv == dv && e.valias == valias) return &e;
  return nullptr;
}

}  // namespace

bool stage1_mfma_supported(int dtype, int dk, int dv, bool v_aliases_k) {
  return dtype == 1 && find(dk, dv, v_aliases_k) != nullptr;
}

hipError_t launch_stage1_mfma(const Stage1Params& p, int dk, int dv, bool v_aliases_k, hipStream_t st) {
  const Entry* e = find(dk, dv, v_aliases_k);
  if (!e) return hipErrorInvalidValue;
  hipLaunchKernelGGL(e->fn, dim3(p.num_wgs), dim3(256), 0, st, p);
  return hipGetLastError();
}

}  // namespace splitkv
