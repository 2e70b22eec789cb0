// Stage 1 of split-KV paged decode on the vector ALUs (gfx950, wave64), for
// fp32 KV caches (bf16 caches run on the matrix cores, at every group size).
//
// One workgroup scores one split of one request's keys against RT query rows
// that share a KV head (aiter PR #4758, "[Gluon][MLA] Deeper async-copy
// pipeline in the bh16 stage-1 decode loop", Motivation: each stage-1
// program walks its split's KV blocks).
//
// NW waves take 64-key blocks of the split in turn, each with its own
// running max / sum / accumulator, merged at the end.  Per wave and block:
//   * page walk: lane t looks up key t's page once and turns it into 32-bit
//     row offsets (16-byte units) for K and V; keys past the visible end are
//     clamped to the last visible key and later get weight 0, so every load
//     is unconditional and all of a block's loads are in flight together;
//   * K: one direct-to-LDS 16-byte load per lane (global_load_lds_dwordx4)
//     moves 4 (or 2) whole rows per instruction, coalesced, into a 1 KB LDS
//     group; groups are padded by 16 bytes, which spreads the lane-per-key
//     reads below over all 64 banks at 4 lanes per bank, the ds_read_b128
//     floor.  A per-row pad is impossible because one instruction fills
//     several rows contiguously; the pad goes between load groups, as
//     rocm-libraries PR #10102 does for its head-dim-64 K tile (Motivation
//     bank table, Technical Details);
//   * Q.K: lane t owns key t and forms all RT dot products with FMAs; the
//     workgroup's query rows sit in LDS and each 16-byte chunk is one
//     broadcast read serving all 64 keys;
//   * softmax: each 16-lane DPP row keeps its own running max per query row;
//   * P.V: the 16 lanes of DPP row g accumulate keys 16g..16g+15; lane x owns
//     a contiguous slice of the head dim, so V rows arrive as coalesced
//     256-byte (or wider) segments, and key i's weight reaches the row's
//     lanes through row_newbcast:i.
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();

template <int DK, int DV, int RT, int NW>
struct Cfg {
  static constexpr int ES = 4;                   // element bytes (fp32)
  static constexpr int KRB = DK * ES;            // bytes of one K row
  static constexpr int VRB = DV * ES;            // bytes of one V row
  static constexpr int KCH = KRB / 16;           // 16-byte chunks of a K row
  static constexpr bool KLDS = KCH <= 64 && 64 % KCH == 0;  // K through the LDS tile
  static constexpr int RPI = KLDS ? 64 / KCH : 0;           // K rows per load instruction
  static constexpr int KINS = KLDS ? KCH : 0;               // load instructions per 64 rows
  static constexpr int GP = 64 * 16 + 16;        // LDS pitch of one load group (1 KB + pad)
  static constexpr int VU4 = VRB / 256;          // 16-byte loads per lane per V row
  static constexpr int VE = VU4 * 16 / ES;       // V elements a lane owns
  static constexpr int KTILE = KLDS ? KINS * GP : 0;
  static constexpr int PART = 4 * RT * DV * 4 + 4 * RT * 2 * 4;  // 4 DPP rows: acc, then m, l
  static constexpr int WAVE_B = ((KTILE > PART ? KTILE : PART) + 15) / 16 * 16;
  static constexpr int QB = RT * KRB;            // the workgroup's query rows
  static constexpr int SMEM = NW * WAVE_B + QB;
  static_assert(VRB % 256 == 0 && KRB % 16 == 0, "row sizes");
  static_assert(KLDS, "K rows of 16 to 64 chunks go through the LDS tile");
  static_assert(RT * VE <= 128, "accumulator budget");
};

template <int DK, int DV, int RT, int NW>
__global__ __launch_bounds__(64 * NW) void stage1_valu_kernel(Stage1Params p) {
  using C = Cfg<DK, DV, RT, NW>;
  constexpr int ES = C::ES, KRB = C::KRB, KCH = C::KCH, VU4 = C::VU4, VE = C::VE;

  __shared__ __align__(16) uint8_t smem[C::SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, in an SGPR
  const int g = lane >> 4;
  const int x = lane & 15;
  uint8_t* wave_lds = smem + C::QB + wave * C::WAVE_B;

  read_stage1_start_args(p);
  const uint32_t lid = (uint32_t)logical_wg(blockIdx.x, p.num_wgs, p.xcd_remap);
  const WgCoord wc = stage1_coord(p, lid);
  // Causal rows: later head tiles hold later query positions, which see more
  // keys, so they are handed out first (longest work first; the numbering
  // is a relabelling and changes no result).
  const int tile = p.causal ? p.head_tiles - 1 - wc.tile : wc.tile;
  const int kvh = wc.kvh, b = wc.b, s = wc.s;

  const int L = launch_ctx(p, b);
  int sb, se;
  split_range(L, p.num_splits, p.fd_splits, p.align_shift, p.split_chunk, s, sb, se);

  int row_end[RT];
  int end_max = sb;
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int gr = tile * RT + r;
    int e = sb;
    if (gr < p.rows_total) {
      const int j = (int)fdiv((uint32_t)gr, p.fd_group);
      const int n = p.causal ? L - p.q_len + 1 + j : L;
      e = n < se ? n : se;
      if (e < sb) e = sb;
    }
    row_end[r] = e;
    end_max = e > end_max ? e : end_max;
  }

  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int P = p.page_size;
  // Page id of this lane's key in the wave's first block.  Keys past the
  // visible end clamp to the last visible key (their weight is 0 later), so
  // every load below is unconditional.
  const int psh = p.page_shift;  // page sizes are powers of two
  auto page_of = [&](int blk) {
    const int t = blk + lane;
    const int tc = t < end_max ? t : end_max - 1;
    return pt[tc >> psh];
  };
  int blk0 = sb + wave * 64;
  int page_next = blk0 < end_max ? page_of(blk0) : 0;

  // The workgroup's query rows are read by every lane (lane = key): staged
  // once in LDS, each chunk of each row is one broadcast ds_read_b128 (all
  // lanes, one address).  Scalar loads would serve the broadcast for free,
  // but scalar loads return out of order, so every use waits for all of
  // them: one scalar-memory round trip per chunk.  LDS reads return in
  // order and pipeline.  Rows past the group repeat row 0 of the tile (their
  // scores are masked).
  uint8_t* q_lds = smem;   // first, so row/chunk offsets fit a ds_read immediate
  for (int idx = threadIdx.x; idx < RT * KCH; idx += 64 * NW) {
    const int r = idx / KCH, c = idx % KCH;
    int gr = tile * RT + r;
    if (gr >= p.rows_total) gr = tile * RT;
    const int j = (int)fdiv((uint32_t)gr, p.fd_group), h = kvh * p.group + gr - j * p.group;
    const uint4* src = (const uint4*)((const uint8_t*)p.q +
                                      ((((int64_t)b * p.q_len + j) * p.num_q_heads + h) * DK) * ES);
    *(uint4*)(q_lds + r * KRB + c * 16) = src[c];
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
  const int64_t ks_page16 = p.ks_page * ES / 16, ks_tok16 = p.ks_tok * ES / 16;
  const int64_t vs_page16 = p.vs_page * ES / 16, vs_tok16 = p.vs_tok * ES / 16;

  for (int blk = blk0; blk < end_max; blk += NW * 64) {
    // ---- page walk ----
    const int t = blk + lane;
    const int tc = t < end_max ? t : end_max - 1;
    const int page = page_next;
    const int slot = tc & (P - 1);
    const uint32_t koff = (uint32_t)(page * ks_page16 + slot * ks_tok16);
    const uint32_t voff = (uint32_t)(page * vs_page16 + slot * vs_tok16);
    if (blk + NW * 64 < end_max) page_next = page_of(blk + NW * 64);

    // ---- issue K (straight into the LDS tile), then V (16 rows per DPP row) ----
    if constexpr (C::RPI == 4) {
      // Load i moves keys i, 16+i, 32+i, 48+i (one per DPP row); each row
      // takes its key's offset by row_newbcast, no LDS round trip.
      [&]<int... I>(std::integer_sequence<int, I...>) {
        auto one = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          const uint32_t off = (uint32_t)row_bcast_i32<i>((int)koff);
          lds_dma16(kbase + (uint64_t)off * 16 + x * 16, wave_lds + i * C::GP);
        };
        (one(std::integral_constant<int, I>{}), ...);
      }(std::make_integer_sequence<int, 16>{});
    } else {
      // Load i moves keys i*RPI .. i*RPI + RPI - 1 (offsets by ds_bpermute).
      uint32_t offs[C::KINS];
#pragma unroll
      for (int i = 0; i < C::KINS; ++i) offs[i] = (uint32_t)__shfl((int)koff, i * C::RPI + lane / KCH);
#pragma unroll
      for (int i = 0; i < C::KINS; ++i)
        lds_dma16(kbase + (uint64_t)offs[i] * 16 + (lane % KCH) * 16, wave_lds + i * C::GP);
    }
    __builtin_amdgcn_sched_barrier(0);
    uint4 vv[16][VU4];
    [&]<int... I>(std::integer_sequence<int, I...>) {
      auto one = [&](auto ic) {
        constexpr int i = decltype(ic)::value;
        const uint32_t off = (uint32_t)row_bcast_i32<i>((int)voff);
        const uint8_t* vrow = vbase + (uint64_t)off * 16;
#pragma unroll
        for (int u = 0; u < VU4; ++u) vv[i][u] = *(const uint4*)(vrow + u * 16);
      };
      (one(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, 16>{});
    __builtin_amdgcn_sched_barrier(0);

    // ---- Q.K, lane t = key t ----
    // An opaque per-block offset keeps the compiler from hoisting every
    // query chunk of every row out of the block loop at once.
    uint32_t qoff = 0;
    asm volatile("" : "+v"(qoff));
    float sc[RT];
#pragma unroll
    for (int r = 0; r < RT; ++r) sc[r] = 0.f;
    auto dot_chunk = [&](const uint4 kc, int c) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        const uint4 qc = *(const uint4*)(q_lds + qoff + r * KRB + c * 16);
        sc[r] = fmaf(__builtin_bit_cast(float, qc.x), __builtin_bit_cast(float, kc.x), sc[r]);
        sc[r] = fmaf(__builtin_bit_cast(float, qc.y), __builtin_bit_cast(float, kc.y), sc[r]);
        sc[r] = fmaf(__builtin_bit_cast(float, qc.z), __builtin_bit_cast(float, kc.z), sc[r]);
        sc[r] = fmaf(__builtin_bit_cast(float, qc.w), __builtin_bit_cast(float, kc.w), sc[r]);
      }
    };
    {
      // K has landed once at most the V loads are outstanding.
      wait_vmcnt<16 * VU4>();
      // Where key `lane` sits in the tile (see the two load orders above).
      const uint8_t* krow = C::RPI == 4 ? wave_lds + (lane & 15) * C::GP + (lane >> 4) * KRB
                                        : wave_lds + (lane / C::RPI) * C::GP + (lane % C::RPI) * KRB;
#pragma unroll 2
      for (int c = 0; c < KCH; ++c) dot_chunk(*(const uint4*)(krow + c * 16), c);
      __builtin_amdgcn_wave_barrier();
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
      changed |= al[r] != 1.f && m[r] != kNegInf;  // a row with no key yet has nothing to rescale
      pr[r] = sc[r] == kNegInf ? 0.f : fast_exp2(sc[r] - mn);
      m[r] = mn;
    }
    if (__any(changed)) {
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        l[r] *= al[r];
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[r][e] *= al[r];
      }
    }

    {
      // P.V with fp32 weights and FMAs.
#pragma unroll
      for (int r = 0; r < RT; ++r) l[r] += pr[r];
      [&]<int... I>(std::integer_sequence<int, I...>) {
        auto one = [&](auto ic) {
          constexpr int i = decltype(ic)::value;
          float pw[RT];
#pragma unroll
          for (int r = 0; r < RT; ++r) pw[r] = row_bcast_f32<i>(pr[r]);
#pragma unroll
          for (int u = 0; u < VU4; ++u) {
            const float vf[4] = {__builtin_bit_cast(float, vv[i][u].x), __builtin_bit_cast(float, vv[i][u].y),
                                 __builtin_bit_cast(float, vv[i][u].z), __builtin_bit_cast(float, vv[i][u].w)};
#pragma unroll
            for (int r = 0; r < RT; ++r)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[r][u * 4 + e] = fmaf(pw[r], vf[e], acc[r][u * 4 + e]);
          }
        };
        (one(std::integral_constant<int, I>{}), ...);
      }(std::make_integer_sequence<int, 16>{});
    }
  }

  // ---- partial states of the 4*NW DPP rows into LDS, then one merge ----
  // Each wave writes its four rows' states into its own region (its K tile
  // is no longer read), so no barrier is needed before the writes.
  float* pacc = (float*)wave_lds;                   // [4][RT][DV]
  float* pml = pacc + 4 * RT * DV;                  // [4][RT] m, then [4][RT] l
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const float lt = row16_sum(l[r]);
#pragma unroll
    for (int e = 0; e < VE; e += 4)
      *(float4*)(pacc + (g * RT + r) * DV + x * VE + e) =
          make_float4(acc[r][e], acc[r][e + 1], acc[r][e + 2], acc[r][e + 3]);
    if (x == 0) {
      pml[g * RT + r] = m[r];
      pml[4 * RT + g * RT + r] = lt;
    }
  }
  __syncthreads();

  // Thread -> (row r, 4 consecutive dims); partials merged in a fixed order.
  for (int idx = threadIdx.x; idx < RT * DV / 4; idx += 64 * NW) {
    const int r = idx / (DV / 4), d = (idx % (DV / 4)) * 4;
    const int gr = tile * RT + r;
    if (gr >= p.rows_total) continue;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < 4 * NW; ++k) {
      const float* ml = (const float*)(smem + C::QB + (k >> 2) * C::WAVE_B) + 4 * RT * DV;
      M = fmaxf(M, ml[(k & 3) * RT + r]);
    }
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lse = kNegInf;
    if (M != kNegInf) {
      float den = 0.f;
      float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int k = 0; k < 4 * NW; ++k) {
        const float* base = (const float*)(smem + C::QB + (k >> 2) * C::WAVE_B);
        const float* ml = base + 4 * RT * DV;
        const float f = fast_exp2(ml[(k & 3) * RT + r] - M);
        den += f * ml[4 * RT + (k & 3) * RT + r];
        const float4 a = *(const float4*)(base + ((k & 3) * RT + r) * DV + d);
        num.x += f * a.x;
        num.y += f * a.y;
        num.z += f * a.z;
        num.w += f * a.w;
      }
      const float inv = 1.f / den;
      o = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
      lse = (M + __log2f(den)) * kLn2;
    }
    const int j = (int)fdiv((uint32_t)gr, p.fd_group), h = kvh * p.group + gr - j * p.group;
    const int64_t row = ((int64_t)b * p.q_len + j) * p.num_q_heads + h;
    if (p.out) {
      store_out4(p.out, 0, row * DV + d, o);
      if (d == 0 && p.lse_out) p.lse_out[row] = lse;
    } else {
      *(float4*)(p.o_part + part_slot(p, row, s) * DV + d) = o;
      if (d == 0) p.lse_part[part_slot(p, row, s)] = lse;
    }
  }
}

struct Entry {
  int dk, dv, rt, nw;
  void (*fn)(Stage1Params);
};

template <int DK, int DV, int RT, int NW = 4>
constexpr Entry entry() {
  return {DK, DV, RT, NW, &stage1_valu_kernel<DK, DV, RT, NW>};
}

constexpr Entry kTable[] = {
    entry<64, 64, 4>(),  entry<64, 64, 8>(),  entry<64, 64, 16>(),
    entry<128, 128, 4>(), entry<128, 128, 8>(),   // 16 rows at 128 would spill: two 8-row tiles
};

const Entry* find(int dtype, int dk, int dv, int rt) {
  if (dtype != 0) return nullptr;   // fp32 only
  for (const Entry& e : kTable)
    if (e.dk == dk && e.dv == dv && e.rt == rt) return &e;
  return nullptr;
}

}  // namespace

bool stage1_valu_supported(int dtype, int dk, int dv, int rows_per_wg) {
  return find(dtype, dk, dv, rows_per_wg) != nullptr;
}

hipError_t launch_stage1_valu(const Stage1Params& p, int dtype, int dk, int dv, hipStream_t st) {
  const Entry* e = find(dtype, dk, dv, p.rows_per_wg);
  if (!e) return hipErrorInvalidValue;
  hipLaunchKernelGGL(e->fn, dim3(p.num_wgs), dim3(64 * e->nw), 0, st, p);
  return hipGetLastError();
}

}  // namespace splitkv
