// Stage 1 of split-KV paged decode on the matrix cores (gfx950), for bf16 KV
// caches: an MLA latent head (aiter PR #4758, "[Gluon][MLA] Deeper
// async-copy pipeline in the bh16 stage-1 decode loop", bh16 / bh64
// regimes), a GQA group, or a wide GQA group with draft tokens.
//
// Each wave owns 16 query rows; smaller groups leave part of the tile empty
// (decode does so few flops per byte that the matrix cores idle either way,
// and one 16x16x32 MFMA still replaces hundreds of vector-ALU issues).  A
// workgroup has RW x KW waves: RW 16-row tiles that share each K/V block
// through a ring of LDS tiles (one barrier per block), or KW key streams that
// take the split's 32-key blocks in turn with their own tile and running max
// / sum / accumulators, merged at the end.  Shapes, by rows per KV head:
//   * 64+ (wide MLA; prefill, where every query position of a GQA group is
//     a row; 128+ at head dim 128 takes 8 tiles), 32 (draft groups): 8, 4 or
//     2 tiles on a ring of 3 (two blocks in flight; a ring of 2 for the four
//     tiles at head dim 128), each block read once per 128, 64 or 32 rows;
//   * 16 (MLA bh16): one tile, four key streams, load -> wait -> compute;
//   * 1-15 (GQA, MLA with few heads): one wave alone on a ring of 3 (two
//     blocks in flight); 25 KB of LDS at head dim 64 and 49 KB at 128 (two
//     workgroups per CU), 97 KB at 256 and 109 KB at 576 (one).
// Head dims 64, 128, 256 and 576/512 share one tile layout (below).  At 64,
// rocm-libraries PR #10102 pads groups of 128-byte K rows in LDS to spread
// its reads over the banks (Motivation bank table); the XOR swizzle here
// does that job without padding, for both the row reads of Q.K and the
// transpose reads of P.V.
// Per block:
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
//   (c/4)*128 + k*4 + ((c%4) ^ swz(k)),  swz(k) = (-(k/4)) mod 4.
// gfx950 LDS has 64 four-byte banks (rocm-libraries PR #10102, Motivation
// bank table) and serves 256 bytes per cycle, so a read is split into
// phases that must each touch every bank once.  Measured on MI355X: a
// 16-byte read's phase is lane quads {0, 3} of one 16-lane window w plus
// quads {1, 2} of window w ^ 1; an 8-byte read's phases are lanes 0-31 and
// 32-63.  With swz, the Q.K reads (window g = chunk column, lane n%16 = key)
// and the transpose reads (groups g, g + 1 on one chunk pair) both sweep all
// 64 banks in every phase.  The plain (k/4)%4, or its two bits swapped,
// leaves one of the two patterns two lanes deep per bank.
#pragma once

#include <utility>

#include "device_common.h"
#include "launch.h"

namespace splitkv {

namespace {

constexpr float kNegInf = -__builtin_inff();

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

template <int DK, int DV, bool VALIAS, int RW, int KW>
struct MCfg {
  static constexpr int NW = RW * KW;               // waves: RW row tiles x KW key streams
  // Ring depth: 3 tiles (two blocks in flight while one is computed) for
  // shared row tiles and a lone wave; none for key streams (one tile each).
  // Measured against 4 tiles: lone wave (64K GQA) 15.7 / 16.4 us, drafts
  // 13.6 / 14.4, prefill 4 x 2048 at head dim 128 139 / 162 (the smaller
  // ring also lets a third workgroup onto the CU), wide MLA 379 / 380.
  // Again for the lone wave at head dim 128 with one workgroup per CU:
  // 2 / 3 / 4 / 5 tiles, stage 1 18.6 / 15.4 / 15.9 / 16.3 us; and for the
  // drafts' work list of 128-key splits, where 4 tiles put all four blocks
  // of a workgroup in flight at once: 10.0 against 10.7 us; 2 tiles (two
  // workgroups per CU, 64-key splits) 13.7.
  // The four-wave shape at head dim 128 (prefill, whose keys mostly come
  // from cache) takes 2 tiles, which fits a fourth workgroup per CU: whole
  // op 4 x 2048 132.3 -> 128.0 us, varlen 95.0 -> 90.8.
  static constexpr int NBUF = KW == 1 ? (DK == 128 && RW == 4 ? 2 : 3) : 1;
  static constexpr int KCH = DK * 2 / 16;          // 16-byte chunks of a K row
  static constexpr int VCH = DV * 2 / 16;          // 16-byte chunks of a V row
  static constexpr int KK = DK / 32;               // Q.K MFMA steps
  static constexpr int DT = DV / 16;               // P.V output tiles
  static constexpr int KINS = KCH / 2;             // DMA instructions for the K tile (32 keys)
  static constexpr int VINS = VALIAS ? 0 : VCH / 2;
  static constexpr int KTILE = KCH * 32 * 16;      // bytes
  static constexpr int VTILE = VALIAS ? 0 : VCH * 32 * 16;
  static constexpr int TILE = ((KTILE + VTILE) + 255) / 256 * 256;
  static constexpr int TILES = KW * NBUF * TILE;
  static constexpr int PIDS = NBUF > 1 ? NW * NBUF * 256 : 0;  // per-wave page-id ring (ring path only)
  // Merge state of a key stream: acc [16][RS], m[16], l[16].  The row
  // stride is padded by 16 bytes so that a write of the 16 rows' 16-byte
  // pieces (lane n: row n) touches all 64 banks once; unpadded, the rows sat
  // a multiple of 256 bytes apart and every write was 16 lanes deep per bank.
  static constexpr int RS = DV + 4;
  static constexpr int PART = 16 * RS * 4 + 2 * 16 * 4;
  static constexpr int PARTS = KW > 1 ? NW * PART : 0;   // only key streams need merging
  static constexpr int SMEM = TILES + PIDS > PARTS ? TILES + PIDS : PARTS;
  static_assert(KCH % 4 == 0 && VCH % 4 == 0, "row sizes");
  static_assert(!VALIAS || DV <= DK, "aliased V");
  static_assert(SMEM <= 160 * 1024, "LDS budget");
  static_assert(KINS % RW == 0 && VINS % RW == 0, "DMA instructions split evenly over the row tiles");
  static_assert(RW == 1 || KW == 1, "shared tiles carry one key stream");
  static_assert(SMEM >= 256 + RW * 16 * 64 * 4, "in-kernel merge: flag word + weights [rows][64 splits]");
  static constexpr int MINE = NBUF > 1 ? (KINS + VINS) / RW : 0;  // DMA instructions per wave per block
};

// 16-byte slot of chunk c of key k (k < 32) in a tile.
__device__ __forceinline__ int tile_swz(int k) { return (-(k >> 2)) & 3; }
__device__ __forceinline__ int tile_slot(int k, int c) { return (c >> 2) * 128 + k * 4 + ((c & 3) ^ tile_swz(k)); }

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kLaK = 4;  // Q.K read steps in flight ahead of the MFMA
constexpr int kLaV = 6;  // P.V read steps in flight ahead of the MFMA
constexpr float kLazyLog2 = 8.f;  // reference-max slack (log2 units) before a rescale

__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)ptr;
}

// The tile reads are written as inline assembly.  A tile is filled by
// global_load_lds, and the compiler, which cannot tell one tile from
// another, would otherwise make every LDS read wait for all of those loads,
// including the ones that fill the next tiles; the kernel orders the tiles
// itself (vmcnt wait + barrier per block).  The reads are then invisible to
// the compiler's counters, so each result passes through lds_wait2, which
// waits until at most N LDS operations are outstanding and ties the
// registers to the wait.  Other LDS or scalar-memory operations in flight
// only make the wait stricter.
template <int OFF>
__device__ __forceinline__ void lds_read2_b128(i32x4_t& r0, i32x4_t& r1, uint32_t a0, uint32_t a1) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b128 %0, %2 offset:%4\n\tds_read_b128 %1, %3 offset:%4"
               : "=&v"(r0), "=&v"(r1)
               : "v"(a0), "v"(a1), "i"(OFF));
}

template <int OFF>
__device__ __forceinline__ void lds_read2_tr16(i16x4_t& r0, i16x4_t& r1, uint32_t a0, uint32_t a1) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%4\n\tds_read_b64_tr_b16 %1, %3 offset:%4"
               : "=&v"(r0), "=&v"(r1)
               : "v"(a0), "v"(a1), "i"(OFF));
}

// Workgroup barrier for the shared tile ring.  Every wave has already
// waited for its own DMA of the block being published (vmcnt) and for its
// own reads of the tile being recycled (lds_wait2 down to 0), so only the
// meeting is needed; a __syncthreads fence would also wait for the DMAs
// still filling the next tiles.  The memory clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void tile_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int OFF>
__device__ __forceinline__ int lds_read_b32(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset");
  int r;
  asm volatile("ds_read_b32 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
  return r;
}

template <int N, typename T>
__device__ __forceinline__ void lds_wait2(T& r0, T& r1) {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(r0), "+v"(r1) : "i"(N));
}

template <int DK, int DV, bool VALIAS, int RW, int KW>
__global__ __launch_bounds__(64 * RW * KW) void stage1_mfma_kernel(Stage1Params p) {
  using C = MCfg<DK, DV, VALIAS, RW, KW>;
  __shared__ __align__(256) uint8_t smem[C::SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rw = wave % RW;   // row tile of this wave
  const int kw = wave / RW;   // key stream of this wave
  const int g = lane >> 4;    // lane group
  const int n = lane & 15;    // query row of this lane in the MFMA output
  auto tile_k = [&](int buf) { return smem + (kw * C::NBUF + buf) * C::TILE; };
  auto tile_v = [&](int buf) { return VALIAS ? tile_k(buf) : tile_k(buf) + C::KTILE; };

  read_stage1_start_args(p);
  const uint32_t lid = (uint32_t)logical_wg(blockIdx.x, p.num_wgs, p.xcd_remap);
  const WgCoord wc = stage1_coord(p, lid);
  // Causal rows: later head tiles hold later query positions, which see more
  // keys, so they are handed out first (longest work first; the numbering
  // is a relabelling and changes no result).
  const int tile = p.causal ? p.head_tiles - 1 - wc.tile : wc.tile;
  const int kvh = wc.kvh, b = wc.b, s = wc.s;

  // The workgroup's last query row (rows differ in visible length only with
  // causal drafts; every row of a workgroup belongs to one request).
  const int first_row = tile * RW * 16;
  int last_row = first_row + RW * 16 - 1;
  if (last_row >= p.rows_total) last_row = p.rows_total - 1;
  // Split bounds [sb_, se_) for context length Lc, and the workgroup's last
  // visible key in the split (emax_, at least sb_).
  auto bounds = [&](int Lc, int& sb_, int& se_, int& emax_) {
    split_range(Lc, p.num_splits, p.fd_splits, p.align_shift, p.split_chunk, s, sb_, se_);
    const int j = (int)fdiv((uint32_t)last_row, p.fd_group);
    const int nv = p.causal ? Lc - p.q_len + 1 + j : Lc;
    emax_ = nv < se_ ? nv : se_;
    if (emax_ < sb_) emax_ = sb_;
  };

  const int32_t* pt = p.page_table + (int64_t)b * p.max_pages;
  const int psh = p.page_shift, P = p.page_size;

  // Ring path: page ids travel through LDS.  Block X's ids are DMA'd into
  // slot X % NB of this wave's ring (lane k: key k % 32).  A page id loaded
  // into a register would make the compiler wait for every DMA in flight
  // before its first use.
  constexpr int NB = C::NBUF, D = NB - 1;
  uint8_t* pid_ring = smem + C::TILES + wave * NB * 256;
  auto issue_pid_at = [&](int sb_, int emax_, int blk_idx, int slot) {
    const int t = sb_ + (kw + blk_idx * KW) * 32 + (lane & 31);
    const int tc = t < emax_ ? t : emax_ - 1;
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(pt + (tc >> psh)),
                                     (__attribute__((address_space(3))) void*)(pid_ring + slot * 256), 4, 0, 0);
  };
  // With one request (p.guess_ctx > 0, the plan's longest context), the
  // first blocks' ids are requested before the context length arrives, on
  // the guess that the request has that length; a wrong guess costs a wait
  // and a second request.  That takes one dependent load off the start.
  int sb_g = 0, se_g = 0, em_g = 0;
  if constexpr (NB > 1) {
    // Under a split table the split starts at s * chunk whatever the length,
    // and ends at (s + 1) * chunk unless it is its request's last.
    int gctx = p.guess_ctx;
    if (p.live_splits > 0 && (s + 1) * p.split_chunk < gctx) gctx = (s + 1) * p.split_chunk;
    if (gctx > 0) bounds(gctx, sb_g, se_g, em_g);
    if (em_g > sb_g) {
#pragma unroll
      for (int j = 0; j < D; ++j) issue_pid_at(sb_g, em_g, j, j);
    }
  }

  const int L = launch_ctx(p, b);
  int sb, se, end_max;
  bounds(L, sb, se, end_max);
  const bool guess_ok = em_g > sb_g && sb_g == sb && em_g == end_max;

  // This lane's query row and its visible end.  Rows past the group are
  // never written; they score every key (their end is unbounded), so they
  // never keep a block on the masked path.
  const int gr = (tile * RW + rw) * 16 + n;
  const bool row_ok = gr < p.rows_total;
  int row_end = 0x7fffffff;
  if (row_ok) {
    const int j = (int)fdiv((uint32_t)gr, p.fd_group);
    const int nv = p.causal ? L - p.q_len + 1 + j : L;
    row_end = nv < se ? nv : se;
    if (row_end < sb) row_end = sb;
  }

  // Stream kw takes blocks it = 0, 1, ... at keys sb + (kw + it*KW)*32.  All
  // streams run the same trip count so shared-tile barriers stay uniform.
  const int nit = (end_max - sb + 32 * KW - 1) / (32 * KW);
  auto blk_of = [&](int it) { return sb + (kw + it * KW) * 32; };

  // Query rows as the B operand of S^T = K Q^T: lane l holds
  // q[row n][kk*32 + g*8 .. +7] for every kk (rows past the group read row 0).
  bf16x8_t qb[C::KK];
  {
    const int qr = row_ok ? gr : first_row;
    const int j = (int)fdiv((uint32_t)qr, p.fd_group), h = kvh * p.group + qr - j * p.group;
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
  // Strides in 16-byte units.  32-bit arithmetic is exact: the host keeps
  // every row of the pool below 2^32 units from its head's base.
  const uint32_t ks_page16 = (uint32_t)(p.ks_page * 2 / 16), ks_tok16 = (uint32_t)(p.ks_tok * 2 / 16);
  const uint32_t vs_page16 = (uint32_t)(p.vs_page * 2 / 16), vs_tok16 = (uint32_t)(p.vs_tok * 2 / 16);

  // DMA lane mapping: instruction i moves key (i%2)*16 + lane/4, the 4 chunks
  // (i/2)*4 + ((lane%4) ^ swz(key)); its LDS slot is i*64 + lane.  With
  // RW waves on one stream, wave rw issues instructions rw, rw + RW, ...
  const int dkey0 = lane >> 2, dkey1 = 16 + (lane >> 2);
  const int dsw0 = (lane & 3) ^ tile_swz(dkey0), dsw1 = (lane & 3) ^ tile_swz(dkey1);
  static_assert(RW == 1 || RW % 2 == 0, "row-tile waves: one, or an even count");
  // Row of key t (clamped to the last visible key like every other key) in
  // page `page`, in 16-byte units from the head's base.
  auto row16 = [&](int t, int page, uint32_t pstride, uint32_t tstride) {
    const int tc = t < end_max ? t : end_max - 1;
    return (uint32_t)page * pstride + (uint32_t)(tc & (P - 1)) * tstride;
  };
  // Moves block blk (page0 / page1: page ids of keys blk + dkey0 and
  // blk + dkey1) into tile buffer buf.  Each lane forms one source address
  // per key it moves and steps through the chunk groups at constant offsets,
  // which the loads carry as immediates.
  auto issue_dma_from = [&](const uint8_t* base, uint32_t pstride, uint32_t tstride, uint8_t* tile, int nins,
                            int blk, int page0, int page1) {
    if constexpr (RW % 2 == 0) {
      // Instruction i = rw + ii*RW always moves key dkey(rw % 2), chunk group
      // rw/2 + ii*RW/2: one source row per lane.
      const bool odd = rw & 1;
      const uint8_t* src = base + ((uint64_t)row16(blk + (odd ? dkey1 : dkey0), odd ? page1 : page0, pstride, tstride) +
                                   (rw >> 1) * 4 + (odd ? dsw1 : dsw0)) * 16;
#pragma unroll
      for (int ii = 0; ii < nins / RW; ++ii) lds_dma16(src + ii * (RW / 2) * 64, tile + (rw + ii * RW) * 1024);
    } else {
      const uint8_t* src0 = base + ((uint64_t)row16(blk + dkey0, page0, pstride, tstride) + dsw0) * 16;
      const uint8_t* src1 = base + ((uint64_t)row16(blk + dkey1, page1, pstride, tstride) + dsw1) * 16;
#pragma unroll
      for (int i = 0; i < nins; ++i) lds_dma16(((i & 1) ? src1 : src0) + (i >> 1) * 64, tile + i * 1024);
    }
  };
  auto issue_dma = [&](int blk, int page0, int page1, int buf) {
    issue_dma_from(kbase, ks_page16, ks_tok16, tile_k(buf), C::KINS, blk, page0, page1);
    if constexpr (!VALIAS) issue_dma_from(vbase, vs_page16, vs_tok16, tile_v(buf), C::VINS, blk, page0, page1);
  };

  // This lane's LDS byte offsets inside a tile.  Q.K step kk reads chunk
  // kk*4 + g of keys n and 16 + n: slot(k, kk*4 + g) = kk*128 + slot(k, g).
  // P.V step dt reads chunk 2dt + q4/2 of keys rk0 and rk1 (half q4%2 of
  // it): slot(k, 2dt + x) = (dt/2)*128 + slot(k, 2(dt%2) + x).  The
  // column-block step (2048 bytes) goes into the read's immediate offset.
  const int rk0 = 4 * g + (lane & 15) / 4, rk1 = 16 + rk0;
  const int q4 = lane & 3, vx = q4 >> 1, half = (q4 & 1) * 8;
  const uint32_t kq0 = tile_slot(n, g) * 16, kq1 = tile_slot(16 + n, g) * 16;
  const uint32_t ve0 = tile_slot(rk0, vx) * 16 + half, ve1 = tile_slot(rk1, vx) * 16 + half;
  const uint32_t vo0 = tile_slot(rk0, 2 + vx) * 16 + half, vo1 = tile_slot(rk1, 2 + vx) * 16 + half;

  // ---- S^T = K Q^T for one tile: two 16-key halves; reads run kLaK steps ahead ----
  auto qk = [&](const uint8_t* ktile, f32x4_t& st0, f32x4_t& st1) {
    const uint32_t kt = lds_addr(ktile);
    st0 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
    constexpr int LA = kLaK;
    i32x4_t kr[LA + 1][2];
    auto rd = [&](auto ic) {
      constexpr int kk = decltype(ic)::value;
      if constexpr (kk < C::KK)
        lds_read2_b128<kk * 2048>(kr[kk % (LA + 1)][0], kr[kk % (LA + 1)][1], kt + kq0, kt + kq1);
    };
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (rd(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, LA>{});
    [&]<int... I>(std::integer_sequence<int, I...>) {
      auto step = [&](auto ic) {
        constexpr int kk = decltype(ic)::value;
        rd(std::integral_constant<int, kk + LA>{});
        constexpr int ahead = C::KK - 1 - kk < LA ? C::KK - 1 - kk : LA;
        i32x4_t& r0 = kr[kk % (LA + 1)][0];
        i32x4_t& r1 = kr[kk % (LA + 1)][1];
        lds_wait2<2 * ahead>(r0, r1);
        st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r0), qb[kk], st0, 0, 0, 0);
        st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r1), qb[kk], st1, 0, 0, 0);
        // Keep the step's MFMAs right after its wait: left alone, the
        // scheduler sinks them below the later steps' waits, so the reads no
        // longer overlap the matrix cores.
        __builtin_amdgcn_sched_barrier(0);
      };
      (step(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, C::KK>{});
  };

  // Dot products q.k of query row n for keys 4g+i and 16+4g+i (-inf where
  // masked), and the max of this lane's eight in log2 units.  The scale is
  // applied once to the max here and inside the weights' FMA below, not per
  // score (scale > 0, so the max of the scaled scores is the scaled max).
  // The row's block max (over its four lane groups) is only formed when a
  // rescale needs it: a row needs none exactly when none of its lanes'
  // maxima passes the reference, which every lane of the row holds.
  // The mask is applied in place on the MFMA results, and only on blocks
  // that reach past some row's visible end: with the scores copied into an
  // array on both paths the compiler moved every score two or three times.
  auto scores = [&](int blk, f32x4_t& st0, f32x4_t& st1) {
    if (!__all(blk + 32 <= row_end)) {
      // keys 4g+i and 16+4g+i of the block are visible while below rem
      const int rem = row_end - blk - 4 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st0[i] = i < rem ? st0[i] : kNegInf;
        st1[i] = 16 + i < rem ? st1[i] : kNegInf;
      }
    }
    float bm = st0[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) bm = fmaxf(bm, st0[i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) bm = fmaxf(bm, st1[i]);
    return bm * p.scale_log2;
  };

  // ---- weights against the reference max m, row sum, O^T += V^T P^T ----
  // Transpose reads run kLaV steps ahead: lane 16g + s addresses 4 dims
  // (s%4) of key 4g + s/4 (first read) or 16 + 4g + s/4 (second read).
  auto pv = [&](const uint8_t* vtile, const f32x4_t& st0, const f32x4_t& st1) {
    const uint32_t vt = lds_addr(vtile);
    // Weight 2^(s * scale_log2 - m), one FMA per score.  A row whose
    // reference is still -inf has only -inf scores; subtracting 0 instead
    // gives exp2(-inf) = 0 without a test per score.
    const float ms = m == kNegInf ? 0.f : m;
    float pw[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pw[e] = fast_exp2(fmaf(e < 4 ? st0[e] : st1[e - 4], p.scale_log2, -ms));
#pragma unroll
    for (int e = 0; e < 8; ++e) l += pw[e];
    uint4 pk;
    pk.x = pack_bf16x2(pw[0], pw[1]);
    pk.y = pack_bf16x2(pw[2], pw[3]);
    pk.z = pack_bf16x2(pw[4], pw[5]);
    pk.w = pack_bf16x2(pw[6], pw[7]);
    const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
    constexpr int LA = kLaV;
    i16x4_t vr[LA + 1][2];
    auto rd = [&](auto ic) {
      constexpr int dt = decltype(ic)::value;
      if constexpr (dt < C::DT) {
        constexpr int off = (dt >> 1) * 2048;
        if constexpr (dt & 1)
          lds_read2_tr16<off>(vr[dt % (LA + 1)][0], vr[dt % (LA + 1)][1], vt + vo0, vt + vo1);
        else
          lds_read2_tr16<off>(vr[dt % (LA + 1)][0], vr[dt % (LA + 1)][1], vt + ve0, vt + ve1);
      }
    };
    [&]<int... I>(std::integer_sequence<int, I...>) {
      (rd(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, LA>{});
    [&]<int... I>(std::integer_sequence<int, I...>) {
      auto step = [&](auto ic) {
        constexpr int dt = decltype(ic)::value;
        rd(std::integral_constant<int, dt + LA>{});
        constexpr int ahead = C::DT - 1 - dt < LA ? C::DT - 1 - dt : LA;
        i16x4_t& r0 = vr[dt % (LA + 1)][0];
        i16x4_t& r1 = vr[dt % (LA + 1)][1];
        lds_wait2<2 * ahead>(r0, r1);
        const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[dt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // as in Q.K
      };
      (step(std::integral_constant<int, I>{}), ...);
    }(std::make_integer_sequence<int, C::DT>{});
  };

  // Lazy rescale (the online-softmax variant that moves the reference max
  // only when a block's max exceeds it by more than kLazyLog2; rocm-libraries
  // PR #10102, Risk Assessment, lists such a switch for its attention
  // kernel): the hot loop
  // below never touches the accumulators outside the matrix cores, so they
  // stay in AGPRs; a block that needs a new reference leaves the loop,
  // rescales here and rejoins.  Weights are then at most 2^kLazyLog2, which
  // fp32 sums and bf16 weights hold exactly as well as weights <= 1.
  auto rescale = [&](float bm) {
    const float mn = fmaxf(m, bm);
    const float al = mn == kNegInf ? 1.f : fast_exp2(m - mn);
    if (al != 1.f && m != kNegInf) {
      l *= al;
#pragma unroll
      for (int d = 0; d < C::DT; ++d) acc[d] *= al;
    }
    m = mn;
  };

  // Runs blocks [0, nb) of this wave: front(it) makes block it readable and
  // returns its tile buffer; mid(it) runs between Q.K and P.V.
  auto run_blocks = [&](int nb, auto&& front, auto&& mid) {
    f32x4_t st0, st1;
    float bm = kNegInf;
    int it = 0;
    while (it < nb) {
      int buf = 0;
      for (; it < nb; ++it) {
        buf = front(it);
        qk(tile_k(buf), st0, st1);
        bm = scores(blk_of(it), st0, st1);
        mid(it);
        if (__any(bm > m + kLazyLog2)) break;
        pv(tile_v(buf), st0, st1);
      }
      if (it < nb) {
        rescale(max_xor32(max_xor16(bm)));   // the row's block max
        pv(tile_v(buf), st0, st1);
        ++it;
      }
    }
  };

  if constexpr (C::NBUF == 1) {
    // One wave per key stream, its own tile: load, wait, compute.  Stream
    // kw has blocks kw, kw + KW, ... below end_max.
    const int first = sb + kw * 32;
    const int nb = first < end_max ? (end_max - first + 32 * KW - 1) / (32 * KW) : 0;
    // Page ids of this lane's two DMA keys, one block ahead.
    auto pages_of = [&](int blk, int& p0, int& p1) {
      const int t0 = blk + dkey0, t1 = blk + dkey1;
      p0 = pt[(t0 < end_max ? t0 : end_max - 1) >> psh];
      p1 = pt[(t1 < end_max ? t1 : end_max - 1) >> psh];
    };
    int pn0 = 0, pn1 = 0;
    if (nb > 0) pages_of(blk_of(0), pn0, pn1);
    run_blocks(nb, [&](int it) {
      __builtin_amdgcn_wave_barrier();   // the previous block's reads are done (lds_wait2 to 0)
      const int p0 = pn0, p1 = pn1;
      if (it + 1 < nb) pages_of(blk_of(it + 1), pn0, pn1);
      issue_dma(blk_of(it), p0, p1, 0);
      wait_vmcnt<0>();
      __builtin_amdgcn_wave_barrier();
      return 0;
    }, [&](int) {});
  } else if (nit > 0) {    // RW waves (or one) share a ring of NBUF tiles; D = NBUF - 1 blocks are in
    // flight while one is computed.  Iteration it waits for block it, meets
    // the other waves (block it is then in LDS, and the buffer block it + D
    // reuses is no longer read), loads the page ids of block it + 2D and
    // issues block it + D.  Page ids are thus loaded D blocks before their
    // DMA, so the compiler's wait for them never drains the DMA queue, and
    // the explicit wait for block it counts exactly the loads issued after
    // it: D - 1 x (one page-id load + this wave's DMAs).  Near the end of the
    // split fewer blocks follow, and the wait is for everything.
    // Block X's ids are requested just before block X - D is issued, so the
    // wait for block X - D covers them.
    const uint32_t pid_addr = lds_addr(pid_ring) + dkey0 * 4;   // entry k: key k % 32
    auto issue_pid = [&](int blk_idx, int slot) { issue_pid_at(sb, end_max, blk_idx, slot); };
    // This lane's two DMA keys' page ids from ring slot `slot` (the caller
    // waits for them with lds_wait2).
    auto read_pids = [&](int slot, int& p0, int& p1) {
      p0 = lds_read_b32<0>(pid_addr + slot * 256);
      p1 = lds_read_b32<64>(pid_addr + slot * 256);
    };
    // Prologue: ids of blocks 0 .. D-1 (unless the guess above already asked
    // for them; a wrong guess's loads land before the second request), then
    // blocks 0 .. D-1 themselves (each preceded by the ids of block j + D).
    if (!guess_ok) {
      wait_vmcnt<0>();
#pragma unroll
      for (int j = 0; j < D; ++j) issue_pid(j, j);
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < D; ++j) {
      issue_pid(j + D, (j + D) % NB);
      int p0, p1;
      read_pids(j, p0, p1);
      lds_wait2<0>(p0, p1);
      __builtin_amdgcn_sched_barrier(0);
      if (j < nit) issue_dma(blk_of(j), p0, p1, j);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Iteration it: wait for block it (all but the D - 1 later steps of
    // this wave: page ids + DMAs), read the ids of block it + D (they came
    // with block it), meet, queue the ids of block it + 2D and block it + D,
    // then compute block it.
    // Waves of odd row tiles issue their share of block it + D after Q.K
    // instead of right after the barrier, so that the row tiles' DMA issue
    // and Q.K reads do not all hit the CU's memory pipeline and LDS at once
    // (wide MLA: 3-5% faster).  The order of each wave's loads, and so the
    // wait counts, stay the same.
    const bool late = RW > 1 && (rw & 1);
    int lp0 = 0, lp1 = 0;
    run_blocks(nit, [&](int it) {
      if (it + D <= nit) {
        wait_vmcnt<(D - 1) * (C::MINE + 1)>();
      } else {
        wait_vmcnt<0>();
      }
      int p0, p1;
      read_pids((it + D) % NB, p0, p1);
      tile_barrier();
      issue_pid(it + 2 * D, (it + 2 * D) % NB);
      lds_wait2<0>(p0, p1);
      __builtin_amdgcn_sched_barrier(0);
      if (!late) {
        if (it + D < nit) issue_dma(blk_of(it + D), p0, p1, (it + D) % NB);
      } else {
        lp0 = p0;
        lp1 = p1;
      }
      __builtin_amdgcn_sched_barrier(0);
      return it % NB;
    }, [&](int it) {
      if (late && it + D < nit) {
        __builtin_amdgcn_sched_barrier(0);
        issue_dma(blk_of(it + D), lp0, lp1, (it + D) % NB);
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  }
  // No direct-to-LDS load (the trailing page-id requests, an unused guess)
  // may still be in flight when the wave's LDS is released.
  if constexpr (C::NBUF > 1) wait_vmcnt<0>();

  l = sum_xor32(sum_xor16(l));
  auto write_row = [&](int grr, int d, float4 o, float lse) {
    const int j = (int)fdiv((uint32_t)grr, p.fd_group), h = kvh * p.group + grr - j * p.group;
    const int64_t row = ((int64_t)b * p.q_len + j) * p.num_q_heads + h;
    if (p.out) {
      store_out4(p.out, 1, row * DV + d, o);
      if (d == 0 && p.lse_out) p.lse_out[row] = lse;
    } else {
      float* const po = p.o_part + part_slot(p, row, s) * DV + d;
      float* const pl = p.lse_part + part_slot(p, row, s);
      if constexpr (DV >= 256) {
        // Wide rows (32 KB of partials per drafts workgroup, 32 KB per MLA
        // one): write through the L2 (device-scope stores), so that the
        // partials are not left dirty in the L2 for the write-back at the
        // kernel's end.  Drafts whole op 15.31 -> 14.54 us, stage 1 10.71 ->
        // 10.21; MLA batch 48 unchanged; at head dim 128 (8 KB per 64K GQA
        // workgroup) stage 1 was 0.2 us slower, so narrower rows keep plain
        // stores.  A store of more than 8 bytes still reads its data VGPRs
        // after issue, and the compiler, which sees only assembly here, may
        // write the next four outputs into the same registers at once: the
        // s_nop supplies the wait state the ISA requires before that write
        // (without it, an epilogue that reused the registers at once stored
        // the last four lanes of every 16 wrong).
        const f32x4_t ov = {o.x, o.y, o.z, o.w};
        asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(po), "v"(ov) : "memory");
        if (d == 0) asm volatile("global_store_dword %0, %1, off sc1" ::"v"(pl), "v"(lse) : "memory");
      } else {
        *(float4*)po = o;
        if (d == 0) *pl = lse;
      }
    }
  };

  if constexpr (KW == 1) {
    // The wave holds its rows' complete state: normalise and write.
    const bool empty = m == kNegInf;
    const float inv = empty ? 0.f : 1.f / l;
    const float lse = empty ? kNegInf : (m + __log2f(l)) * kLn2;
    if (p.out) {
      // Final bf16 output.  Lanes l and l + 16 hold the same row; for each
      // pair of 16-dim tiles they trade one 4-dim piece (even lane groups
      // keep tile dt, odd ones tile dt + 1), so that every lane stores 8
      // consecutive dims as one 16-byte write instead of two 8-byte ones
      // (prefill whole op: 4 x 2048 d128 101.0 -> 99.4 us, varlen d128
      // 76.1 -> 73.7).  The swap runs in every lane; a lane's partner shares
      // its row, so both or neither store.
      const int j = row_ok ? (int)fdiv((uint32_t)gr, p.fd_group) : 0;
      const int64_t row = ((int64_t)b * p.q_len + j) * p.num_q_heads + kvh * p.group + gr - j * p.group;
      const bool odd = g & 1;
#pragma unroll
      for (int dt = 0; dt < C::DT; dt += 2) {
        float a0 = __builtin_bit_cast(float, pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv));
        float a1 = __builtin_bit_cast(float, pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv));
        float b0 = __builtin_bit_cast(float, pack_bf16x2(acc[dt + 1][0] * inv, acc[dt + 1][1] * inv));
        float b1 = __builtin_bit_cast(float, pack_bf16x2(acc[dt + 1][2] * inv, acc[dt + 1][3] * inv));
        // Each swap trades an even lane's b for its odd partner's a: even
        // lanes end with tile dt's 8 dims, odd ones with tile dt + 1's.
        swap16(a0, b0);
        swap16(a1, b1);
        if (row_ok) {
          const int d = (odd ? dt + 1 : dt) * 16 + 4 * (g & ~1);
          uint4 v;
          v.x = __builtin_bit_cast(uint32_t, a0);
          v.y = __builtin_bit_cast(uint32_t, a1);
          v.z = __builtin_bit_cast(uint32_t, b0);
          v.w = __builtin_bit_cast(uint32_t, b1);
          *(uint4*)((uint16_t*)p.out + row * DV + d) = v;
        }
      }
      if (row_ok && g == 0 && p.lse_out) p.lse_out[row] = lse;
    } else if (row_ok) {
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
        write_row(gr, dt * 16 + 4 * g,
                  make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv), lse);
    }
  } else {
    // ---- wave state into LDS: acc^T [16 rows][RS], m[16], l[16] ----
    __syncthreads();  // the tiles are no longer read
    constexpr int RS = C::RS;
    float* pacc = (float*)(smem + wave * C::PART);
    float* pml = pacc + 16 * RS;
    // Lane l holds O^T[dims dt*16 + 4g + i][row n].
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
      *(float4*)(pacc + n * RS + dt * 16 + 4 * g) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
    if (g == 0) {
      pml[n] = m;
      pml[16 + n] = l;
    }
    __syncthreads();

    // ---- merge the KW streams of each row tile: thread -> (row, 4 dims) ----
    for (int idx = threadIdx.x; idx < RW * 16 * DV / 4; idx += 64 * C::NW) {
      const int rt = idx / (16 * DV / 4);
      const int r = (idx / (DV / 4)) % 16, d = (idx % (DV / 4)) * 4;
      const int grr = (tile * RW + rt) * 16 + r;
      if (grr >= p.rows_total) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < KW; ++w)
        M = fmaxf(M, ((const float*)(smem + (w * RW + rt) * C::PART))[16 * RS + r]);
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      float lse = kNegInf;
      if (M != kNegInf) {
        float den = 0.f;
        float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const float* base = (const float*)(smem + (w * RW + rt) * C::PART);
          const float f = fast_exp2(base[16 * RS + r] - M);
          den += f * base[16 * RS + 16 + r];
          const float4 a = *(const float4*)(base + r * RS + d);
          num.x += f * a.x;
          num.y += f * a.y;
          num.z += f * a.z;
          num.w += f * a.w;
        }
        const float inv = 1.f / den;
        o = make_float4(num.x * inv, num.y * inv, num.z * inv, num.w * inv);
        lse = (M + __log2f(den)) * kLn2;
      }
      write_row(grr, d, o, lse);
    }
  }

  // ---- In-kernel merge: the last workgroup of a row group merges it ----
  // Every workgroup of the group (same request, KV head and head tile; one
  // per split) releases its partials and counts itself in; the one that
  // brings the count to S reads all S partials back and merges them as
  // stage 2 would (weights e^(lse_s - max) / sum, natural log), then resets
  // the counter.  Nothing waits on another workgroup, so no ordering of the
  // grid can stall it.
  if (p.counters) {
    const uint32_t grp = ((uint32_t)b * p.num_kv_heads + kvh) * p.head_tiles + tile;
    const int S = p.num_splits;
    // Device-scope ordering costs an L2 write-back (release) and an L2
    // invalidation (acquire) on the issuing XCD, so one lane does each, once:
    // the barrier puts every lane's partial stores before lane 0's release
    // count, and only the merging workgroup acquires.
    __syncthreads();   // every lane's partials are stored; LDS is free
    volatile int* flag = (volatile int*)smem;
    if (threadIdx.x == 0) {
      const uint32_t prev = __hip_atomic_fetch_add(p.counters + grp, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      const int last = prev == (uint32_t)(S - 1);
      if (last) {
        __hip_atomic_store(p.counters + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other workgroups' partials, not stale lines
      }
      *flag = last;
    }
    __syncthreads();
    if (!*flag) return;

    const int nrows = last_row - first_row + 1;
    auto out_row = [&](int r) {
      const int grr = first_row + r;
      const int j = (int)fdiv((uint32_t)grr, p.fd_group);
      return ((int64_t)b * p.q_len + j) * p.num_q_heads + kvh * p.group + grr - j * p.group;
    };
    // Weights: one wave per row, lane s holds split s (S <= 64).
    float* wts = (float*)(smem + 256);   // [RW * 16][64]
    for (int r = wave; r < nrows; r += C::NW) {
      const int64_t row = out_row(r);
      const float x = lane < S ? p.lse_part[row * S + lane] : kNegInf;
      const float M = max_xor32(max_xor16(row16_max(x)));
      const float w = M == kNegInf ? 0.f : fast_exp2((x - M) * kLog2e);
      const float den = sum_xor32(sum_xor16(row16_sum(w)));
      wts[r * 64 + lane] = M == kNegInf ? 0.f : w * (1.f / den);
      if (lane == 0 && p.fin_lse) p.fin_lse[row] = M == kNegInf ? kNegInf : M + __logf(den);
    }
    __syncthreads();
    // Outputs: lane -> two (row, 4 dims) items at a time, eight splits of
    // each loaded before the first is used (16 loads in flight per lane).
    constexpr int T = 64 * C::NW, IT = 2;
    const int items = nrows * (DV / 4);
    for (int i0 = threadIdx.x; i0 < items; i0 += IT * T) {
      const float* src[IT];
      const float* wr[IT];
      int64_t orow[IT];
      float4 o[IT];
#pragma unroll
      for (int k = 0; k < IT; ++k) {
        const int idx = i0 + k * T < items ? i0 + k * T : i0;   // a spare item repeats the first
        const int r = idx / (DV / 4), c = idx - r * (DV / 4);
        orow[k] = out_row(r) * DV + c * 4;
        src[k] = p.o_part + out_row(r) * S * DV + c * 4;
        wr[k] = wts + r * 64;
        o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll 8
      for (int s2 = 0; s2 < S; ++s2) {
#pragma unroll
        for (int k = 0; k < IT; ++k) {
          const float wv = wr[k][s2];
          const float4 v = *(const float4*)(src[k] + (int64_t)s2 * DV);
          o[k].x = fmaf(wv, v.x, o[k].x);
          o[k].y = fmaf(wv, v.y, o[k].y);
          o[k].z = fmaf(wv, v.z, o[k].z);
          o[k].w = fmaf(wv, v.w, o[k].w);
        }
      }
#pragma unroll
      for (int k = 0; k < IT; ++k)
        if (i0 + k * T < items) store_out4(p.fin_out, 1, orow[k], o[k]);
    }
  }
}

}  // namespace

// One compiled shape of the kernel above.
struct MfmaEntry {
  int dk, dv;
  bool valias;
  int rw, kw;
  int min_rows;   // rows per KV head this shape needs
  void (*fn)(Stage1Params);
  int smem;       // LDS bytes per workgroup
};

template <int DK, int DV, bool VALIAS, int RW, int KW>
constexpr MfmaEntry mfma_entry(int min_rows) {
  return {DK, DV, VALIAS, RW, KW, min_rows, &stage1_mfma_kernel<DK, DV, VALIAS, RW, KW>,
          MCfg<DK, DV, VALIAS, RW, KW>::SMEM};
}

// The MLA latent-head shapes (576/512, V aliased), compiled in their own
// file: {pointer, count}.
const MfmaEntry* stage1_mfma_mla_table(int* count);

}  // namespace splitkv
