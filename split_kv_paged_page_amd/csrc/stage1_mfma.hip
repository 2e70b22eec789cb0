// Matrix-core stage 1 of split-KV paged decode: the shape table and the
// launchers.  The kernel itself is in stage1_mfma_kernel.h.  This file holds
// the shapes at head dims 64, 128 and 256 and is compiled with the compiler
// option that puts MFMA results in ordinary VGPRs instead of AGPRs (no AGPR
// to VGPR copies of the scores; measured, stage 1: prefill 4 x 2048 d128
// 139.6 -> 136.1 us, d64 98.4 -> 96.8, drafts 13.96 -> 13.59, 64K GQA
// 15.92 -> 15.80).  The MLA shapes (576/512) are in stage1_mfma_mla.hip,
// compiled without it: their 128 accumulator registers per lane do not fit
// beside the rest in VGPRs, and the mixed form was slower (wide MLA stage 1
// 386.7 -> 389.0 us).
#include "stage1_mfma_kernel.h"

namespace splitkv {

namespace {

// Per head-dim pair, in order of preference: the first entry whose min_rows
// the group reaches is used.
constexpr MfmaEntry kTable[] = {
    mfma_entry<256, 256, false, 2, 1>(32),
    mfma_entry<256, 256, false, 1, 4>(16),
    mfma_entry<256, 256, false, 1, 1>(1),
    // 128+ rows (prefill): each block in LDS serves twice the rows of the
    // four-tile shape, which halves the key reads per row out of the L2;
    // prefill 4 x 2048 stage 1 90.0 -> 87.5 us, varlen 67.4 -> 63.0.  With
    // a ring of 2 tiles it was no faster (88.0, 68.7).
    mfma_entry<128, 128, false, 8, 1>(128),
    mfma_entry<128, 128, false, 4, 1>(64),
    mfma_entry<128, 128, false, 1, 4>(16),
    mfma_entry<128, 128, false, 1, 1>(1),
    mfma_entry<64, 64, false, 4, 1>(64),
    mfma_entry<64, 64, false, 1, 4>(16),
    mfma_entry<64, 64, false, 1, 1>(1),
};

// Calls f(entry) for every shape, MLA first, until f returns true.
template <class F>
const MfmaEntry* find_entry(F&& f) {
  int n = 0;
  const MfmaEntry* mla = stage1_mfma_mla_table(&n);
  for (int i = 0; i < n; ++i)
    if (f(mla[i])) return &mla[i];
  for (const MfmaEntry& e : kTable)
    if (f(e)) return &e;
  return nullptr;
}

}  // namespace

MfmaShape stage1_mfma_shape(int dtype, int dk, int dv, bool v_aliases_k, int rows, bool streams) {
  if (dtype != 1) return MfmaShape{0, 0, 0};
  const MfmaEntry* e = find_entry([&](const MfmaEntry& x) {
    return x.dk == dk && x.dv == dv && x.valias == v_aliases_k && rows >= x.min_rows && (streams || x.kw == 1);
  });
  return e ? MfmaShape{e->rw, e->kw, e->smem} : MfmaShape{0, 0, 0};
}

hipError_t launch_stage1_mfma(const Stage1Params& p, int dk, int dv, bool v_aliases_k, MfmaShape sh,
                              hipStream_t st) {
  const MfmaEntry* e = find_entry([&](const MfmaEntry& x) {
    return x.dk == dk && x.dv == dv && x.valias == v_aliases_k && x.rw == sh.rw && x.kw == sh.kw;
  });
  if (!e) return hipErrorInvalidValue;
  hipLaunchKernelGGL(e->fn, dim3(p.num_wgs), dim3(64 * e->rw * e->kw), 0, st, p);
  return hipGetLastError();
}

}  // namespace splitkv
