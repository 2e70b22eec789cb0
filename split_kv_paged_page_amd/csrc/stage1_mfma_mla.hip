// Matrix-core stage 1, MLA latent-head shapes (K 576 / V 512, V aliased to
// the first 512 dims of K).  Kept apart from stage1_mfma.hip so that it is
// compiled without the MFMA-results-in-VGPRs option (see there).
#include "stage1_mfma_kernel.h"

namespace splitkv {

namespace {

// In order of preference: the first entry whose min_rows the group reaches
// is used.
constexpr MfmaEntry kMla[] = {
    mfma_entry<576, 512, true, 4, 1>(64),
    mfma_entry<576, 512, true, 1, 4>(16),
    mfma_entry<576, 512, true, 1, 1>(1),
};

}  // namespace

const MfmaEntry* stage1_mfma_mla_table(int* count) {
  *count = (int)(sizeof(kMla) / sizeof(kMla[0]));
  return kMla;
}

}  // namespace splitkv
