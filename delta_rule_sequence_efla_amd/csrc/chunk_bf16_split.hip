// chunk_bf16_split.hip -- bf16 instantiations of the recurrence with each
// chunk's work spread over nine wavefronts (recurrence_split.h), in a
// translation unit of its own so that it builds in parallel with the others.
#include <stdlib.h>

#include "launchers.h"
#include "recurrence_split.h"

namespace efla {
constexpr int kSplitDmaWaves = 1;
bool recurrence_split_supported(int DK, int C, int BV) { return split_supported(DK, C, BV); }
hipError_t launch_recurrence_split_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                        int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                        const int32_t* cu, int N, const int32_t* order, hipStream_t s,
                                        uint16_t* statesT) {
  // EFLA_SPLIT_DMA=1|2 sets the number of DMA wavefronts (for comparisons;
  // two share each chunk's transfers by tile, which measured slower with the
  // caches flushed and the same with them warm)
  const char* env = getenv("EFLA_SPLIT_DMA");
  const int ndma = (env && atoi(env) == 1) ? 1 : (env && atoi(env) == 2) ? 2 : kSplitDmaWaves;
  return launch_recurrence_split(q, k, v, tws, s0, o, sfin, B, H, L, DK, DV, C, BV, cu, N, order, ndma, s, statesT);
}
}  // namespace efla
