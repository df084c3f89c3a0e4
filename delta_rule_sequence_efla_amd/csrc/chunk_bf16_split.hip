// chunk_bf16_split.hip -- bf16 instantiations of the recurrence with each
// chunk's work spread over nine wavefronts (recurrence_split.h), in a
// translation unit of its own so that it builds in parallel with the others.
#include "launchers.h"
#include "recurrence_split.h"

namespace efla {
bool recurrence_split_supported(int DK, int C, int BV) { return split_supported(DK, C, BV); }
hipError_t launch_recurrence_split_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                        int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                        const int32_t* cu, int N, const int32_t* order, hipStream_t s) {
  return launch_recurrence_split(q, k, v, tws, s0, o, sfin, B, H, L, DK, DV, C, BV, cu, N, order, s);
}
}  // namespace efla
