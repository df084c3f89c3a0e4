// chunk_bf16_v6.hip -- bf16 instantiations of the one-role-per-wavefront
// recurrence (recurrence_v6.h), in a translation unit of its own so that the
// build compiles it in parallel with the others.
#include "launchers.h"
#include "recurrence_v6.h"

namespace efla {
bool recurrence_v6_supported(int DK, int C, int BV) { return v6_supported(DK, C, BV); }
hipError_t launch_recurrence_v6_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                     hipStream_t s) {
  return launch_recurrence_v6(q, k, v, tws, s0, o, sfin, B, H, L, DK, DV, C, BV, s);
}
}  // namespace efla
