// chunk_bf16_v7.hip -- bf16 instantiations of the recurrence with one chain
// wavefront per state tile (recurrence_v7.h), in a translation unit of its own so
// that the build compiles it in parallel with the others.
#include "launchers.h"
#include "recurrence_v7.h"

namespace efla {
bool recurrence_v7_supported(int DK, int C, int BV) { return v7_supported(DK, C, BV); }
hipError_t launch_recurrence_v7_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                     hipStream_t s) {
  return launch_recurrence_v7(q, k, v, tws, s0, o, sfin, B, H, L, DK, DV, C, BV, s);
}
}  // namespace efla
