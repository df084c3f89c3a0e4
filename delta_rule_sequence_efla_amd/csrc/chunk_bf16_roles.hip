// chunk_bf16_roles.hip -- bf16 instantiations of the recurrence with one role
// per wavefront (recurrence_roles.h), in a translation unit of its own so that
// the build compiles it in parallel with the others.
#include "launchers.h"
#include "recurrence_roles.h"

namespace efla {
bool recurrence_roles_supported(int DK, int C, int BV) { return roles_supported(DK, C, BV); }
hipError_t launch_recurrence_roles_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                        int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                        const int32_t* cu, int N, hipStream_t s, uint16_t* states, bool trans,
                                        const int32_t* order) {
  return launch_recurrence_roles(q, k, v, tws, s0, o, sfin, B, H, L, DK, DV, C, BV, cu, N, states, trans, order, s);
}
}  // namespace efla
