// chunk_bf16_states.hip -- bf16 instantiations of the state-only pass of the
// segment scan and of the backward (recurrence_states.h) and of the
// backward's reverse pass (recurrence_reverse.h), in a translation unit of
// their own.
#include "launchers.h"
#include "recurrence_reverse.h"
#include "recurrence_states.h"

namespace efla {
bool recurrence_states_supported(int DK, int DV, int C) { return states_supported(DK, C, 32) && DV % 32 == 0; }
hipError_t launch_recurrence_states_bf16(const uint16_t* k, const uint16_t* v, const uint16_t* tws, float* nout,
                                         float* mout, int B, int H, int64_t L, int DK, int DV, int C,
                                         const int32_t* cu, int N, hipStream_t s) {
  if (!recurrence_states_supported(DK, DV, C)) return hipErrorInvalidValue;
  if (DK == 64)
    return recurrence_states_launch_impl<64, 64, 32, false>(k, v, tws, nout, mout, B, H, L, DV, cu, N, nullptr,
                                                            nullptr, s);
  return recurrence_states_launch_impl<128, 64, 32, false>(k, v, tws, nout, mout, B, H, L, DV, cu, N, nullptr,
                                                           nullptr, s);
}
hipError_t launch_chunk_states_t_bf16(const uint16_t* k, const uint16_t* v, const uint16_t* tws, const float* s0,
                                      uint16_t* statesT, int B, int H, int64_t L, int DK, int DV, int C,
                                      hipStream_t s) {
  if (!recurrence_states_supported(DK, DV, C)) return hipErrorInvalidValue;
  if (DK == 64)
    return recurrence_states_launch_impl<64, 64, 32, true>(k, v, tws, nullptr, nullptr, B, H, L, DV, nullptr, 0, s0,
                                                           statesT, s);
  return recurrence_states_launch_impl<128, 64, 32, true>(k, v, tws, nullptr, nullptr, B, H, L, DV, nullptr, 0, s0,
                                                          statesT, s);
}
bool reverse_states_supported(int DK, int DV, int C) { return reverse_supported(DK, DV, C); }
hipError_t launch_reverse_states_bf16(const uint16_t* k, const uint16_t* qe, const uint16_t* tws,
                                      const uint16_t* dout, const float* dsf, float* ds0, uint16_t* dstatesT, int B,
                                      int H, int64_t L, int DK, int DV, int C, hipStream_t s) {
  if (!reverse_supported(DK, DV, C)) return hipErrorInvalidValue;
  if (DK == 64)
    return reverse_states_launch_impl<64, 64, 32>(k, qe, tws, dout, dsf, ds0, dstatesT, B, H, L, DV, s);
  return reverse_states_launch_impl<128, 64, 32>(k, qe, tws, dout, dsf, ds0, dstatesT, B, H, L, DV, s);
}
}  // namespace efla
