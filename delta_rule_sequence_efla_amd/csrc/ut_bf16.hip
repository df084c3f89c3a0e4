// ut_bf16.hip -- bf16 instantiations of the one-wavefront-per-chunk UT
// transform (ut_wave.h).
#include "launchers.h"
#include "ut_wave.h"

namespace efla {
bool ut_wave_bf16_supported(int DK, int C) { return ut_wave_supported(DK, C); }
hipError_t launch_ut_wave_bf16(const uint16_t* k, const uint16_t* beta, uint16_t* tws, int B, int H, int64_t L,
                               int DK, int C, int rule, const int32_t* cu, int N, hipStream_t s, int32_t* order) {
  return launch_ut_wave(k, beta, tws, B, H, L, DK, C, rule, cu, N, order, s);
}
}  // namespace efla
