// ut_bf16.hip -- bf16 instantiations of the one-wavefront-per-chunk UT
// transform (ut_wave.h): the forward's and the backward's with bf16 P.
#include "launchers.h"
#include "ut_wave.h"

namespace efla {
bool ut_wave_bf16_supported(int DK, int C) { return ut_wave_supported(DK, C); }
hipError_t launch_ut_wave_bf16(const uint16_t* k, const uint16_t* beta, uint16_t* tws, int B, int H, int64_t L,
                               int DK, int C, int rule, const int32_t* cu, int N, hipStream_t s, int32_t* order) {
  return launch_ut_wave(k, beta, tws, B, H, L, DK, C, rule, cu, N, order, s);
}

namespace {
template <int DK, int C>
hipError_t ut_bwd_impl(const uint16_t* k, const uint16_t* beta, const uint16_t* q, uint16_t* tws, float* xws,
                       float* aws, float* pws, uint16_t* qe, int B, int H, int64_t L, int rule, hipStream_t s,
                       bool t_plain) {
  constexpr int NW = UtWaveShape<DK, C>::WAVES;
  const int NC = int((L + C - 1) / C);
  const int64_t slots = int64_t(B) * H * NC, nwg = (slots + NW - 1) / NW;
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL((ut_wave_kernel<DK, C, true, true>), dim3(unsigned(nwg)), dim3(64 * NW), 0, s, k, beta, tws, H, L,
                     NC, slots, rule, static_cast<const int32_t*>(nullptr), 0, nwg, static_cast<int32_t*>(nullptr), q,
                     xws, aws, pws, qe, t_plain ? 1 : 0);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_ut_wave_bwd_bf16(const uint16_t* k, const uint16_t* beta, const uint16_t* q, uint16_t* tws,
                                   float* xws, float* aws, float* pws, uint16_t* qe, int B, int H, int64_t L, int DK,
                                   int C, int rule, hipStream_t s, bool t_plain) {
  if (C == 32) {
    switch (DK) {
      case 32: return ut_bwd_impl<32, 32>(k, beta, q, tws, xws, aws, pws, qe, B, H, L, rule, s, t_plain);
      case 64: return ut_bwd_impl<64, 32>(k, beta, q, tws, xws, aws, pws, qe, B, H, L, rule, s, t_plain);
      case 128: return ut_bwd_impl<128, 32>(k, beta, q, tws, xws, aws, pws, qe, B, H, L, rule, s, t_plain);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return ut_bwd_impl<32, 64>(k, beta, q, tws, xws, aws, pws, qe, B, H, L, rule, s, t_plain);
      case 64: return ut_bwd_impl<64, 64>(k, beta, q, tws, xws, aws, pws, qe, B, H, L, rule, s, t_plain);
      case 128: return ut_bwd_impl<128, 64>(k, beta, q, tws, xws, aws, pws, qe, B, H, L, rule, s, t_plain);
    }
  }
  return hipErrorInvalidValue;
}
}  // namespace efla
