// chunk_bf16.hip -- bf16 instantiations of the chunked EFLA kernels: the
// generic UT transform and recurrence (chunk_kernels.h) and the recurrence
// with one wavefront per state tile (recurrence_tile.h).
#include "chunk_kernels.h"
#include "recurrence_tile.h"

namespace efla {
template hipError_t launch_ut_transform<uint16_t>(const uint16_t*, const uint16_t*, uint16_t*, int, int,
                                                  int64_t, int, int, int, const int32_t*, int, hipStream_t, int32_t*);
template hipError_t launch_recurrence<uint16_t>(const uint16_t*, const uint16_t*, const uint16_t*,
                                                const uint16_t*, const float*, uint16_t*, float*, int,
                                                int, int64_t, int, int, int, int, const int32_t*, int,
                                                hipStream_t, int, const int32_t*);

bool recurrence_tile_supported(int DK, int C, int BV) { return tile_supported(DK, C, BV); }
hipError_t launch_recurrence_tile_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       hipStream_t s) {
  return launch_recurrence_tile(q, k, v, tws, s0, o, sfin, B, H, L, DK, DV, C, BV, s);
}
}  // namespace efla
