// chunk_bf16.hip -- bf16 instantiations of the chunked EFLA kernels.
#include "chunk_kernels.h"

namespace efla {
template hipError_t launch_ut_transform<uint16_t>(const uint16_t*, const uint16_t*, uint16_t*, int, int,
                                                  int64_t, int, int, hipStream_t);
template hipError_t launch_recurrence<uint16_t>(const uint16_t*, const uint16_t*, const uint16_t*,
                                                const uint16_t*, const float*, uint16_t*, float*, int,
                                                int, int64_t, int, int, int, int, hipStream_t);
}  // namespace efla
