// chunk_f32.hip -- fp32 instantiations of the chunked EFLA kernels.
#include "chunk_kernels.h"

namespace efla {
template hipError_t launch_ut_transform<float>(const float*, const float*, float*, int, int, int64_t,
                                               int, int, int, const int32_t*, int, hipStream_t, int32_t*);
template hipError_t launch_recurrence<float>(const float*, const float*, const float*, const float*,
                                             const float*, float*, float*, int, int, int64_t, int, int,
                                             int, int, const int32_t*, int, hipStream_t, int, const int32_t*);
}  // namespace efla
