// launchers.h -- host-side launch functions of the EFLA kernels, one set per
// element type (float, or bf16 carried as uint16_t).  Each returns the HIP
// error of its launch; argument validation happens in the C ABI layer.
#pragma once

#include "common.h"

namespace efla {

template <typename T>
hipError_t launch_coeff(const T* k, const T* beta, float* lam, float* alpha, int64_t n, int DK,
                        hipStream_t s);

template <typename T>
hipError_t launch_step(const T* q, const T* k, const T* v, const T* beta, float* state, T* o,
                       int64_t units, int DK, int DV, hipStream_t s);

template <typename T>
hipError_t launch_ut_transform(const T* k, const T* beta, T* tws, int B, int H, int64_t L, int DK,
                               int C, hipStream_t stream);

template <typename T>
hipError_t launch_recurrence(const T* q, const T* k, const T* v, const T* tws, const float* s0,
                             T* o, float* sfin, int B, int H, int64_t L, int DK, int DV, int C,
                             int BV, hipStream_t stream);

}  // namespace efla
