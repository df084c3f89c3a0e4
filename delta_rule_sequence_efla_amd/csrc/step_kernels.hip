// step_kernels.hip -- decode step and standalone coefficient kernels (gfx950).
//
// Decode applies the update rule of the pages' Method step 3 to one token per
// (n, h):  S <- (I - a k k^T) S + a k v^T,  o = S^T q.  Written as
//     r = S^T k,  p = S^T q,  u = v - r,  S <- S + a k u^T,  o = p + a (k.q) u
// it reads and writes each fp32 state exactly once, which is the whole cost
// (the step is bound by HBM bandwidth: 2 * 4 * d_k * d_v bytes per head).
#include "launchers.h"

namespace efla {

// One workgroup per (n, h).  Thread (rg, cq) owns value columns 4cq..4cq+3 of
// rows rg, rg + NRG, ...; the two column reductions go through LDS.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void step_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v,
                                                        const T* __restrict__ beta,
                                                        float* __restrict__ state, T* __restrict__ o,
                                                        int rule) {
  constexpr int NCQ = DV / 4;
  constexpr int NRG = kThreads / NCQ;
  constexpr int RPT = cdiv(DK, NRG);
  __shared__ float ks[DK], qs[DK], us[DV];
  __shared__ __align__(16) float red_k[NRG * DV];
  __shared__ __align__(16) float red_q[NRG * DV];
  __shared__ float coef[2];

  const int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  const int cq = tid % NCQ, rg = tid / NCQ;
  float* Su = state + u * DK * DV;

  f32x4 S[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * NRG;
    S[i] = (r < DK) ? *reinterpret_cast<const f32x4*>(Su + r * DV + 4 * cq) : zero4();
  }
  if (tid < DK) {
    ks[tid] = to_f32(k[u * DK + tid]);
    qs[tid] = to_f32(q[u * DK + tid]);
  }
  __syncthreads();

  if (tid < kWave) {
    float lam = 0.0f, kq = 0.0f;
    for (int d = tid; d < DK; d += kWave) {
      lam = fmaf(ks[d], ks[d], lam);
      kq = fmaf(ks[d], qs[d], kq);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lam += __shfl_xor(lam, off);
      kq += __shfl_xor(kq, off);
    }
    if (tid == 0) {
      const float a = efla_alpha_rule(to_f32(beta[u]), lam, rule);
      coef[0] = a;
      coef[1] = a * kq;
    }
  }

  f32x4 pk = zero4(), pq = zero4();
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * NRG;
    if (r < DK) {
      pk += ks[r] * S[i];
      pq += qs[r] * S[i];
    }
  }
  *reinterpret_cast<f32x4*>(red_k + rg * DV + 4 * cq) = pk;
  *reinterpret_cast<f32x4*>(red_q + rg * DV + 4 * cq) = pq;
  __syncthreads();

  if (tid < DV) {
    float rk = 0.0f, rq = 0.0f;
    for (int p = 0; p < NRG; ++p) {
      rk += red_k[p * DV + tid];
      rq += red_q[p * DV + tid];
    }
    const float uu = to_f32(v[u * DV + tid]) - rk;
    us[tid] = uu;
    o[u * DV + tid] = from_f32<T>(rq + coef[1] * uu);
  }
  __syncthreads();

  const float a = coef[0];
  const f32x4 uq = *reinterpret_cast<const f32x4*>(us + 4 * cq);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + i * NRG;
    if (r < DK) *reinterpret_cast<f32x4*>(Su + r * DV + 4 * cq) = S[i] + (a * ks[r]) * uq;
  }
}

// lambda = ||k||^2 (sequential fp32 fma over the key dims) and alpha per row.
template <typename T, int DK>
__global__ __launch_bounds__(kThreads) void coeff_kernel(const T* __restrict__ k, const T* __restrict__ beta,
                                                         float* __restrict__ lam_out,
                                                         float* __restrict__ alpha, int64_t n, int rule) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= n) return;
  const T* kt = k + t * DK;
  float lam = 0.0f;
  for (int d = 0; d < DK; ++d) {
    const float x = to_f32(kt[d]);
    lam = fmaf(x, x, lam);
  }
  if (lam_out != nullptr) lam_out[t] = lam;
  alpha[t] = efla_alpha_rule(to_f32(beta[t]), lam, rule);
}

template <typename T, int DK, int DV>
static hipError_t step_impl(const T* q, const T* k, const T* v, const T* beta, float* state, T* o,
                            int64_t units, int rule, hipStream_t s) {
  hipLaunchKernelGGL((step_kernel<T, DK, DV>), dim3(unsigned(units)), dim3(kThreads), 0, s, q, k, v,
                     beta, state, o, rule);
  return hipGetLastError();
}

template <typename T, int DK>
static hipError_t step_dv(const T* q, const T* k, const T* v, const T* beta, float* state, T* o,
                          int64_t units, int DV, int rule, hipStream_t s) {
  switch (DV) {
    case 16: return step_impl<T, DK, 16>(q, k, v, beta, state, o, units, rule, s);
    case 32: return step_impl<T, DK, 32>(q, k, v, beta, state, o, units, rule, s);
    case 64: return step_impl<T, DK, 64>(q, k, v, beta, state, o, units, rule, s);
    case 128: return step_impl<T, DK, 128>(q, k, v, beta, state, o, units, rule, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_step(const T* q, const T* k, const T* v, const T* beta, float* state, T* o,
                       int64_t units, int DK, int DV, int rule, hipStream_t s) {
  if (units == 0) return hipSuccess;
  switch (DK) {
    case 16: return step_dv<T, 16>(q, k, v, beta, state, o, units, DV, rule, s);
    case 32: return step_dv<T, 32>(q, k, v, beta, state, o, units, DV, rule, s);
    case 64: return step_dv<T, 64>(q, k, v, beta, state, o, units, DV, rule, s);
    case 128: return step_dv<T, 128>(q, k, v, beta, state, o, units, DV, rule, s);
  }
  return hipErrorInvalidValue;
}

template <typename T, int DK>
static hipError_t coeff_impl(const T* k, const T* beta, float* lam, float* alpha, int64_t n, int rule,
                             hipStream_t s) {
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL((coeff_kernel<T, DK>), dim3(unsigned(blocks)), dim3(kThreads), 0, s, k, beta, lam,
                     alpha, n, rule);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_coeff(const T* k, const T* beta, float* lam, float* alpha, int64_t n, int DK, int rule,
                        hipStream_t s) {
  if (n == 0) return hipSuccess;
  switch (DK) {
    case 16: return coeff_impl<T, 16>(k, beta, lam, alpha, n, rule, s);
    case 32: return coeff_impl<T, 32>(k, beta, lam, alpha, n, rule, s);
    case 64: return coeff_impl<T, 64>(k, beta, lam, alpha, n, rule, s);
    case 128: return coeff_impl<T, 128>(k, beta, lam, alpha, n, rule, s);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_step<float>(const float*, const float*, const float*, const float*, float*,
                                       float*, int64_t, int, int, int, hipStream_t);
template hipError_t launch_step<uint16_t>(const uint16_t*, const uint16_t*, const uint16_t*,
                                          const uint16_t*, float*, uint16_t*, int64_t, int, int, int,
                                          hipStream_t);
template hipError_t launch_coeff<float>(const float*, const float*, float*, float*, int64_t, int, int,
                                        hipStream_t);
template hipError_t launch_coeff<uint16_t>(const uint16_t*, const uint16_t*, float*, float*, int64_t,
                                           int, int, hipStream_t);

}  // namespace efla
