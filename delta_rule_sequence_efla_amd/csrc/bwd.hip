// bwd.hip -- launches of the chunked backward pass (bwd_kernels.h), fp32 and
// bf16 inputs.  Workspace layout, every region 256-byte aligned, per chunk
// slot s of the dense batch ((b H + h) NC + n):
//   T  [slots][C][C]     input dtype   UT transform (as in the forward pass)
//   X  [slots][C][C]     fp32          (I + A)^{-1}
//   P  [slots][C][C]     fp32          tril(Q K^T) (bf16, packed from the
//                                      region's start, where the bf16
//                                      matrix-core kernels read it)
//   a  [slots][C]        fp32          coefficients
//   S  [slots][dk][dv]   input dtype   state at the start of the chunk (bf16
//                                      inputs: the operand values the forward
//                                      products use; [slots][dv][dk] where
//                                      the state-only kernel writes them)
//   dS [slots][dk][dv]   fp32          loss gradient at the end of the chunk
//                                      (bf16, packed from the region's start,
//                                      for the bf16 matrix-core kernels;
//                                      [slots][dv][dk] where the reverse pass
//                                      of recurrence_reverse.h writes it)
//   Qe [slots][C][dk]    bf16          Q - P T K (bf16 inputs only), read by
//                                      that reverse pass
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "bwd_bf16.h"
#include "bwd_kernels.h"
#include "chunk_kernels.h"
#include "launchers.h"
#include "ut_wave.h"

namespace efla {

namespace {
size_t align256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

BwdLayout bwd_layout(int B, int H, int64_t L, int DK, int DV, int C, size_t esz) {
  const int64_t NC = (L + C - 1) / C;
  const size_t slots = size_t(B) * H * NC;
  BwdLayout w{};
  w.t = 0;
  w.x = w.t + align256(slots * C * C * esz);
  w.p = w.x + align256(slots * C * C * 4);
  w.a = w.p + align256(slots * C * C * 4);
  w.s = w.a + align256(slots * C * 4);
  w.ds = w.s + align256(slots * size_t(DK) * DV * esz);
  w.qe = w.ds + align256(slots * size_t(DK) * DV * 4);
  w.total = w.qe + (esz == 2 ? align256(slots * size_t(C) * DK * 2) : 0);
  return w;
}

// The forward recurrence again, storing the state at the start of every chunk
// and no output.  With allow_t, where the state-only kernel covers the shape,
// that kernel writes the states transposed ([slots][DV][DK]) and *transposed
// is set; else the role kernel for the bf16 shapes it covers (its output and
// P wavefronts then idle), else the generic kernel, both [slots][DK][DV].
template <typename T, int DK, int C>
hipError_t chunk_states(const T* q, const T* k, const T* v, const T* tws, const float* s0, T* states, int B,
                        int H, int64_t L, int DV, hipStream_t s, bool allow_t = false, bool* transposed = nullptr) {
  if (transposed != nullptr) *transposed = false;
  if constexpr (sizeof(T) == 2) {
    const char* impl = getenv("EFLA_BWD_STATES");
    if (allow_t && !(impl && strcmp(impl, "roles") == 0) && recurrence_states_supported(DK, DV, C)) {
      *transposed = true;
      return launch_chunk_states_t_bf16(k, v, tws, s0, states, B, H, L, DK, DV, C, s);
    }
    const int bv = DV >= 32 ? 32 : 16;
    if (recurrence_roles_supported(DK, C, bv))
      return launch_recurrence_roles_bf16(q, k, v, tws, s0, nullptr, nullptr, B, H, L, DK, DV, C, bv, nullptr, 0, s,
                                          states);
  }
  const int NC = int((L + C - 1) / C), NVB = DV / 16;
  hipLaunchKernelGGL((recurrence_kernel<T, DK, C, 16>), dim3(unsigned(B * H * NVB)), dim3(kThreads), 0, s, q, k, v,
                     tws, s0, static_cast<T*>(nullptr), static_cast<float*>(nullptr), H, L, NC, DV, NVB, 0,
                     static_cast<const int32_t*>(nullptr), states);
  return hipGetLastError();
}

template <typename T, int DK, int C>
hipError_t bwd_launch_impl(const T* q, const T* k, const T* v, const T* beta, const float* s0, const T* dout,
                           const float* dsf, T* dq, T* dk, T* dv, T* dbeta, float* ds0, int B, int H, int64_t L,
                           int DV, int rule, unsigned char* ws, hipStream_t s, bool saved) {
  const int NC = int((L + C - 1) / C);
  const int BH = B * H;
  const int64_t slots = int64_t(BH) * NC;
  const BwdLayout lay = bwd_layout(B, H, L, DK, DV, C, sizeof(T));
  T* tws = reinterpret_cast<T*>(ws + lay.t);
  float* xws = reinterpret_cast<float*>(ws + lay.x);
  float* pws = reinterpret_cast<float*>(ws + lay.p);
  float* aws = reinterpret_cast<float*>(ws + lay.a);
  T* sws = reinterpret_cast<T*>(ws + lay.s);
  float* dsws = reinterpret_cast<float*>(ws + lay.ds);
  // bf16 matrix-core kernels for steps 3 and 4 where the shape allows
  // (EFLA_BWD_IMPL=fp32 keeps the fp32 ones); they read P as bf16, which the
  // one-wavefront UT kernel then writes (it covers every such shape)
  bool bf16k = false;
  if constexpr (sizeof(T) == 2 && (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64)) {
    const char* impl = getenv("EFLA_BWD_IMPL");
    bf16k = !(impl && strcmp(impl, "fp32") == 0) && bwd_bf16_supported(DK, DV, C);
  }
  const uint16_t* pws16 = reinterpret_cast<const uint16_t*>(pws);
  uint16_t* qews = reinterpret_cast<uint16_t*>(ws + lay.qe);
  // reverse pass in the form of the forward's state-only pass (its UT
  // instance writes Qe; EFLA_BWD_REVERSE=stager keeps the sixteen-wavefront
  // kernel)
  bool rev = false;
  if constexpr (sizeof(T) == 2) {
    const char* impl = getenv("EFLA_BWD_REVERSE");
    rev = bf16k && !(impl && strcmp(impl, "stager") == 0) && reverse_states_supported(DK, DV, C);
  }
  bool states_t = false;  // the chunk states are stored transposed
  // saved: the training forward left steps 1 and 2's results in the workspace
  // (T, X, a, bf16 P, Qe and the transposed chunk states), read only by the
  // bf16 matrix-core kernels; else both steps run here
  const bool from_fwd = saved && bf16k;
  if (from_fwd) states_t = true;
  if (slots > 0 && !from_fwd) {
    // 1. T, X, P and a of every chunk: one wavefront per chunk for the bf16
    // shapes that kernel covers (EFLA_UT_IMPL=workgroup keeps the other unless
    // the bf16 kernels follow), else one workgroup per chunk
    bool ut_done = false;
    if constexpr (sizeof(T) == 2 && (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64)) {
      const char* impl = getenv("EFLA_UT_IMPL");
      if (bf16k || !(impl && strcmp(impl, "workgroup") == 0)) {
        constexpr int NW = UtWaveShape<DK, C>::WAVES;
        const int64_t nwg = (slots + NW - 1) / NW;
        if (bf16k) {
          if (hipError_t e = launch_ut_wave_bwd_bf16(reinterpret_cast<const uint16_t*>(k),
                                                     reinterpret_cast<const uint16_t*>(beta),
                                                     reinterpret_cast<const uint16_t*>(q),
                                                     reinterpret_cast<uint16_t*>(tws), xws, aws, pws,
                                                     rev ? qews : nullptr, B, H, L, DK, C, rule, s);
              e != hipSuccess)
            return e;
        } else
          hipLaunchKernelGGL((ut_wave_kernel<DK, C, true>), dim3(unsigned(nwg)), dim3(64 * NW), 0, s, k, beta, tws,
                             H, L, NC, slots, rule, static_cast<const int32_t*>(nullptr), 0, nwg,
                             static_cast<int32_t*>(nullptr), q, xws, aws, pws);
        ut_done = true;
      }
    }
    if (!ut_done)
      hipLaunchKernelGGL((ut_transform_kernel<T, DK, C, true>), dim3(unsigned(slots)), dim3(kThreads), 0, s, k,
                         beta, tws, H, L, NC, rule, nullptr, 0, q, xws, aws, pws);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    // 2. the state at the start of every chunk (no output)
    if (hipError_t e = chunk_states<T, DK, C>(q, k, v, tws, s0, sws, B, H, L, DV, s, bf16k, &states_t);
        e != hipSuccess)
      return e;
  }
  // 3. reverse pass over chunks: dS at every chunk end, and dS_0 (bf16 inputs
  // on bf16 matrix cores where the shape allows, like step 4)
  bool state_done = false;
  if constexpr (sizeof(T) == 2 && DK % 32 == 0 && C % 32 == 0) {
    if (rev) {
      if (hipError_t e = launch_reverse_states_bf16(reinterpret_cast<const uint16_t*>(k), qews,
                                                    reinterpret_cast<const uint16_t*>(tws),
                                                    reinterpret_cast<const uint16_t*>(dout), dsf, ds0,
                                                    reinterpret_cast<uint16_t*>(dsws), B, H, L, DK, DV, C, s);
          e != hipSuccess)
        return e;
      state_done = true;
    } else if (bf16k) {
      hipLaunchKernelGGL((bwd_state_bf16_kernel<DK, C>), dim3(unsigned(BH * (DV / kBwdBV))),
                         dim3(BwdStateBf16Shape<DK, C>::NTH), 0, s,
                         q, k, dout, tws, pws16, dsf, reinterpret_cast<uint16_t*>(dsws), ds0, H, L, NC, DV,
                         DV / kBwdBV, BH % 8 == 0 ? 1 : 0);
      state_done = true;
    }
  }
  if (!state_done)
    hipLaunchKernelGGL((bwd_state_kernel<T, DK, C>), dim3(unsigned(BH * (DV / 16))), dim3(kThreads), 0, s, q, k,
                       dout, tws, pws, dsf, dsws, ds0, H, L, NC, DV, DV / 16);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (slots == 0) return hipSuccess;
  // 4. every chunk's gradients: bf16 inputs on bf16 matrix cores where the
  // shape allows (EFLA_BWD_IMPL=fp32 keeps the fp32 kernel), else fp32
  if constexpr (sizeof(T) == 2 && DK % 32 == 0 && C % 32 == 0) {
    if (bf16k) {
      const auto* ds16 = reinterpret_cast<const uint16_t*>(dsws);
      // the two-workgroup kernel where both state arrays are transposed
      // (EFLA_BWD_CHUNK=stager keeps the one-workgroup kernel)
      const char* cimpl = getenv("EFLA_BWD_CHUNK");
      if (states_t && rev && !(cimpl && strcmp(cimpl, "stager") == 0) && bwd_chunk_tr_bf16_supported(DK, DV, C))
        return launch_bwd_chunk_tr_bf16(reinterpret_cast<const uint16_t*>(q), reinterpret_cast<const uint16_t*>(k),
                                        reinterpret_cast<const uint16_t*>(v), reinterpret_cast<const uint16_t*>(beta),
                                        reinterpret_cast<const uint16_t*>(dout), reinterpret_cast<const uint16_t*>(tws),
                                        xws, aws, pws16, reinterpret_cast<const uint16_t*>(sws), ds16,
                                        reinterpret_cast<uint16_t*>(dq), reinterpret_cast<uint16_t*>(dk),
                                        reinterpret_cast<uint16_t*>(dv), reinterpret_cast<uint16_t*>(dbeta), B, H, L,
                                        DK, DV, C, rule, s);
      auto chunk = [&](auto stt, auto dstt) {
        hipLaunchKernelGGL((bwd_chunk_bf16_kernel<DK, C, decltype(stt)::value, decltype(dstt)::value>),
                           dim3(unsigned(slots)), dim3(BwdBf16Shape<DK, C>::NTH), 0, s, q, k, v, beta, dout, tws, xws,
                           aws, pws16, sws, ds16, dq, dk, dv, dbeta, H, L, NC, DV, rule);
      };
      using Y = std::true_type;
      using N = std::false_type;
      if (states_t && rev) chunk(Y{}, Y{});
      else if (states_t) chunk(Y{}, N{});
      else if (rev) chunk(N{}, Y{});
      else chunk(N{}, N{});
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((bwd_chunk_kernel<T, DK, C>), dim3(unsigned(slots)), dim3(kThreads), 0, s, q, k, v, beta,
                     dout, tws, xws, aws, pws, sws, dsws, dq, dk, dv, dbeta, H, L, NC, DV, rule);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t bwd_dispatch_c(const T* q, const T* k, const T* v, const T* beta, const float* s0, const T* dout,
                          const float* dsf, T* dq, T* dk, T* dv, T* dbeta, float* ds0, int B, int H, int64_t L,
                          int DV, int C, int rule, unsigned char* ws, hipStream_t s, bool saved) {
  switch (C) {
    case 16: return bwd_launch_impl<T, DK, 16>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, rule, ws, s, saved);
    case 32: return bwd_launch_impl<T, DK, 32>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, rule, ws, s, saved);
    case 64: return bwd_launch_impl<T, DK, 64>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, rule, ws, s, saved);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_chunk_bwd(const T* q, const T* k, const T* v, const T* beta, const float* s0, const T* dout,
                            const float* dsf, T* dq, T* dk, T* dv, T* dbeta, float* ds0, int B, int H, int64_t L,
                            int DK, int DV, int C, int rule, void* ws, hipStream_t s, bool saved) {
  auto* w = static_cast<unsigned char*>(ws);
  switch (DK) {
    case 16: return bwd_dispatch_c<T, 16>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, C, rule, w, s, saved);
    case 32: return bwd_dispatch_c<T, 32>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, C, rule, w, s, saved);
    case 64: return bwd_dispatch_c<T, 64>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, C, rule, w, s, saved);
    case 128: return bwd_dispatch_c<T, 128>(q, k, v, beta, s0, dout, dsf, dq, dk, dv, dbeta, ds0, B, H, L, DV, C, rule, w, s, saved);
  }
  return hipErrorInvalidValue;
}

template hipError_t launch_chunk_bwd<float>(const float*, const float*, const float*, const float*, const float*,
                                            const float*, const float*, float*, float*, float*, float*, float*, int,
                                            int, int64_t, int, int, int, int, void*, hipStream_t, bool);
template hipError_t launch_chunk_bwd<uint16_t>(const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                               const float*, const uint16_t*, const float*, uint16_t*, uint16_t*,
                                               uint16_t*, uint16_t*, float*, int, int, int64_t, int, int, int, int,
                                               void*, hipStream_t, bool);

bool train_saves_states(int DK, int DV, int C) {
  return recurrence_split_supported(DK, C, 32) && DV % 32 == 0 && bwd_bf16_supported(DK, DV, C);
}

}  // namespace efla
