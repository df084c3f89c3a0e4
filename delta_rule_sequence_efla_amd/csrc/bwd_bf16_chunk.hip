// bwd_bf16_chunk.hip -- the two-workgroup per-chunk backward kernel
// (bwd_chunk_tr.h), in a translation unit built with VGPR-form accumulators.
#include "bwd_chunk_tr.h"
#include "launchers.h"

namespace efla {
bool bwd_chunk_tr_bf16_supported(int DK, int DV, int C) { return bwd_chunk_tr_supported(DK, DV, C); }
hipError_t launch_bwd_chunk_tr_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* beta,
                                    const uint16_t* dout, const uint16_t* tws, const float* xws, const float* aws,
                                    const uint16_t* pws, const uint16_t* statesT, const uint16_t* dstatesT,
                                    uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbeta, int B, int H, int64_t L,
                                    int DK, int DV, int C, int rule, hipStream_t s) {
  if (!bwd_chunk_tr_supported(DK, DV, C)) return hipErrorInvalidValue;
  const int NC = int((L + C - 1) / C);
  const int64_t slots = int64_t(B) * H * NC;
  if (slots == 0) return hipSuccess;
  if (DK == 64)
    hipLaunchKernelGGL((bwd_chunk_tr_kernel<64, 64>), dim3(unsigned(slots)), dim3(BwdTrShape<64, 64>::NTH), 0, s, q, k,
                       v, beta, dout, tws, xws, aws, pws, statesT, dstatesT, dq, dk, dv, dbeta, H, L, NC, DV, rule);
  else
    hipLaunchKernelGGL((bwd_chunk_tr_kernel<128, 64>), dim3(unsigned(slots)), dim3(BwdTrShape<128, 64>::NTH), 0, s, q,
                       k, v, beta, dout, tws, xws, aws, pws, statesT, dstatesT, dq, dk, dv, dbeta, H, L, NC, DV, rule);
  return hipGetLastError();
}
}  // namespace efla
