// seg.hip -- the intra-GPU segment scan for batches of few long sequences.
//
// The state recurrence is affine in the state: over a run of chunks,
//     S_out = M S_in + N,   M = prod over the chunks of (I - K^T T K),
// N = the state the run reaches from zero.  So each sequence of a dense batch
// [B, L, H, d] is cut into G segments that run in parallel as sequences of a
// packed batch (see SeqSpan): one pass gives every segment's N (true V, zero
// start), one its M (V = 0, identity start, d_k "value" columns), this file's
// combine kernel chains S_in(g+1) = M_g S_in(g) + N_g along each sequence,
// and a last pass reruns every segment from its true incoming state with
// output.  That is three passes of the work instead of one, spread over G
// times as many workgroups, for batches with too few (b, h) to fill the GPU.
#include "bwd_kernels.h"
#include "launchers.h"

namespace efla {

// Offsets of the packed view: segment g of sequence b is tokens
// b L + g Ls .. b L + min((g+1) Ls, L) - 1.
__global__ void seg_offsets_kernel(int32_t* cu, int B, int G, int64_t L, int64_t Ls) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i > B * G) return;
  const int b = i / G, g = i % G;
  const int64_t off = (i == B * G) ? int64_t(B) * L : int64_t(b) * L + (int64_t(g) * Ls < L ? int64_t(g) * Ls : L);
  cu[i] = int32_t(off);
}

// One workgroup per (b, h, 16 value columns): S (d_k x 16, fp32, LDS) runs
// along the segments of sequence b,
//     sin[u] = S;   S = M[u] S + N[u],   u = b G + g,
// and ends in sfin[b, h] (NULL: not written).  M [U, H, d_k, d_k], N and sin
// [U, H, d_k, d_v], fp32.
template <int DK>
__global__ __launch_bounds__(kThreads) void seg_combine_kernel(const float* __restrict__ M,
                                                               const float* __restrict__ Nf,
                                                               const float* s0,
                                                               float* __restrict__ sin, float* sfin,
                                                               int H, int G, int DV) {
  constexpr int DKP = round_up(DK, 32), MP = DKP + 4, VP = 16 + 4;
  __shared__ __align__(16) float Ms[DKP * MP];
  __shared__ __align__(16) float Ss[DKP * VP];
  const int nvb = DV / 16, x = blockIdx.x, bh = x / nvb, v0 = 16 * (x % nvb);
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  for (int i = tid; i < DKP * MP; i += kThreads) Ms[i] = 0.0f;
  for (int i = tid; i < DKP * 16; i += kThreads) {
    const int d = i / 16, c = i % 16;
    Ss[d * VP + c] = (s0 != nullptr && d < DK) ? s0[(int64_t(bh) * DK + d) * DV + v0 + c] : 0.0f;
  }
  __syncthreads();
  for (int gi = 0; gi < G; ++gi) {
    const int64_t u = int64_t(b) * G + gi;
    const float* Mu = M + (u * H + h) * DK * DK;
    const float* Nu = Nf + (u * H + h) * DK * DV;
    float* su = sin + (u * H + h) * DK * DV;
    for (int i = tid; i < DK * 16; i += kThreads) {
      const int d = i / 16, c = i % 16;
      su[d * DV + v0 + c] = Ss[d * VP + c];
    }
    for (int i = tid; i < DK * DK; i += kThreads) Ms[(i / DK) * MP + i % DK] = Mu[i];
    __syncthreads();
    f32x4 acc[DKP / 64 > 0 ? DKP / 64 : 1];
    int nt = 0;
    for (int dt = w; dt < DKP / 16; dt += 4, ++nt) {
      acc[nt] = zero4();
      tile_mma16<false, false>(acc[nt], Ms, MP, Ss, VP, 16 * dt, 0, DKP, li, g);
    }
    __syncthreads();  // every wave has read S
    nt = 0;
    for (int dt = w; dt < DKP / 16; dt += 4, ++nt) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 16 * dt + 4 * g + qq;
        Ss[d * VP + li] = d < DK ? acc[nt][qq] + Nu[d * DV + v0 + li] : 0.0f;
      }
    }
    __syncthreads();
  }
  if (sfin != nullptr) {
    for (int i = tid; i < DK * 16; i += kThreads) {
      const int d = i / 16, c = i % 16;
      sfin[(int64_t(bh) * DK + d) * DV + v0 + c] = Ss[d * VP + c];
    }
  }
}

hipError_t launch_seg_offsets(int32_t* cu, int B, int G, int64_t L, int64_t Ls, hipStream_t s) {
  const int n = B * G + 1;
  hipLaunchKernelGGL(seg_offsets_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, cu, B, G, L, Ls);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const float* M, const float* N, const float* s0, float* sin, float* sfin, int B, int H,
                              int G, int DK, int DV, hipStream_t s) {
  const dim3 grid{unsigned(B * H * (DV / 16))}, block{unsigned(kThreads)};
  switch (DK) {
    case 16: hipLaunchKernelGGL((seg_combine_kernel<16>), grid, block, 0, s, M, N, s0, sin, sfin, H, G, DV); break;
    case 32: hipLaunchKernelGGL((seg_combine_kernel<32>), grid, block, 0, s, M, N, s0, sin, sfin, H, G, DV); break;
    case 64: hipLaunchKernelGGL((seg_combine_kernel<64>), grid, block, 0, s, M, N, s0, sin, sfin, H, G, DV); break;
    case 128: hipLaunchKernelGGL((seg_combine_kernel<128>), grid, block, 0, s, M, N, s0, sin, sfin, H, G, DV); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace efla
