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

// One workgroup per (b, h, 16 value columns); S (d_k x 16, fp32) runs along
// the segments of sequence b,
//     sin[u] = S;   S = M[u] S + N[u],   u = b G + g,
// and ends in sfin[b, h] (NULL: not written).  M [U, H, d_k, d_k], N and sin
// [U, H, d_k, d_v], fp32.  Wavefront w keeps key rows 16 w .. 16 w + 15 of S
// in a matrix-core accumulator (lane (i, g): rows 16 w + 4 g + q, column
// v0 + i) and forms those rows of M[u] S + N[u] with v_mfma_f32_16x16x4f32.
// Product j of k-block kb takes, in lane group g, key index 16 kb + 4 g + j:
// then a lane's A operands are four consecutive floats of one row of M (one
// 16-byte load), and its B operands are element j of the accumulator that
// the same lane of wavefront kb holds, read back through LDS.  M[u+1] and
// N[u+1] are in flight while step u computes.
template <int DK>
__global__ __launch_bounds__(DK * 4) void seg_combine_kernel(const float* __restrict__ M,
                                                             const float* __restrict__ Nf, const float* s0,
                                                             float* __restrict__ sin, float* sfin, int H, int G,
                                                             int DV) {
  constexpr int NKB = DK / 16;  // k-blocks, and wavefronts
  __shared__ f32x4 Sb[2][NKB][kWave];
  const int nvb = DV / 16, x = blockIdx.x, bh = x / nvb, v0 = 16 * (x % nvb);
  const int b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, i = lane & 15, g = lane >> 4;
  const int row = 16 * w + 4 * g;  // this lane's accumulator rows: row .. row + 3
  f32x4 S;
#pragma unroll
  for (int qq = 0; qq < 4; ++qq) S[qq] = s0 != nullptr ? s0[(int64_t(bh) * DK + row + qq) * DV + v0 + i] : 0.0f;
  f32x4 Mr[NKB], Nr;
  auto load = [&](int gi) {
    const int64_t u = int64_t(b) * G + gi;
    const float* Mu = M + (u * H + h) * DK * DK + (16 * w + i) * DK + 4 * g;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Mr[kb] = *reinterpret_cast<const f32x4*>(Mu + 16 * kb);
    const float* Nu = Nf + ((u * H + h) * DK + row) * DV + v0 + i;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) Nr[qq] = Nu[qq * DV];
  };
  load(0);
  for (int gi = 0; gi < G; ++gi) {
    const int64_t u = int64_t(b) * G + gi;
    float* su = sin + ((u * H + h) * DK + row) * DV + v0 + i;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) su[qq * DV] = S[qq];
    // two buffers: a wavefront writes buffer (gi & 1) only after every
    // wavefront has passed the barrier of step gi - 1, i.e. has finished
    // reading that buffer in step gi - 2
    Sb[gi & 1][w][lane] = S;
    __syncthreads();
    f32x4 Mc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) Mc[kb] = Mr[kb];
    f32x4 acc = Nr;
    if (gi + 1 < G) load(gi + 1);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const f32x4 sb = Sb[gi & 1][kb][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(Mc[kb][j], sb[j], acc, 0, 0, 0);
    }
    S = acc;
  }
  if (sfin != nullptr) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) sfin[(int64_t(bh) * DK + row + qq) * DV + v0 + i] = S[qq];
  }
}

hipError_t launch_seg_offsets(int32_t* cu, int B, int G, int64_t L, int64_t Ls, hipStream_t s) {
  const int n = B * G + 1;
  hipLaunchKernelGGL(seg_offsets_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, s, cu, B, G, L, Ls);
  return hipGetLastError();
}

hipError_t launch_seg_combine(const float* M, const float* N, const float* s0, float* sin, float* sfin, int B, int H,
                              int G, int DK, int DV, hipStream_t s) {
  const dim3 grid{unsigned(B * H * (DV / 16))}, block{unsigned(DK * 4)};
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
