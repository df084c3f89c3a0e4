// varlen.hip -- the schedule of a packed variable-length batch.
//
// The recurrence runs one workgroup per (sequence, head, value block), and a
// workgroup's time grows with its sequence's chunk count.  Workgroups are
// dispatched in index order as compute units free up, so handing out the
// sequences longest first is a longest-processing-time-first list schedule:
// the longest chains no longer start last.  The order is computed on the
// device from the offsets, so no launch waits on a copy to the host.
#include "launchers.h"

namespace efla {

namespace {

constexpr int kOrderThreads = 256, kOrderTile = 2048;

// Chunk count of sequence u, with the offsets clamped exactly as SeqSpan does.
__device__ __forceinline__ int seq_chunks(const int32_t* __restrict__ cu, int u, int64_t T, int C) {
  const int64_t a = clamp_offset(cu[u], 0, T);
  const int64_t e = clamp_offset(cu[u + 1], a, T);
  return int((e - a + C - 1) / C);
}

// rank(u) = #{v : n(v) > n(u)} + #{v < u : n(v) = n(u)}, a bijection onto
// [0, N); order[rank(u)] = u.  One thread per sequence, the counts of all
// sequences streamed through LDS in tiles.
__global__ __launch_bounds__(kOrderThreads) void varlen_order_kernel(const int32_t* __restrict__ cu, int N,
                                                                     int64_t T, int C,
                                                                     int32_t* __restrict__ order) {
  __shared__ int tile[kOrderTile];
  const int u = blockIdx.x * kOrderThreads + threadIdx.x;
  const int nu = u < N ? seq_chunks(cu, u, T, C) : 0;
  int rank = 0;
  for (int base = 0; base < N; base += kOrderTile) {
    const int n = N - base < kOrderTile ? N - base : kOrderTile;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kOrderThreads) tile[i] = seq_chunks(cu, base + i, T, C);
    __syncthreads();
    if (u < N)
      for (int i = 0; i < n; ++i) {
        const int nv = tile[i];
        rank += (nv > nu || (nv == nu && base + i < u)) ? 1 : 0;
      }
  }
  if (u < N) order[rank] = u;
}

}  // namespace

hipError_t launch_varlen_order(const int32_t* cu, int N, int64_t T, int C, int32_t* order, hipStream_t s) {
  if (N <= 0) return hipSuccess;
  const int nwg = (N + kOrderThreads - 1) / kOrderThreads;
  hipLaunchKernelGGL(varlen_order_kernel, dim3(unsigned(nwg)), dim3(kOrderThreads), 0, s, cu, N, T, C, order);
  return hipGetLastError();
}

}  // namespace efla
