// common.h -- device helpers shared by the EFLA kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used by every kernel
// --------------------------------------------
// All products run on 16x16 output tiles.  A lane `l` of a 64-wide wavefront has
// li = l % 16 and g = l / 16.  An accumulator tile holds D[4g + q][li] in its
// element q (q = 0..3), the CDNA layout of v_mfma_f32_16x16x*.
//
// The reduction (k) index is consumed in "k-units" of 32.  A k-unit is two
// 16-wide k tiles; element e (0..7) of a lane's operand fragment carries
//       k = 32*ku + 16*(e/4) + 4*g + (e%4).
// For bf16 one k-unit is one v_mfma_f32_16x16x32_bf16 (8 bf16 per lane); for
// fp32 it is eight v_mfma_f32_16x16x4_f32 (one float per lane each).  The sum
// over k does not depend on which k a (lane, element) slot carries as long as
// the A and B fragments agree, and with this assignment the four rows 4g..4g+3
// that an accumulator tile keeps in one lane are exactly the k values that lane
// feeds to the next product.  So a product's result can be fed back as the next
// product's operand straight from registers (accumulator -> fragment), with no
// trip through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace efla {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kThreads = 256;  // four wavefronts per workgroup

// Index of this wavefront in its workgroup, as a wave-uniform (scalar) value:
// branches on it are scalar branches, and addresses derived from it stay in
// scalar registers, where threadIdx.x / 64 would look lane-dependent.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6); }

__host__ __device__ constexpr int round_up(int x, int m) { return (x + m - 1) / m * m; }
__host__ __device__ constexpr int cdiv(int x, int m) { return (x + m - 1) / m; }

// ---- element types: float, or bf16 carried as its 16-bit pattern ----------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
  // round to nearest even (the hardware conversion on gfx950)
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

// ---- the coefficient of the exact flow ------------------------------------
// alpha = (1 - e^{-beta*lambda}) / lambda, written as beta * (1 - e^{-x}) / x
// with x = beta * lambda: no 0/0 at lambda = 0 and no loss when x underflows
// (both give beta); x = +inf (stiff limit) gives 1/lambda.
__device__ __forceinline__ float efla_alpha(float beta, float lam) {
  const float x = beta * lam;
  if (x == 0.0f) return beta;
  if (x == __builtin_inff()) return 1.0f / lam;
  return beta * (-expm1f(-x) / x);
}

// The coefficient under an update rule: rule 0 is the exact flow above; rule 1
// is one explicit Euler step of length beta (the delta-rule / DeltaNet update
// the pages contrast EFLA with), whose coefficient is beta itself.
__device__ __forceinline__ float efla_alpha_rule(float beta, float lam, int rule) {
  return rule == 1 ? beta : efla_alpha(beta, lam);
}

// ---- operand fragments ------------------------------------------------------
template <typename T> struct Frag;
template <> struct Frag<uint16_t> { bf16x8 v; };
template <> struct Frag<float> { float v[8]; };

__device__ __forceinline__ void mma(f32x4& acc, const Frag<uint16_t>& a, const Frag<uint16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Fragment of a row-major LDS matrix X (pitch in elements): row `row`, k-unit ku.
// Needs pitch % 4 == 0 and 8-byte (bf16) / 16-byte (fp32) aligned X.
__device__ __forceinline__ Frag<uint16_t> lds_frag(const uint16_t* X, int pitch, int row, int ku, int g) {
  const uint16_t* p = X + row * pitch + 32 * ku + 4 * g;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  Frag<uint16_t> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ Frag<float> lds_frag(const float* X, int pitch, int row, int ku, int g) {
  const float* p = X + row * pitch + 32 * ku + 4 * g;
  const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 16);
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = lo[e];
    f.v[4 + e] = hi[e];
  }
  return f;
}

// Fragment of the TRANSPOSE of a row-major LDS matrix X[k][m]: operand row m = col.
__device__ __forceinline__ Frag<uint16_t> lds_frag_t(const uint16_t* X, int pitch, int col, int ku, int g) {
  Frag<uint16_t> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = 32 * ku + 16 * (e / 4) + 4 * g + (e % 4);
    f.v[e] = __builtin_bit_cast(__bf16, X[k * pitch + col]);
  }
  return f;
}
__device__ __forceinline__ Frag<float> lds_frag_t(const float* X, int pitch, int col, int ku, int g) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int k = 32 * ku + 16 * (e / 4) + 4 * g + (e % 4);
    f.v[e] = X[k * pitch + col];
  }
  return f;
}

// Fragment from two accumulator tiles (k tiles 2ku and 2ku+1 of the operand).
template <typename T> __device__ __forceinline__ Frag<T> acc_frag(const f32x4& lo, const f32x4& hi);
template <> __device__ __forceinline__ Frag<uint16_t> acc_frag<uint16_t>(const f32x4& lo, const f32x4& hi) {
  Frag<uint16_t> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = static_cast<__bf16>(lo[e]);
    f.v[4 + e] = static_cast<__bf16>(hi[e]);
  }
  return f;
}
template <> __device__ __forceinline__ Frag<float> acc_frag<float>(const f32x4& lo, const f32x4& hi) {
  Frag<float> f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f.v[e] = lo[e];
    f.v[4 + e] = hi[e];
  }
  return f;
}

// Store four consecutive values (converted to T) to LDS: 8 B for bf16, 16 B for fp32.
__device__ __forceinline__ void st4(uint16_t* p, const f32x4& x) {
  bf16x4 h;
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = static_cast<__bf16>(x[e]);
  *reinterpret_cast<bf16x4*>(p) = h;
}
__device__ __forceinline__ void st4(float* p, const f32x4& x) { *reinterpret_cast<f32x4*>(p) = x; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.0f, 0.0f, 0.0f, 0.0f}; }

// 16-byte vector of T (8 bf16 or 4 fp32) used for global <-> LDS staging.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <typename T> struct Vec16 { static constexpr int n = 16 / sizeof(T); };

// ---------------------------------------------------------------------------
// Where the tokens and workspace chunk slots of sequence u live.
//  * Dense batch [B, L, H, d] (cu == nullptr): u = b, tokens u L .. u L + L - 1
//    of the token-major rows; the chunks of (u, h) use slots (u H + h) NC + n.
//  * Packed variable-length batch [T, H, d] with offsets cu[0..N]
//    (`L` = T): tokens cu[u] .. cu[u+1] - 1; the chunks of (u, h) use slots
//    h NC + floor(cu[u] / C) + u + n, NC = floor(T / C) + N slots per head.
//    Sequences get disjoint slot ranges with no prefix sum over the lengths,
//    because floor(a / C) + ceil(l / C) <= floor((a + l) / C) + 1.
//    Offsets are clamped into [0, T] (and each end to at least its start), so
//    malformed offsets give wrong numbers but no access out of bounds.
struct SeqSpan {
  int64_t bos;    // first token
  int64_t len;    // number of tokens
  int nc;         // number of chunks
  int64_t slot0;  // workspace slot of chunk 0
};

__device__ __forceinline__ int64_t clamp_offset(int64_t a, int64_t lo, int64_t hi) {
  return a < lo ? lo : (a > hi ? hi : a);
}

template <int C>
__device__ __forceinline__ SeqSpan seq_span(const int32_t* __restrict__ cu, int u, int64_t h, int H, int64_t L,
                                            int NC) {
  SeqSpan s;
  if (cu == nullptr) {
    s.bos = int64_t(u) * L;
    s.len = L;
    s.nc = NC;
    s.slot0 = (int64_t(u) * H + h) * NC;
  } else {
    const int64_t a = clamp_offset(cu[u], 0, L);
    const int64_t e = clamp_offset(cu[u + 1], a, L);
    s.bos = a;
    s.len = e - a;
    s.nc = int((s.len + C - 1) / C);
    s.slot0 = h * NC + a / C + u;
  }
  return s;
}

// Packed batches: slot j (0 .. NC-1) of head h belongs to chunk n of sequence
// u, found by binary search over the slot offsets floor(cu[u] / C) + u (which
// increase with u); false for a slot no chunk uses.
// Schedule of a packed batch.  The recurrence runs one workgroup per
// (sequence, head, value block), and a workgroup's time grows with its
// sequence's chunk count; workgroups are dispatched in index order as compute
// units free up, so handing out the sequences longest first is a
// longest-processing-time-first list schedule.  The order is computed on the
// device, by extra workgroups of the UT-transform launch:
//     rank(u) = #{v : n(v) > n(u)} + #{v < u : n(v) = n(u)},  order[rank(u)] = u,
// with n the chunk count from offsets clamped exactly as seq_span clamps them,
// a bijection onto [0, N) whatever the offsets hold.
constexpr int kRankSeqs = 256;  // sequences ranked per workgroup (one per thread of kThreads)

template <int C>
__device__ __forceinline__ int seq_chunks(const int32_t* __restrict__ cu, int u, int64_t T) {
  const int64_t a = clamp_offset(cu[u], 0, T);
  const int64_t e = clamp_offset(cu[u + 1], a, T);
  return int((e - a + C - 1) / C);
}

// Ranks sequences blk * kRankSeqs .. +kRankSeqs - 1; every thread of the
// (kThreads-wide) workgroup calls it; tile: kRankSeqs ints of LDS.
template <int C>
__device__ __forceinline__ void rank_sequences(const int32_t* __restrict__ cu, int N, int64_t T, int blk,
                                               int32_t* __restrict__ order, int* tile) {
  static_assert(kRankSeqs == kThreads, "one sequence per thread");
  const int tid = threadIdx.x, u = blk * kRankSeqs + tid;
  const int nu = u < N ? seq_chunks<C>(cu, u, T) : 0;
  int rank = 0;
  for (int base = 0; base < N; base += kRankSeqs) {
    __syncthreads();
    if (base + tid < N) tile[tid] = seq_chunks<C>(cu, base + tid, T);
    __syncthreads();
    const int n = N - base < kRankSeqs ? N - base : kRankSeqs;
    if (u < N)
      for (int i = 0; i < n; ++i) {
        const int nv = tile[i];
        rank += (nv > nu || (nv == nu && base + i < u)) ? 1 : 0;
      }
  }
  if (u < N) order[rank] = u;
}

// Sequence handled in rank r of a packed batch of N sequences (order: the
// permutation of [0, N) written by rank_sequences; an entry outside it falls
// back to r).
__device__ __forceinline__ int seq_of_rank(const int32_t* __restrict__ order, int r, int N) {
  const int u = order[r];
  return (u >= 0 && u < N) ? u : r;
}

template <int C>
__device__ __forceinline__ bool slot_chunk(const int32_t* __restrict__ cu, int N, int64_t j, int64_t h, int H,
                                           int64_t L, int NC, SeqSpan& sp, int& n) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (clamp_offset(cu[mid], 0, L) / C + mid <= j) lo = mid;
    else hi = mid - 1;
  }
  sp = seq_span<C>(cu, lo, h, H, L, NC);
  const int64_t nn = h * NC + j - sp.slot0;
  n = int(nn);
  return nn >= 0 && nn < sp.nc;
}

}  // namespace efla
