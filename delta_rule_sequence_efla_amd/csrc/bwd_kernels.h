// bwd_kernels.h -- the chunked backward pass of the EFLA forward recurrence.
//
// The pages give the forward recurrence only (Method step 3); its gradient
// follows by calculus.  Per chunk of C tokens with start state S, end-state
// gradient dS' and the forward quantities
//     A = tril(diag(a) K K^T, -1),  X = (I + A)^{-1},  T = X diag(a),
//     D = V - K S,  U = T D,  P = tril(Q K^T),  O = Q S + P U,  S' = S + K^T U,
// the gradients of a scalar loss are
//     dU = P^T dO + K dS'            dD = T^T dU            dV = dD
//     dP = tril(dO U^T)              dT = tril(dU D^T)
//     dQ = dO S^T + dP K
//     dK = dP^T Q + U dS'^T - dD S^T + (dG + dG^T) K + 2 diag(dlambda) K
//     dX = dT diag(a),  da_j = sum_i dT_ij X_ij,  dA = -X^T dX X^T (strictly lower)
//     da_i += sum_{j<i} dA_ij G_ij,  dG = diag(a) dA  (strictly lower),  G = K K^T
//     dbeta = da * d a / d beta,  dlambda = da * d a / d lambda
//     dS = dS' + Q^T dO - K^T dD     (the gradient at the chunk's start)
// Stages (efla_chunk_bwd):
//   1. the UT transform's backward instance: T (input dtype), and in fp32
//      X, a and P per chunk slot;
//   2. the forward recurrence again, storing the state at the start of every
//      chunk (in the input dtype: for bf16 inputs the operand values the
//      forward's products use);
//   3. bwd_state_kernel: the sequential pass in reverse over chunks, per
//      (b, h, 16 value columns), storing dS' of every chunk and dS_0;
//   4. bwd_chunk_kernel: every chunk in parallel, the formulas above, streamed
//      over 16-column value blocks.
// All arithmetic is fp32 on fp32 matrix cores (v_mfma_f32_16x16x4_f32); bf16
// inputs are widened exactly.
#pragma once

#include "common.h"

namespace efla {

// acc (a 16x16 tile at rows r0.., columns c0..) += opA(A) opB(B) over k = 0..K-1
// (K % 16 == 0), operands in LDS as fp32.  AT: A is stored [K][M] (its
// transpose is used); BT: B is stored [N][K].  Lane (li, g) feeds k = kb + 4g + e
// to the e-th product of each 16-wide k block, for A and B alike.
template <bool AT, bool BT>
__device__ __forceinline__ void tile_mma16(f32x4& acc, const float* A, int lda, const float* B, int ldb, int r0,
                                           int c0, int K, int li, int g) {
  for (int kb = 0; kb < K; kb += 16) {
    f32x4 av, bv;
    if constexpr (AT) {
#pragma unroll
      for (int e = 0; e < 4; ++e) av[e] = A[(kb + 4 * g + e) * lda + r0 + li];
    } else {
      av = *reinterpret_cast<const f32x4*>(A + (r0 + li) * lda + kb + 4 * g);
    }
    if constexpr (BT) {
      bv = *reinterpret_cast<const f32x4*>(B + (c0 + li) * ldb + kb + 4 * g);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) bv[e] = B[(kb + 4 * g + e) * ldb + c0 + li];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc, 0, 0, 0);
  }
}

// d a / d beta and d a / d lambda of the coefficient (Method step 3) under a
// rule, x = beta * lambda:  e^{-x}  and  beta^2 psi(x) with
// psi(x) = -(1 - (1 + x) e^{-x}) / x^2, a series below x = 0.1
// (-1/2 + x/3 - x^2/8 + x^3/30 - x^4/144 + x^5/840).  Euler rule: 1 and 0.
__device__ __forceinline__ void efla_alpha_grad(float beta, float lam, int rule, float& da_db, float& da_dl) {
  if (rule == 1) {
    da_db = 1.0f;
    da_dl = 0.0f;
    return;
  }
  const float x = beta * lam;
  da_db = expf(-x);
  float psi;
  if (x == __builtin_inff()) {
    da_dl = -1.0f / (lam * lam);
    return;
  }
  if (x < 0.1f) {
    psi = -(0.5f - x * (1.0f / 3.0f - x * (1.0f / 8.0f - x * (1.0f / 30.0f - x * (1.0f / 144.0f - x / 840.0f)))));
  } else {
    psi = -((-expm1f(-x)) - x * expf(-x)) / (x * x);
  }
  da_dl = beta * beta * psi;
}

// A ROWS x COLS tile of T (rows `stride` elements apart) moved into fp32 LDS
// in two steps, so that the loads of several tiles are all in flight before
// any is waited on: load() issues 16-byte loads into registers (rows at or
// past `valid` read as zero), store() widens them into dst (pitch in floats).
// COLS * sizeof(T) must be a multiple of 16 and rows 16-byte aligned.
template <typename T, int ROWS, int COLS, int NTH = kThreads>  // NTH: threads of the workgroup
struct F32Stager {
  static constexpr int VN = 16 / int(sizeof(T)), VPR = COLS / VN, TOT = ROWS * VPR, CNT = cdiv(TOT, NTH);
  u32x4 r[CNT];
  __device__ __forceinline__ void load(const T* src, int64_t stride, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      const int t = idx / VPR, c = (idx % VPR) * VN;
      r[i] = u32x4{0u, 0u, 0u, 0u};
      if (idx < TOT && t < valid) r[i] = *reinterpret_cast<const u32x4*>(src + t * stride + c);
    }
  }
  __device__ __forceinline__ void store(float* dst, int pitch, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      if (idx < TOT) {
        const int t = idx / VPR, c = (idx % VPR) * VN;
        union {
          u32x4 u;
          T e[VN];
        } x;
        x.u = r[i];
#pragma unroll
        for (int e = 0; e < VN; ++e) dst[t * pitch + c + e] = to_f32(x.e[e]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Stage 3: reverse sequential pass.  One workgroup per (b, h, 16 value
// columns); dS (d_k x 16, fp32) lives in LDS.  For chunk n = last .. 0:
//   dstates[n] = dS   (the gradient at the chunk's end)
//   E = P^T dO + K dS,  F = T^T E,  dS += Q^T dO - K^T F
// ---------------------------------------------------------------------------
template <typename T, int DK, int C>
__global__ __launch_bounds__(kThreads) void bwd_state_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ dout, const T* __restrict__ tws,
    const float* __restrict__ pws, const float* __restrict__ dsf, float* __restrict__ dstates,
    float* __restrict__ ds0, int H, int64_t L, int NC, int DV, int NVB) {
  constexpr int DKP = round_up(DK, 32), CP = round_up(C, 32);
  constexpr int QP = DKP + 4, CPP = CP + 4, VP = 16 + 4;
  __shared__ __align__(16) float Qs[CP * QP];
  __shared__ __align__(16) float Ks[CP * QP];
  __shared__ __align__(16) float Ts[CP * CPP];
  __shared__ __align__(16) float Ps[CP * CPP];
  __shared__ __align__(16) float dOs[CP * VP];
  __shared__ __align__(16) float Es[CP * VP];
  __shared__ __align__(16) float Fs[CP * VP];
  __shared__ __align__(16) float dSs[DKP * VP];

  const int x = blockIdx.x, bh = x / NVB, vb = x % NVB;
  const int64_t h = bh % H;
  const SeqSpan sp = seq_span<C>(nullptr, bh / H, h, H, L, NC);
  const int v0 = 16 * vb;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;

  // zero what the stagers never write: padding rows / columns
  for (int i = tid; i < CP * QP; i += kThreads) Qs[i] = Ks[i] = 0.0f;
  for (int i = tid; i < CP * CPP; i += kThreads) Ts[i] = Ps[i] = 0.0f;
  for (int i = tid; i < CP * VP; i += kThreads) dOs[i] = 0.0f;
  for (int i = tid; i < DKP * 16; i += kThreads) {
    const int d = i / 16, c = i % 16;
    dSs[d * VP + c] = (dsf != nullptr && d < DK) ? dsf[(int64_t(bh) * DK + d) * DV + v0 + c] : 0.0f;
  }

  // chunk n's operands, staged through registers one chunk ahead
  F32Stager<T, C, DK> sq, sk;
  F32Stager<T, C, C> st;
  F32Stager<float, C, C> spp;
  F32Stager<T, C, 16> sdo;
  auto load = [&](int n) {
    const int64_t t0 = int64_t(n) * C;
    const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
    const int64_t row0 = (sp.bos + t0) * H + h;
    sq.load(q + row0 * DK, qk_stride, valid, tid);
    sk.load(k + row0 * DK, qk_stride, valid, tid);
    sdo.load(dout + row0 * DV + v0, v_stride, valid, tid);
    st.load(tws + (sp.slot0 + n) * C * C, C, C, tid);
    spp.load(pws + (sp.slot0 + n) * C * C, C, C, tid);
  };
  if (sp.nc > 0) load(sp.nc - 1);
  __syncthreads();

  for (int n = sp.nc - 1; n >= 0; --n) {
    float* dst = dstates + (sp.slot0 + n) * DK * DV;
    for (int i = tid; i < DK * 16; i += kThreads) {
      const int d = i / 16, c = i % 16;
      dst[d * DV + v0 + c] = dSs[d * VP + c];
    }
    sq.store(Qs, QP, tid);
    sk.store(Ks, QP, tid);
    sdo.store(dOs, VP, tid);
    st.store(Ts, CPP, tid);
    spp.store(Ps, CPP, tid);
    if (n > 0) load(n - 1);  // in flight during this chunk
    __syncthreads();
    // E = P^T dO + K dS
    for (int rt = w; rt < CP / 16; rt += 4) {
      f32x4 acc = zero4();
      tile_mma16<true, false>(acc, Ps, CPP, dOs, VP, 16 * rt, 0, CP, li, g);
      tile_mma16<false, false>(acc, Ks, QP, dSs, VP, 16 * rt, 0, DKP, li, g);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) Es[(16 * rt + 4 * g + qq) * VP + li] = acc[qq];
    }
    __syncthreads();
    // F = T^T E
    for (int rt = w; rt < CP / 16; rt += 4) {
      f32x4 acc = zero4();
      tile_mma16<true, false>(acc, Ts, CPP, Es, VP, 16 * rt, 0, CP, li, g);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) Fs[(16 * rt + 4 * g + qq) * VP + li] = acc[qq];
    }
    __syncthreads();
    // dS += Q^T dO - K^T F
    for (int dt = w; dt < DKP / 16; dt += 4) {
      f32x4 plus = zero4(), minus = zero4();
      tile_mma16<true, false>(plus, Qs, QP, dOs, VP, 16 * dt, 0, CP, li, g);
      tile_mma16<true, false>(minus, Ks, QP, Fs, VP, 16 * dt, 0, CP, li, g);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) dSs[(16 * dt + 4 * g + qq) * VP + li] += plus[qq] - minus[qq];
    }
    __syncthreads();
  }
  if (ds0 != nullptr) {
    for (int i = tid; i < DK * 16; i += kThreads) {
      const int d = i / 16, c = i % 16;
      ds0[(int64_t(bh) * DK + d) * DV + v0 + c] = dSs[d * VP + c];
    }
  }
}

// ---------------------------------------------------------------------------
// Stage 4: every chunk in parallel.  One workgroup per (b, h, chunk); value
// columns are streamed 16 at a time, accumulating dQ, dK, dP and dT in
// registers; then the UT-transform part of the gradient.
// ---------------------------------------------------------------------------
template <typename T, int DK, int C>
struct BwdChunkShape {
  static constexpr int DKP = round_up(DK, 32), CP = round_up(C, 32);
  static constexpr int QP = DKP + 4, CPP = CP + 4, VP = 16 + 4;
  static constexpr int NQ = (CP / 16) * (DKP / 16) / 4;  // dQ / dK tiles per wave
  static constexpr int NP = (CP / 16) * (CP / 16) / 4;   // dP / dT tiles per wave
  static constexpr int VBUF = 2 * DKP * VP + 6 * CP * VP;  // per-value-block buffers
  static constexpr int RBUF = VBUF > 3 * CP * CPP ? VBUF : 3 * CP * CPP;
};

// The part of a chunk's gradients after the value blocks (fp32 throughout),
// shared by both chunk kernels: dP and dT from their accumulators, then
//   dQ += dP K;  dK += dP^T Q;  dX = dT diag(a);  da_j = sum_i dT_ij X_ij;
//   W = X^T dX;  dA = -W X^T (strictly lower);  da_i += sum_{j<i} dA_ij G_ij;
//   dG = diag(a) dA;  dbeta, dlambda;  dK += (dG + dG^T) K + 2 diag(dlambda) K
// and the stores of dq, dk and dbeta.  Qs, Ks: fp32 [CP][QP]; M0, M1: fp32
// [CP][CPP]; R: fp32, at least 3 CP CPP; as: the chunk's coefficients.
// Called by all threads after a barrier that frees M0, M1 and R.
template <typename T, int DK, int C>
__device__ __forceinline__ void bwd_chunk_tail(
    const float* __restrict__ Qs, const float* __restrict__ Ks, float* __restrict__ M0, float* __restrict__ M1,
    float* __restrict__ R, const float* __restrict__ as, float* __restrict__ das, float* __restrict__ dls,
    f32x4 (&dQa)[BwdChunkShape<T, DK, C>::NQ], f32x4 (&dKa)[BwdChunkShape<T, DK, C>::NQ],
    const f32x4 (&dPa)[BwdChunkShape<T, DK, C>::NP], const f32x4 (&dTa)[BwdChunkShape<T, DK, C>::NP],
    const float* __restrict__ xws, const T* __restrict__ beta, T* __restrict__ dq, T* __restrict__ dk,
    T* __restrict__ dbeta, int64_t slot, int64_t row0, int valid, int H, int rule) {
  using S = BwdChunkShape<T, DK, C>;
  constexpr int DKP = S::DKP, CP = S::CP, QP = S::QP, CPP = S::CPP, NQ = S::NQ, NP = S::NP;
  constexpr int NCQ = DKP / 16, NCP = CP / 16;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t qk_stride = int64_t(H) * DK;
  // dP (lower, diagonal included) -> M1; dT (lower) -> M0; X -> R0
  float* X = R;
  float* R1 = R + CP * CPP;
  float* R2 = R1 + CP * CPP;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + 4 * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 4 * g + qq, c = c0 + li;
      M1[r * CPP + c] = c <= r ? dPa[i][qq] : 0.0f;
      M0[r * CPP + c] = c <= r ? dTa[i][qq] : 0.0f;
    }
  }
  {
    F32Stager<float, C, C> sx;
    sx.load(xws + slot * C * C, C, C, tid);
    if constexpr (C < CP) {
      for (int i = tid; i < CP * CPP; i += kThreads) X[i] = 0.0f;
      __syncthreads();
    }
    sx.store(X, CPP, tid);  // X's rows and columns < C; the zeros above cover the padding
  }
  __syncthreads();
  // dQ += dP K;  dK += dP^T Q;  dX = dT diag(a);  da_j = sum_i dT_ij X_ij
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int t = w + 4 * i, r0 = 16 * (t / NCQ), c0 = 16 * (t % NCQ);
    tile_mma16<false, false>(dQa[i], M1, CPP, Ks, QP, r0, c0, CP, li, g);
    tile_mma16<true, false>(dKa[i], M1, CPP, Qs, QP, r0, c0, CP, li, g);
  }
  for (int i = tid; i < CP * CP; i += kThreads) {
    const int r = i / CP, c = i % CP;
    R1[r * CPP + c] = M0[r * CPP + c] * as[c];
  }
  if (tid < CP) {
    float s = 0.0f;
    for (int r = 0; r < CP; ++r) s = fmaf(M0[r * CPP + tid], X[r * CPP + tid], s);
    das[tid] = s;
  }
  __syncthreads();
  // W = X^T dX -> M1
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + 4 * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
    f32x4 acc = zero4();
    tile_mma16<true, false>(acc, X, CPP, R1, CPP, r0, c0, CP, li, g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) M1[(r0 + 4 * g + qq) * CPP + c0 + li] = acc[qq];
  }
  __syncthreads();
  // dA = -W X^T (strictly lower) -> R2;  G = K K^T -> R1
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + 4 * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
    f32x4 acc = zero4(), gg = zero4();
    tile_mma16<false, true>(acc, M1, CPP, X, CPP, r0, c0, CP, li, g);
    tile_mma16<false, true>(gg, Ks, QP, Ks, QP, r0, c0, DKP, li, g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 4 * g + qq, c = c0 + li;
      R2[r * CPP + c] = c < r ? -acc[qq] : 0.0f;
      R1[r * CPP + c] = gg[qq];
    }
  }
  __syncthreads();
  // da_i += sum_{j<i} dA_ij G_ij;  dG = diag(a) dA -> R0 (X is done)
  if (tid < CP) {
    float s = 0.0f;
    for (int c = 0; c < tid; ++c) s = fmaf(R2[tid * CPP + c], R1[tid * CPP + c], s);
    das[tid] += s;
  }
  for (int i = tid; i < CP * CP; i += kThreads) {
    const int r = i / CP, c = i % CP;
    X[r * CPP + c] = as[r] * R2[r * CPP + c];
  }
  __syncthreads();
  // dbeta, dlambda
  if (tid < CP) {
    float db = 0.0f, dl = 0.0f;
    if (tid < valid) {
      const float bt = to_f32(beta[row0 + int64_t(tid) * H]);
      float da_db, da_dl;
      efla_alpha_grad(bt, R1[tid * CPP + tid], rule, da_db, da_dl);
      db = das[tid] * da_db;
      dl = das[tid] * da_dl;
      dbeta[row0 + int64_t(tid) * H] = from_f32<T>(db);
    }
    dls[tid] = dl;
  }
  __syncthreads();
  // dK += (dG + dG^T) K + 2 diag(dlambda) K;  write dq, dk
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int t = w + 4 * i, r0 = 16 * (t / NCQ), c0 = 16 * (t % NCQ);
    tile_mma16<false, false>(dKa[i], X, CPP, Ks, QP, r0, c0, CP, li, g);
    tile_mma16<true, false>(dKa[i], X, CPP, Ks, QP, r0, c0, CP, li, g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 4 * g + qq, c = c0 + li;
      if (r < valid && c < DK) {
        dq[row0 * DK + r * qk_stride + c] = from_f32<T>(dQa[i][qq]);
        dk[row0 * DK + r * qk_stride + c] = from_f32<T>(dKa[i][qq] + 2.0f * dls[r] * Ks[r * QP + c]);
      }
    }
  }
}

template <typename T, int DK, int C>
__global__ __launch_bounds__(kThreads) void bwd_chunk_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const T* __restrict__ beta,
    const T* __restrict__ dout, const T* __restrict__ tws, const float* __restrict__ xws,
    const float* __restrict__ aws, const float* __restrict__ pws, const T* __restrict__ states,
    const float* __restrict__ dstates, T* __restrict__ dq, T* __restrict__ dk, T* __restrict__ dv,
    T* __restrict__ dbeta, int H, int64_t L, int NC, int DV, int rule) {
  using S = BwdChunkShape<T, DK, C>;
  constexpr int DKP = S::DKP, CP = S::CP, QP = S::QP, CPP = S::CPP, VP = S::VP, NQ = S::NQ, NP = S::NP;
  constexpr int NCQ = DKP / 16, NCP = CP / 16;  // tile columns of the C x DK and C x C grids
  __shared__ __align__(16) float Qs[CP * QP];
  __shared__ __align__(16) float Ks[CP * QP];
  __shared__ __align__(16) float M0[CP * CPP];  // T, then dT
  __shared__ __align__(16) float M1[CP * CPP];  // P, then dP, then X^T dX
  __shared__ __align__(16) float R[S::RBUF];    // value-block buffers, then X, dX, G, dA, dG
  __shared__ float as[CP], das[CP], dls[CP];

  const int64_t slot = blockIdx.x;
  const int n = int(slot % NC);
  const int64_t bh = slot / NC, h = bh % H;
  const SeqSpan sp = seq_span<C>(nullptr, int(bh / H), h, H, L, NC);
  const int64_t t0 = int64_t(n) * C;
  const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
  const int64_t row0 = (sp.bos + t0) * H + h;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;

  // chunk operands (16-byte loads, all in flight before the first use)
  {
    F32Stager<T, C, DK> sq, sk;
    F32Stager<T, C, C> st;
    F32Stager<float, C, C> spp;
    sq.load(q + row0 * DK, qk_stride, valid, tid);
    sk.load(k + row0 * DK, qk_stride, valid, tid);
    st.load(tws + slot * C * C, C, C, tid);
    spp.load(pws + slot * C * C, C, C, tid);
    if constexpr (C < CP || DK < DKP) {
      for (int i = tid; i < CP * QP; i += kThreads) Qs[i] = Ks[i] = 0.0f;
      for (int i = tid; i < CP * CPP; i += kThreads) M0[i] = M1[i] = 0.0f;
      __syncthreads();
    }
    sq.store(Qs, QP, tid);
    sk.store(Ks, QP, tid);
    st.store(M0, CPP, tid);
    spp.store(M1, CPP, tid);
  }
  if (tid < CP) as[tid] = tid < C ? aws[slot * C + tid] : 0.0f;

  float* Sv = R;               // S[:, block]      DKP x 16
  float* dSv = Sv + DKP * VP;  // dS'[:, block]    DKP x 16
  float* Vv = dSv + DKP * VP;  // V rows, block    CP x 16
  float* dOv = Vv + CP * VP;
  float* Dv = dOv + CP * VP;
  float* Uv = Dv + CP * VP;
  float* dUv = Uv + CP * VP;
  float* dDv = dUv + CP * VP;

  f32x4 dQa[NQ], dKa[NQ], dPa[NP], dTa[NP];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dQa[i] = dKa[i] = zero4();
#pragma unroll
  for (int i = 0; i < NP; ++i) dPa[i] = dTa[i] = zero4();

  const T* st = states + slot * DK * DV;
  const float* dst = dstates + slot * DK * DV;
  // one 16-column value block's operands, staged through registers one block ahead
  F32Stager<T, DK, 16> ss;
  F32Stager<float, DK, 16> sds;
  F32Stager<T, C, 16> sv, sdo;
  auto load_block = [&](int v0) {
    ss.load(st + v0, DV, DK, tid);
    sds.load(dst + v0, DV, DK, tid);
    sv.load(v + row0 * DV + v0, v_stride, valid, tid);
    sdo.load(dout + row0 * DV + v0, v_stride, valid, tid);
  };
  load_block(0);
  if constexpr (C < CP || DK < DKP) {  // padding rows of the block buffers stay zero
    __syncthreads();
    for (int i = tid; i < S::VBUF; i += kThreads) R[i] = 0.0f;
  }
  for (int v0 = 0; v0 < DV; v0 += 16) {
    __syncthreads();  // previous block's buffers are free (and the operands above are in place)
    ss.store(Sv, VP, tid);
    sds.store(dSv, VP, tid);
    sv.store(Vv, VP, tid);
    sdo.store(dOv, VP, tid);
    if (v0 + 16 < DV) load_block(v0 + 16);  // in flight during this block
    __syncthreads();
    // D = V - K S,  dU = P^T dO + K dS'
    for (int t = w; t < 2 * NCP; t += 4) {
      const int rt = t % NCP;
      f32x4 acc = zero4();
      if (t < NCP) {
        tile_mma16<false, false>(acc, Ks, QP, Sv, VP, 16 * rt, 0, DKP, li, g);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int r = 16 * rt + 4 * g + qq;
          Dv[r * VP + li] = Vv[r * VP + li] - acc[qq];
        }
      } else {
        tile_mma16<true, false>(acc, M1, CPP, dOv, VP, 16 * rt, 0, CP, li, g);
        tile_mma16<false, false>(acc, Ks, QP, dSv, VP, 16 * rt, 0, DKP, li, g);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) dUv[(16 * rt + 4 * g + qq) * VP + li] = acc[qq];
      }
    }
    __syncthreads();
    // U = T D,  dD = T^T dU (= dV)
    for (int t = w; t < 2 * NCP; t += 4) {
      const int rt = t % NCP;
      f32x4 acc = zero4();
      if (t < NCP) {
        tile_mma16<false, false>(acc, M0, CPP, Dv, VP, 16 * rt, 0, CP, li, g);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) Uv[(16 * rt + 4 * g + qq) * VP + li] = acc[qq];
      } else {
        tile_mma16<true, false>(acc, M0, CPP, dUv, VP, 16 * rt, 0, CP, li, g);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int r = 16 * rt + 4 * g + qq;
          dDv[r * VP + li] = acc[qq];
          if (r < valid) dv[row0 * DV + r * v_stride + v0 + li] = from_f32<T>(acc[qq]);
        }
      }
    }
    __syncthreads();
    // dQ += dO S^T;  dK += U dS'^T - dD S^T;  dP += dO U^T;  dT += dU D^T  (16-column contraction)
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int t = w + 4 * i, r0 = 16 * (t / NCQ), c0 = 16 * (t % NCQ);
      tile_mma16<false, true>(dQa[i], dOv, VP, Sv, VP, r0, c0, 16, li, g);
      tile_mma16<false, true>(dKa[i], Uv, VP, dSv, VP, r0, c0, 16, li, g);
      f32x4 m = zero4();
      tile_mma16<false, true>(m, dDv, VP, Sv, VP, r0, c0, 16, li, g);
      dKa[i] -= m;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = w + 4 * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
      tile_mma16<false, true>(dPa[i], dOv, VP, Uv, VP, r0, c0, 16, li, g);
      tile_mma16<false, true>(dTa[i], dUv, VP, Dv, VP, r0, c0, 16, li, g);
    }
  }
  __syncthreads();  // done with T, P and the value-block buffers

  bwd_chunk_tail<T, DK, C>(Qs, Ks, M0, M1, R, as, das, dls, dQa, dKa, dPa, dTa, xws, beta, dq, dk, dbeta, slot,
                           row0, valid, H, rule);
}

}  // namespace efla
