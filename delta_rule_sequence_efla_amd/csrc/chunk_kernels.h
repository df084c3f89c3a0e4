// chunk_kernels.h -- chunkwise-parallel EFLA forward on gfx950.
//
// The update rule of the pages' Method step 3,
//     S_t = (I - a_t k_t k_t^T) S_{t-1} + a_t k_t v_t^T,   o_t = S_t^T q_t,
// keeps the rank-1 structure of the delta rule, so a chunk of C tokens with
// start state S can be processed with dense products (the WY/UT scheme the
// pages name).  With K, V, Q the chunk's rows and a the chunk's coefficients:
//     T  = (I + tril(diag(a) K K^T, -1))^{-1} diag(a)          [UT transform]
//     U' = T (V - K S)                                           [pseudo-values]
//     O  = Q S + tril(Q K^T) U'          (diagonal included: o_t sees S_t)
//     S <- S + K^T U'
// Stage 1 (ut_transform_kernel) computes T for every chunk in parallel.
// Stage 2 (recurrence_kernel) walks the chunks of one (batch, head, value
// block) in order, keeping that block of S in registers in fp32.
#pragma once

#include "launchers.h"

namespace efla {

// Lower-triangular 16x16 tile pairs (r >= c) in row-major order: i -> (r, c).
__device__ __forceinline__ void lower_tile(int i, int& r, int& c) {
  r = 0;
  c = i;
  while (c > r) {
    c -= r + 1;
    ++r;
  }
}

// Rows [0, ROWS) x cols [0, COLS) of a strided global matrix (row t at
// src + t*rowstride), moved in 16-byte vectors through registers so that the
// loads of the next chunk can be in flight while the current one is computed.
// Rows at or past `valid` load as zeros.
template <typename T, int ROWS, int COLS>
struct RowStager {
  static constexpr int VN = Vec16<T>::n, VPR = COLS / VN, TOT = ROWS * VPR, CNT = cdiv(TOT, kThreads);
  u32x4 r[CNT];

  __device__ __forceinline__ void load(const T* src, int64_t rowstride, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * kThreads;
      const int t = idx / VPR, c = (idx % VPR) * VN;
      r[i] = u32x4{0u, 0u, 0u, 0u};
      if (idx < TOT && t < valid) r[i] = *reinterpret_cast<const u32x4*>(src + t * rowstride + c);
    }
  }
  __device__ __forceinline__ void store(T* dst, int pitch, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < TOT) {
        const int t = idx / VPR, c = (idx % VPR) * VN;
        *reinterpret_cast<u32x4*>(dst + t * pitch + c) = r[i];
      }
    }
  }
  // Transposed copy: element (t, c + e) goes to dst[(c + e) * pitch + t].
  __device__ __forceinline__ void store_t(T* dst, int pitch, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * kThreads;
      if (idx < TOT) {
        const int t = idx / VPR, c = (idx % VPR) * VN;
        union {
          u32x4 u;
          T e[VN];
        } x;
        x.u = r[i];
#pragma unroll
        for (int e = 0; e < VN; ++e) dst[(c + e) * pitch + t] = x.e[e];
      }
    }
  }
};

// Zero `n` elements of an LDS array (n * sizeof(T) a multiple of 16 bytes).
template <typename T>
__device__ __forceinline__ void lds_zero(T* p, int n, int tid) {
  u32x4* v = reinterpret_cast<u32x4*>(p);
  const int nv = n * int(sizeof(T)) / 16;
  for (int i = tid; i < nv; i += kThreads) v[i] = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Stage 1: per-chunk UT transform.  One workgroup per (b, h, chunk).
//   G   = K K^T                                   (matrix cores; diagonal = lambda)
//   a_t = beta_t * phi(beta_t * lambda_t)         (fused coefficient)
//   X   = (I + diag(a) tril(G, -1))^{-1}          (blocked forward substitution, fp32)
//   T   = X diag(a)                               -> workspace [B,H,NC,C,C]
// The row scaling diag(a) is applied inside the solve instead of to G.
// The instance for the backward pass (BWD) also writes, in fp32 per chunk
// slot: X (C x C, zeros above the diagonal), a (C) and P = tril(Q K^T)
// (C x C, the diagonal included), all zero for tokens past the end.
// ---------------------------------------------------------------------------
template <typename T, int DK, int C, bool BWD = false>
__global__ __launch_bounds__(kThreads) void ut_transform_kernel(const T* __restrict__ k,
                                                                const T* __restrict__ beta,
                                                                T* __restrict__ tws, int H,
                                                                int64_t L, int NC, int rule,
                                                                const int32_t* __restrict__ cu, int N,
                                                                const T* __restrict__ q = nullptr,
                                                                float* __restrict__ xout = nullptr,
                                                                float* __restrict__ aout = nullptr,
                                                                float* __restrict__ pout = nullptr,
                                                                int64_t nwg_ut = 0,
                                                                int32_t* __restrict__ order = nullptr) {
  constexpr int DKP = round_up(DK, 32), CP = round_up(C, 32);
  constexpr int NRT = C / 16, NKU_D = DKP / 32;
  constexpr int KP = DKP + (sizeof(T) == 2 ? 8 : 4);
  constexpr int AP = C + 4;
  __shared__ __align__(16) T Ks[CP * KP];
  __shared__ __align__(16) T Qs[BWD ? CP * KP : 8];
  __shared__ float lam_s[CP], alpha_s[CP];
  __shared__ __align__(16) float Gs[C * AP];  // strictly lower part of K K^T
  __shared__ __align__(16) float Xs[C * AP];  // X = (I + A)^{-1}, lower blocks
  static_assert(sizeof(Ks) >= kRankSeqs * sizeof(int), "ranking workgroups reuse Ks");

  if (order != nullptr && int64_t(blockIdx.x) >= nwg_ut) {  // packed batch: rank the sequences
    rank_sequences<C>(cu, N, L, int(blockIdx.x - nwg_ut), order, reinterpret_cast<int*>(Ks));
    return;
  }
  const int64_t wg = blockIdx.x;  // workspace slot of this workgroup's chunk
  // slot -> sequence and chunk (dense: wg = (b H + h) NC + chunk)
  SeqSpan sp;
  int chunk;
  const int64_t h = cu == nullptr ? (wg / NC) % H : wg / NC;
  if (cu == nullptr) {
    chunk = int(wg % NC);
    sp = seq_span<C>(nullptr, int(wg / NC / H), h, H, L, NC);
  } else if (!slot_chunk<C>(cu, N, wg % NC, h, H, L, NC, sp, chunk)) {
    return;  // a slot no chunk of the packed batch uses (uniform: before any barrier)
  }
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t t0 = int64_t(chunk) * C;
  const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
  const int64_t row0 = (sp.bos + t0) * H + h;  // token t0 of this sequence and head

  if constexpr (DK < DKP || C < CP) {
    lds_zero(Ks, CP * KP, tid);
    if constexpr (BWD) lds_zero(Qs, CP * KP, tid);
  }
  float bt = 0.0f;
  if (tid < valid) bt = to_f32(beta[row0 + int64_t(tid) * H]);
  {
    RowStager<T, C, DK> sk, sq;
    sk.load(k + row0 * DK, int64_t(H) * DK, valid, tid);
    if constexpr (BWD) sq.load(q + row0 * DK, int64_t(H) * DK, valid, tid);
    if constexpr (DK < DKP || C < CP) __syncthreads();
    sk.store(Ks, KP, tid);
    if constexpr (BWD) sq.store(Qs, KP, tid);
  }
  __syncthreads();
  if constexpr (BWD) {
    // P = tril(Q K^T), diagonal included
    float* pdst = pout + wg * int64_t(C) * C;
    for (int i = w; i < NRT * NRT; i += 4) {
      const int r = i / NRT, c = i % NRT;
      f32x4 acc = zero4();
      if (c <= r) {
#pragma unroll
        for (int ku = 0; ku < NKU_D; ++ku)
          mma(acc, lds_frag(Qs, KP, 16 * r + li, ku, g), lds_frag(Ks, KP, 16 * c + li, ku, g));
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int ii = 16 * r + 4 * g + qq, jj = 16 * c + li;
        pdst[ii * C + jj] = jj <= ii ? acc[qq] : 0.0f;
      }
    }
  }

  // G tiles on and below the diagonal; the diagonal gives lambda.
  constexpr int NTILE = NRT * (NRT + 1) / 2;
  for (int i = w; i < NTILE; i += 4) {
    int r, c;
    lower_tile(i, r, c);
    f32x4 acc = zero4();
#pragma unroll
    for (int ku = 0; ku < NKU_D; ++ku)
      mma(acc, lds_frag(Ks, KP, 16 * r + li, ku, g), lds_frag(Ks, KP, 16 * c + li, ku, g));
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int ii = 16 * r + 4 * g + qq, jj = 16 * c + li;
      if (ii > jj) Gs[ii * AP + jj] = acc[qq];
      if (ii == jj) lam_s[ii] = acc[qq];
    }
  }
  __syncthreads();
  if (tid < C) alpha_s[tid] = (tid < valid) ? efla_alpha_rule(bt, lam_s[tid], rule) : 0.0f;
  __syncthreads();

  // Diagonal 16x16 blocks of X: forward substitution, one lane per column:
  //   x_r = delta_rc - a_r * sum_{m < r} G_rm x_m
  if (w < NRT && lane < 16) {
    const int base = 16 * w, c = lane;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = 0.0f;
#pragma unroll
      for (int m = 0; m < r; ++m) s = fmaf(Gs[(base + r) * AP + base + m], x[m], s);
      x[r] = (r == c ? 1.0f : 0.0f) - alpha_s[base + r] * s;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) Xs[(base + r) * AP + base + c] = x[r];
  }
  __syncthreads();

  // Off-diagonal blocks, one block row at a time (fp32 matrix cores):
  //   X_ij = -X_ii * diag(a_i) * sum_{j <= m < i} G_im X_mj
  for (int i = 1; i < NRT; ++i) {
    for (int j = w; j < i; j += 4) {
      f32x4 R = zero4();
      for (int m = j; m < i; ++m) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const float a = Gs[(16 * i + li) * AP + 16 * m + 4 * g + qq];
          const float bb = Xs[(16 * m + 4 * g + qq) * AP + 16 * j + li];
          R = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bb, R, 0, 0, 0);
        }
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) R[qq] *= alpha_s[16 * i + 4 * g + qq];
      f32x4 Y = zero4();
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const float a = Xs[(16 * i + li) * AP + 16 * i + 4 * g + qq];
        Y = __builtin_amdgcn_mfma_f32_16x16x4f32(a, R[qq], Y, 0, 0, 0);
      }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) Xs[(16 * i + 4 * g + qq) * AP + 16 * j + li] = -Y[qq];
    }
    __syncthreads();
  }

  if constexpr (BWD) {
    float* xdst = xout + wg * int64_t(C) * C;
    for (int i = tid; i < C * C; i += kThreads) {
      const int t = i / C, s = i % C;
      xdst[i] = s <= t ? Xs[t * AP + s] : 0.0f;
    }
    if (tid < C) aout[wg * int64_t(C) + tid] = alpha_s[tid];
  }

  // T = X diag(a), lower triangle, zeros above.
  constexpr int VN = Vec16<T>::n;
  constexpr int VPR = C / VN;
  T* out = tws + wg * int64_t(C) * C;
  for (int i = tid; i < C * VPR; i += kThreads) {
    const int t = i / VPR, s0 = (i % VPR) * VN;
    union {
      u32x4 u;
      T e[VN];
    } pk;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      const int s = s0 + e;
      pk.e[e] = from_f32<T>(s <= t ? Xs[t * AP + s] * alpha_s[s] : 0.0f);
    }
    *reinterpret_cast<u32x4*>(out + t * C + s0) = pk.u;
  }
}

// ---------------------------------------------------------------------------
// Stage 2: the sequential pass.  One workgroup of four wavefronts per
// (b, h, value block of BV columns); columns of S evolve independently, so
// value blocks are exact splits.  Wave w owns value tile cw = w % NCT and the
// key-dim k-units {pw, pw + NDP, ...} with pw = w / NCT: its part of S stays
// in registers (fp32) for the whole sequence.  Per chunk:
//   Y_p = K[:, dims_p] S_p,  Z_p = Q[:, dims_p] S_p     (partial, own dims)
//   P   = tril(Q K^T)                                    (shared via LDS)
//   Y = sum_p Y_p, Z = sum_p Z_p                         (LDS exchange)
//   U' = T (V - Y)          (every part computes all rows of its value tile)
//   S_p += K^T[dims_p, :] U'
//   O   = Z + P U'          (rows rt with rt % NDP == pw)
// The global loads of chunk n+1 are issued before chunk n is computed and land
// in LDS after it, so HBM latency overlaps the per-chunk dependency chain.
// ---------------------------------------------------------------------------
template <typename T, int DK, int C, int BV>
__global__ __launch_bounds__(kThreads) void recurrence_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ tws, const float* s0, T* __restrict__ o,
    float* sfin, int H, int64_t L, int NC, int DV, int NVB, int remap,
    const int32_t* __restrict__ cu, T* __restrict__ states = nullptr, int trans = 0,
    const int32_t* __restrict__ order = nullptr, int nseq = 0) {
  constexpr int DKP = round_up(DK, 32), CP = round_up(C, 32);
  constexpr int NRT = C / 16, NKU_D = DKP / 32, NKU_C = CP / 32;
  constexpr int NCT = BV / 16, NDP = 4 / NCT;
  constexpr int MAXO = cdiv(NKU_D, NDP);
  constexpr bool kBF16 = sizeof(T) == 2;
  constexpr int PADE = kBF16 ? 8 : 4;
  constexpr int QP = DKP + PADE, VP = BV + PADE, TP = CP + PADE;
  constexpr int KTP = CP + PADE;                 // pitch of the transposed K copy
  constexpr int NX = NDP > 1 ? NDP * NRT * NCT * kWave : 1;
  constexpr int OP = 16 + PADE;                  // pitch of a wave's output staging tile
  static_assert(NCT * NDP == 4, "four wavefronts per workgroup");
  __shared__ __align__(16) T Qs[CP * QP];
  __shared__ __align__(16) T Ks[CP * QP];
  __shared__ __align__(16) T Kt[kBF16 ? DKP * KTP : 8];  // K^T for the state update (bf16)
  __shared__ __align__(16) T Vs[C * VP];
  __shared__ __align__(16) T Ts[C * TP];
  __shared__ __align__(16) T Ps[C * TP];
  __shared__ __align__(16) T Os[4 * 16 * OP];
  __shared__ __align__(16) f32x4 Xy[NX];
  __shared__ __align__(16) f32x4 Xz[NX];

  // Workgroup -> (bh, value block).  With remap, all value blocks of one (b, h)
  // get the same blockIdx % 8, i.e. the same XCD and L2, so their shared reads
  // of q, k and T hit one cache.
  const int x = blockIdx.x;
  int bh, vb;
  if (remap) {
    const int slot = x >> 3;
    vb = slot % NVB;
    bh = (slot / NVB) * 8 + (x & 7);
  } else {
    bh = x / NVB;
    vb = x % NVB;
  }
  if (order != nullptr) bh = seq_of_rank(order, bh / H, nseq) * H + bh % H;  // packed: longest first
  const int64_t h = bh % H;
  const SeqSpan sp = seq_span<C>(cu, bh / H, h, H, L, NC);  // sequence bh / H
  const int nc = sp.nc;
  const int v0 = vb * BV;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int cw = w % NCT, pw = w / NCT;
  const int col = v0 + 16 * cw + li;  // this lane's value column
  T* Ow = Os + w * 16 * OP;            // this wave's output staging tile

  // Zero what staging never writes: padding rows/columns and the upper part of P.
  if constexpr (DK < DKP || C < CP) {
    lds_zero(Qs, CP * QP, tid);
    lds_zero(Ks, CP * QP, tid);
    if constexpr (kBF16) lds_zero(Kt, DKP * KTP, tid);
  }
  if constexpr (C < CP) lds_zero(Ts, C * TP, tid);
  lds_zero(Ps, C * TP, tid);

  // S tiles: Sacc[j][hh] covers key dims 32*ku + 16*hh + (0..15), ku = pw + j*NDP.
  f32x4 Sacc[MAXO][2];
#pragma unroll
  for (int j = 0; j < MAXO; ++j) {
    const int ku = pw + j * NDP;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int dim = 32 * ku + 16 * hh + 4 * g + qq;
        // trans: the chunk-transition run, from the identity with V = 0
        Sacc[j][hh][qq] = trans ? (dim == col ? 1.0f : 0.0f)
                        : (s0 != nullptr && ku < NKU_D && dim < DK) ? s0[(int64_t(bh) * DK + dim) * DV + col] : 0.0f;
      }
  }

  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;
  RowStager<T, C, DK> sq, sk;
  RowStager<T, C, BV> sv;
  RowStager<T, C, C> st;
  auto load_chunk = [&](int n) {
    const int64_t t0 = int64_t(n) * C;
    const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
    const int64_t row0 = (sp.bos + t0) * H + h;
    sq.load(q + row0 * DK, qk_stride, valid, tid);
    sk.load(k + row0 * DK, qk_stride, valid, tid);
    sv.load(v + row0 * DV + v0, v_stride, trans ? 0 : valid, tid);
    st.load(tws + (sp.slot0 + n) * C * C, C, C, tid);
  };
  auto store_chunk = [&]() {
    sq.store(Qs, QP, tid);
    sk.store(Ks, QP, tid);
    if constexpr (kBF16) sk.store_t(Kt, KTP, tid);
    sv.store(Vs, VP, tid);
    st.store(Ts, TP, tid);
  };

  if (nc > 0) load_chunk(0);
  __syncthreads();  // zero-fill done
  if (nc > 0) store_chunk();
  __syncthreads();

  for (int n = 0; n < nc; ++n) {
    const int64_t t0 = int64_t(n) * C;
    const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
    const int64_t row0 = (sp.bos + t0) * H + h;
    if (n + 1 < nc) load_chunk(n + 1);  // in flight during this chunk
    if (states != nullptr) {  // the state at the start of this chunk (backward pass)
      T* dst = states + (sp.slot0 + n) * DK * DV;
#pragma unroll
      for (int j = 0; j < MAXO; ++j) {
        const int ku = pw + j * NDP;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int dim = 32 * ku + 16 * hh + 4 * g + qq;
            if (ku < NKU_D && dim < DK) dst[dim * DV + col] = from_f32<T>(Sacc[j][hh][qq]);
          }
      }
    }

    // partial K S and Q S over this wave's key dims
    f32x4 Y[NRT], Z[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      Y[rt] = zero4();
      Z[rt] = zero4();
    }
#pragma unroll
    for (int j = 0; j < MAXO; ++j) {
      const int ku = pw + j * NDP;
      if (ku < NKU_D) {
        const Frag<T> bS = acc_frag<T>(Sacc[j][0], Sacc[j][1]);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          mma(Y[rt], lds_frag(Ks, QP, 16 * rt + li, ku, g), bS);
          mma(Z[rt], lds_frag(Qs, QP, 16 * rt + li, ku, g), bS);
        }
      }
    }

    // P = tril(Q K^T), computed as P^T tiles (s-tile c <= t-tile r), into LDS.
    constexpr int NTILE = NRT * (NRT + 1) / 2;
    for (int i = w; i < NTILE; i += 4) {
      int r, c;
      lower_tile(i, r, c);
      f32x4 acc = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
        mma(acc, lds_frag(Ks, QP, 16 * c + li, ku, g), lds_frag(Qs, QP, 16 * r + li, ku, g));
      // acc[qq] = P[t = 16r + li][s = 16c + 4g + qq]
      if (r == c) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (4 * g + qq > li) acc[qq] = 0.0f;
      }
      st4(Ps + (16 * r + li) * TP + 16 * c + 4 * g, acc);
    }

    if constexpr (NDP > 1) {
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        Xy[((pw * NRT + rt) * NCT + cw) * kWave + lane] = Y[rt];
        Xz[((pw * NRT + rt) * NCT + cw) * kWave + lane] = Z[rt];
      }
    }
    __syncthreads();
    if constexpr (NDP > 1) {
      // Sum the partials in part order 0..NDP-1 (own part from registers), so
      // every part of a value tile gets bitwise the same K S.
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f32x4 sy = zero4(), sz = zero4();
#pragma unroll
        for (int p = 0; p < NDP; ++p) {
          if (p == pw) {
            sy += Y[rt];
            sz += Z[rt];
          } else {
            sy += Xy[((p * NRT + rt) * NCT + cw) * kWave + lane];
            if (rt % NDP == pw) sz += Xz[((p * NRT + rt) * NCT + cw) * kWave + lane];
          }
        }
        Y[rt] = sy;
        Z[rt] = sz;
      }
    }

    // D = V - K S  (in place of Y), then U' = T D
    f32x4 U[2 * NKU_C];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        Y[rt][qq] = to_f32(Vs[(16 * rt + 4 * g + qq) * VP + 16 * cw + li]) - Y[rt][qq];
#pragma unroll
    for (int rt = 0; rt < 2 * NKU_C; ++rt) {
      U[rt] = zero4();
      if (rt < NRT) {
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku) {
          if (32 * ku <= 16 * rt + 15) {
            const f32x4 dlo = Y[2 * ku];
            const f32x4 dhi = (2 * ku + 1 < NRT) ? Y[(2 * ku + 1) % NRT] : zero4();
            mma(U[rt], lds_frag(Ts, TP, 16 * rt + li, ku, g), acc_frag<T>(dlo, dhi));
          }
        }
      }
    }

    // S_p += K^T[dims_p, :] U'
#pragma unroll
    for (int j = 0; j < MAXO; ++j) {
      const int ku = pw + j * NDP;
      if (ku < NKU_D) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int dt = 2 * ku + hh;
          if (16 * dt < DK) {
#pragma unroll
            for (int kt = 0; kt < NKU_C; ++kt) {
              Frag<T> aK;
              if constexpr (kBF16)
                aK = lds_frag(Kt, KTP, 16 * dt + li, kt, g);
              else
                aK = lds_frag_t(Ks, QP, 16 * dt + li, kt, g);
              mma(Sacc[j][hh], aK, acc_frag<T>(U[2 * kt], U[2 * kt + 1]));
            }
          }
        }
      }
    }

    // O = Q S + P U' for this wave's rows, staged through a wave-private LDS
    // tile so that each row leaves as whole 16-byte stores.
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      if (rt % NDP == pw) {
        f32x4 acc = Z[rt];
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15)
            mma(acc, lds_frag(Ps, TP, 16 * rt + li, ku, g), acc_frag<T>(U[2 * ku], U[2 * ku + 1]));
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) Ow[(4 * g + qq) * OP + li] = from_f32<T>(acc[qq]);
        constexpr int VN = Vec16<T>::n, VPRow = 16 / VN;  // vectors per 16-wide row
        if (lane < 16 * VPRow) {
          const int r = lane / VPRow, c = (lane % VPRow) * VN;
          const int t = 16 * rt + r;
          const u32x4 val = *reinterpret_cast<const u32x4*>(Ow + r * OP + c);
          if (t < valid && o != nullptr)
            *reinterpret_cast<u32x4*>(o + (row0 + int64_t(t) * H) * DV + v0 + 16 * cw + c) = val;
        }
      }
    }

    __syncthreads();  // every wave is done reading this chunk's LDS
    if (n + 1 < nc) store_chunk();
    __syncthreads();
  }

  if (sfin != nullptr) {
#pragma unroll
    for (int j = 0; j < MAXO; ++j) {
      const int ku = pw + j * NDP;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int dim = 32 * ku + 16 * hh + 4 * g + qq;
          if (ku < NKU_D && dim < DK) sfin[(int64_t(bh) * DK + dim) * DV + col] = Sacc[j][hh][qq];
        }
    }
  }
}

template <typename T, int DK, int C>
hipError_t ut_transform_launch_impl(const T* k, const T* beta, T* tws, int B, int H, int64_t L, int rule,
                                    const int32_t* cu, int N, int32_t* order, hipStream_t stream) {
  const int NC = cu == nullptr ? int((L + C - 1) / C) : int(L / C) + N;  // chunk slots per sequence / head
  const int64_t nwg = int64_t(cu == nullptr ? B : 1) * H * NC;
  if (cu == nullptr) order = nullptr;
  const int64_t nrank = order != nullptr ? (N + kRankSeqs - 1) / kRankSeqs : 0;
  if (nwg + nrank == 0) return hipSuccess;
  hipLaunchKernelGGL((ut_transform_kernel<T, DK, C>), dim3(unsigned(nwg + nrank)), dim3(kThreads), 0, stream,
                     k, beta, tws, H, L, NC, rule, cu, N, nullptr, nullptr, nullptr, nullptr, nwg, order);
  return hipGetLastError();
}

template <typename T, int DK, int C, int BV>
hipError_t recurrence_launch_impl(const T* q, const T* k, const T* v, const T* tws, const float* s0,
                                  T* o, float* sfin, int B, int H, int64_t L, int DV,
                                  const int32_t* cu, int N, hipStream_t stream, int trans, const int32_t* order) {
  const int NC = cu == nullptr ? int((L + C - 1) / C) : int(L / C) + N;
  const int BH = (cu == nullptr ? B : N) * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  if (cu == nullptr) order = nullptr;  // dense batches keep their order
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((recurrence_kernel<T, DK, C, BV>), dim3(unsigned(nwg)), dim3(kThreads), 0, stream,
                     q, k, v, tws, s0, o, sfin, H, L, NC, DV, NVB, remap, cu, static_cast<T*>(nullptr), trans,
                     order, N);
  return hipGetLastError();
}

template <typename T, int DK>
hipError_t ut_dispatch_c(const T* k, const T* beta, T* tws, int B, int H, int64_t L, int C, int rule,
                         const int32_t* cu, int N, int32_t* order, hipStream_t s) {
  switch (C) {
    case 16: return ut_transform_launch_impl<T, DK, 16>(k, beta, tws, B, H, L, rule, cu, N, order, s);
    case 32: return ut_transform_launch_impl<T, DK, 32>(k, beta, tws, B, H, L, rule, cu, N, order, s);
    case 64: return ut_transform_launch_impl<T, DK, 64>(k, beta, tws, B, H, L, rule, cu, N, order, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_ut_transform(const T* k, const T* beta, T* tws, int B, int H, int64_t L, int DK,
                               int C, int rule, const int32_t* cu, int N, hipStream_t s, int32_t* order) {
  switch (DK) {
    case 16: return ut_dispatch_c<T, 16>(k, beta, tws, B, H, L, C, rule, cu, N, order, s);
    case 32: return ut_dispatch_c<T, 32>(k, beta, tws, B, H, L, C, rule, cu, N, order, s);
    case 64: return ut_dispatch_c<T, 64>(k, beta, tws, B, H, L, C, rule, cu, N, order, s);
    case 128: return ut_dispatch_c<T, 128>(k, beta, tws, B, H, L, C, rule, cu, N, order, s);
  }
  return hipErrorInvalidValue;
}

// Value-block widths compiled per element type: bf16 gets 16/32/64, fp32 16.
template <typename T> struct BVSet { static constexpr bool has32 = true, has64 = true; };
template <> struct BVSet<float> { static constexpr bool has32 = false, has64 = false; };

template <typename T, int DK, int C>
hipError_t rec_dispatch_bv(const T* q, const T* k, const T* v, const T* tws, const float* s0, T* o,
                           float* sfin, int B, int H, int64_t L, int DV, int BV, const int32_t* cu, int N,
                           hipStream_t s, int trans, const int32_t* order) {
  if (BV == 16) return recurrence_launch_impl<T, DK, C, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, s, trans, order);
  if constexpr (BVSet<T>::has32)
    if (BV == 32) return recurrence_launch_impl<T, DK, C, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, s, trans, order);
  if constexpr (BVSet<T>::has64)
    if (BV == 64) return recurrence_launch_impl<T, DK, C, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, s, trans, order);
  return hipErrorInvalidValue;
}

template <typename T, int DK>
hipError_t rec_dispatch_c(const T* q, const T* k, const T* v, const T* tws, const float* s0, T* o,
                          float* sfin, int B, int H, int64_t L, int DV, int C, int BV, const int32_t* cu,
                          int N, hipStream_t s, int trans, const int32_t* order) {
  switch (C) {
    case 16: return rec_dispatch_bv<T, DK, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, s, trans, order);
    case 32: return rec_dispatch_bv<T, DK, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, s, trans, order);
    case 64: return rec_dispatch_bv<T, DK, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, s, trans, order);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_recurrence(const T* q, const T* k, const T* v, const T* tws, const float* s0,
                             T* o, float* sfin, int B, int H, int64_t L, int DK, int DV, int C,
                             int BV, const int32_t* cu, int N, hipStream_t s, int trans, const int32_t* order) {
  switch (DK) {
    case 16: return rec_dispatch_c<T, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, C, BV, cu, N, s, trans, order);
    case 32: return rec_dispatch_c<T, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, C, BV, cu, N, s, trans, order);
    case 64: return rec_dispatch_c<T, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, C, BV, cu, N, s, trans, order);
    case 128: return rec_dispatch_c<T, 128>(q, k, v, tws, s0, o, sfin, B, H, L, DV, C, BV, cu, N, s, trans, order);
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
