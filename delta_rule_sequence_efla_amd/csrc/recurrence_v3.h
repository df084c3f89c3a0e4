// recurrence_v3.h -- the sequential chunk pass for bf16 inputs, one wavefront
// per 16-column tile of the state.
//
// Same algebra as recurrence_kernel (chunk_kernels.h):
//     U' = T (V - K S),   O = Q S + tril(Q K^T) U',   S <- S + K^T U'
// but laid out so that the per-chunk dependency chain S -> K S -> U' -> S
// never leaves one wavefront:
//   * wave w of a workgroup owns value columns v0 + 16w .. v0 + 16w + 15 and
//     ALL key dims of S (d_k/16 fp32 accumulator tiles): no partial sums to
//     exchange, no barrier inside a chunk;
//   * K^T and the V tile are read from row-major LDS with the gfx950
//     transposing read ds_read_b64_tr_b16 (no transposed copy);
//   * P = tril(Q K^T) stays in registers as the A operand of P U';
//   * the workgroup's chunk inputs (Q, K, V block, T) go global -> registers
//     two chunks ahead and registers -> LDS one chunk ahead, into a
//     double-buffered LDS slot, with one barrier per chunk.
#pragma once

#include "chunk_kernels.h"

namespace efla {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives halfword
// (i % 4) of the 8-byte words addressed by lanes 4e + i/4, e = 0..3.  So if
// lane j addresses row r0 + j/4, columns c0 + 4(j%4) .. +3 of a row-major
// bf16 matrix, lane i receives column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p)));
  return __builtin_bit_cast(bf16x4, v);
}

// Operand fragment of X^T for operand row m0 + li, k-unit ku, where X is a
// row-major LDS matrix [k][m]: element e carries X[32ku + 16(e/4) + 4g + e%4][m0 + li].
__device__ __forceinline__ Frag<uint16_t> lds_frag_tr(const uint16_t* X, int pitch, int m0, int ku,
                                                      int lane) {
  const int j = lane & 15, g = lane >> 4;
  const uint16_t* p = X + (32 * ku + 4 * g + (j >> 2)) * pitch + m0 + 4 * (j & 3);
  const bf16x4 lo = lds_read_tr(p);
  const bf16x4 hi = lds_read_tr(p + 16 * pitch);
  Frag<uint16_t> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

template <int DK, int C, int BV>
struct V3Shape {
  static constexpr int NW = BV / 16;                  // wavefronts = value tiles
  static constexpr int THREADS = NW * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int PADE = 8;
  static constexpr int QP = DK + PADE, TP = C + PADE, VP = BV + PADE, OP = 16 + PADE;
  static constexpr int SLOT = 2 * C * QP + C * TP + C * VP;  // elements per LDS slot
  static constexpr int QOFF = 0, KOFF = C * QP, TOFF = 2 * C * QP, VOFF = 2 * C * QP + C * TP;
};

// Rows of a strided global matrix staged through registers by THREADS lanes.
template <int ROWS, int COLS, int THREADS>
struct RegStage {
  static constexpr int VPR = COLS / 8, TOT = ROWS * VPR, CNT = (TOT + THREADS - 1) / THREADS;
  u32x4 r[CNT];
  // Rows at or past `valid` re-read row 0 of the chunk: they are never used
  // unmasked (T is zero in those rows and columns), so any finite data will do.
  __device__ __forceinline__ void load(const uint16_t* src, int64_t rowstride, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * THREADS;
      if (TOT % THREADS == 0 || idx < TOT) {
        int t = idx / VPR;
        const int c = (idx % VPR) * 8;
        t = t < valid ? t : 0;
        r[i] = *reinterpret_cast<const u32x4*>(src + t * rowstride + c);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int pitch, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * THREADS;
      if (TOT % THREADS == 0 || idx < TOT) {
        const int t = idx / VPR, c = (idx % VPR) * 8;
        *reinterpret_cast<u32x4*>(dst + t * pitch + c) = r[i];
      }
    }
  }
};

template <int DK, int C, int BV>
struct V3Stager {
  using S = V3Shape<DK, C, BV>;
  RegStage<C, DK, S::THREADS> q, k;
  RegStage<C, C, S::THREADS> t;
  RegStage<C, BV, S::THREADS> v;
  __device__ __forceinline__ void load(const uint16_t* qg, const uint16_t* kg, const uint16_t* vg,
                                       const uint16_t* tg, int64_t qk_stride, int64_t v_stride,
                                       int valid, int tid) {
    q.load(qg, qk_stride, valid, tid);
    k.load(kg, qk_stride, valid, tid);
    t.load(tg, C, C, tid);
    v.load(vg, v_stride, valid, tid);
  }
  __device__ __forceinline__ void store(uint16_t* slot, int tid) const {
    q.store(slot + S::QOFF, S::QP, tid);
    k.store(slot + S::KOFF, S::QP, tid);
    t.store(slot + S::TOFF, S::TP, tid);
    v.store(slot + S::VOFF, S::VP, tid);
  }
};

template <int DK, int C, int BV>
__global__ __launch_bounds__(4 * BV) void recurrence_v3_kernel(  // 4*BV = (BV/16) wavefronts
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ tws, const float* __restrict__ s0, uint16_t* __restrict__ o,
    float* __restrict__ sfin, int H, int64_t L, int NC, int DV, int NVB, int remap) {
  using S = V3Shape<DK, C, BV>;
  constexpr int NRT = S::NRT, NDT = S::NDT, NKU_D = S::NKU_D, NKU_C = S::NKU_C;
  constexpr int QP = S::QP, TP = S::TP, VP = S::VP, OP = S::OP;
  __shared__ __align__(16) uint16_t lds[2 * S::SLOT];
  __shared__ __align__(16) uint16_t Os[S::NW * 16 * OP];

  const int x = blockIdx.x;
  int bh, vb;
  if (remap) {  // all value blocks of one (b, h) on one XCD (same blockIdx % 8)
    const int slot = x >> 3;
    vb = slot % NVB;
    bh = (slot / NVB) * 8 + (x & 7);
  } else {
    bh = x / NVB;
    vb = x % NVB;
  }
  const int64_t b = bh / H, h = bh % H;
  const int v0 = vb * BV;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int col = v0 + 16 * w + li;
  uint16_t* Ow = Os + w * 16 * OP;

  // state tiles: S[dt] holds key dims 16 dt + 4g + (0..3), value column `col`
  f32x4 St[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      St[dt][qq] = s0 != nullptr ? s0[(int64_t(bh) * DK + 16 * dt + 4 * g + qq) * DV + col] : 0.0f;

  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;
  auto chunk_valid = [&](int n) { return int(L - int64_t(n) * C < C ? L - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (b * L + int64_t(n) * C) * H + h; };
  V3Stager<DK, C, BV> stg;  // registers holding the chunk after the next
  auto load_chunk = [&](int n) {
    const int64_t r0 = row_of(n);
    stg.load(q + r0 * DK, k + r0 * DK, v + r0 * DV + v0, tws + (int64_t(bh) * NC + n) * C * C, qk_stride,
             v_stride, chunk_valid(n), tid);
  };

  if (NC > 0) {
    load_chunk(0);
    stg.store(lds, tid);
  }
  if (NC > 1) load_chunk(1);
  __syncthreads();

  for (int n = 0; n < NC; ++n) {
    uint16_t* cur = lds + (n & 1) * S::SLOT;
    uint16_t* nxt = lds + ((n + 1) & 1) * S::SLOT;
    const uint16_t* Qs = cur + S::QOFF;
    const uint16_t* Ks = cur + S::KOFF;
    const uint16_t* Ts = cur + S::TOFF;
    const uint16_t* Vs = cur + S::VOFF;
    const int valid = chunk_valid(n);
    const int64_t row0 = row_of(n);

    // chunk n+1 (already in registers) goes to the other slot; chunk n+2 is
    // fetched into the registers just freed and stays in flight while chunk n
    // is computed.
    if (n + 1 < NC) stg.store(nxt, tid);
    if (n + 2 < NC) load_chunk(n + 2);

    // S as bf16 B operands, one per 32 key dims
    Frag<uint16_t> bS[NKU_D];
#pragma unroll
    for (int ku = 0; ku < NKU_D; ++ku) bS[ku] = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);

    // Y = K S and Z = Q S (all rows of this chunk, this wave's 16 columns)
    f32x4 Y[NRT], Z[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      Y[rt] = zero4();
      Z[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        mma(Y[rt], lds_frag(Ks, QP, 16 * rt + li, ku, g), bS[ku]);
        mma(Z[rt], lds_frag(Qs, QP, 16 * rt + li, ku, g), bS[ku]);
      }
    }

    // P^T tiles (s-tile c <= t-tile r): P[16r + li][16c + 4g + qq] in Pt[r][c][qq]
    f32x4 Pt[NRT][NRT];
#pragma unroll
    for (int r = 0; r < NRT; ++r)
#pragma unroll
      for (int c = 0; c < NRT; ++c) {
        Pt[r][c] = zero4();
        if (c <= r) {
#pragma unroll
          for (int ku = 0; ku < NKU_D; ++ku)
            mma(Pt[r][c], lds_frag(Ks, QP, 16 * c + li, ku, g), lds_frag(Qs, QP, 16 * r + li, ku, g));
          if (c == r) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              if (4 * g + qq > li) Pt[r][c][qq] = 0.0f;
          }
        }
      }

    // D = V - K S  (V tile read transposed: rows 16rt + 4g + e, column li)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int j = lane & 15;
      const bf16x4 vv = lds_read_tr(Vs + (16 * rt + 4 * g + (j >> 2)) * VP + 16 * w + 4 * (j & 3));
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) Y[rt][qq] = static_cast<float>(vv[qq]) - Y[rt][qq];
    }

    // U' = T D
    f32x4 U[2 * NKU_C];
#pragma unroll
    for (int rt = 0; rt < 2 * NKU_C; ++rt) {
      U[rt] = zero4();
      if (rt < NRT) {
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15)
            mma(U[rt], lds_frag(Ts, TP, 16 * rt + li, ku, g), acc_frag<uint16_t>(Y[2 * ku], Y[2 * ku + 1]));
      }
    }
    Frag<uint16_t> bU[NKU_C];
#pragma unroll
    for (int ku = 0; ku < NKU_C; ++ku) bU[ku] = acc_frag<uint16_t>(U[2 * ku], U[2 * ku + 1]);

    // S += K^T U'
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kt = 0; kt < NKU_C; ++kt) mma(St[dt], lds_frag_tr(Ks, QP, 16 * dt, kt, lane), bU[kt]);

    // O = Q S + P U', staged through this wave's LDS tile into 16-byte row stores
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 acc = Z[rt];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku <= 16 * rt + 15) {
          const f32x4 plo = Pt[rt][2 * ku];
          const f32x4 phi = (2 * ku + 1 <= rt) ? Pt[rt][(2 * ku + 1) % NRT] : zero4();
          mma(acc, acc_frag<uint16_t>(plo, phi), bU[ku]);
        }
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) Ow[(4 * g + qq) * OP + li] = from_f32<uint16_t>(acc[qq]);
      if (lane < 32) {
        const int r = lane >> 1, c8 = (lane & 1) * 8;
        const int t = 16 * rt + r;
        const u32x4 val = *reinterpret_cast<const u32x4*>(Ow + r * OP + c8);
        if (t < valid) *reinterpret_cast<u32x4*>(o + (row0 + int64_t(t) * H) * DV + v0 + 16 * w + c8) = val;
      }
    }
    __syncthreads();
  }

  if (sfin != nullptr) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sfin[(int64_t(bh) * DK + 16 * dt + 4 * g + qq) * DV + col] = St[dt][qq];
  }
}

// Shapes this kernel covers (bf16, d_k >= 32, chunk >= 32); others use recurrence_kernel.
inline bool v3_supported(int DK, int C) { return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64); }

template <int DK, int C, int BV>
hipError_t recurrence_v3_launch_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DV, hipStream_t stream) {
  using S = V3Shape<DK, C, BV>;
  const int NC = int((L + C - 1) / C);
  const int BH = B * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((recurrence_v3_kernel<DK, C, BV>), dim3(unsigned(nwg)), dim3(S::THREADS), 0, stream, q,
                     k, v, tws, s0, o, sfin, H, L, NC, DV, NVB, remap);
  return hipGetLastError();
}

template <int DK, int C>
hipError_t recurrence_v3_bv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* tws,
                            const float* s0, uint16_t* o, float* sfin, int B, int H, int64_t L, int DV,
                            int BV, hipStream_t s) {
  switch (BV) {
    case 16: return recurrence_v3_launch_impl<DK, C, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
    case 32: return recurrence_v3_launch_impl<DK, C, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
    case 64: return recurrence_v3_launch_impl<DK, C, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
  }
  return hipErrorInvalidValue;
}

inline hipError_t launch_recurrence_v3(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       hipStream_t s) {
  if (C == 32) {
    switch (DK) {
      case 32: return recurrence_v3_bv<32, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_v3_bv<64, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_v3_bv<128, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return recurrence_v3_bv<32, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_v3_bv<64, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_v3_bv<128, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
