// recurrence_v5.h -- the sequential chunk pass for bf16 inputs with the work
// of each 16-column state tile split between two wavefronts.
//
// Per chunk (start state S, T from the UT transform):
//     U' = T (V - K S),   S <- S + K^T U',   O = Q S + tril(Q K^T) U'
// The dependency chain S -> K S -> U' -> S is short; the output products
// (Q S, tril(Q K^T), P U') are off the chain.  A workgroup for BV value
// columns therefore runs 2 * BV/16 wavefronts:
//   * chain wave c (value tile c) keeps its 16 columns of S in fp32 registers
//     and per chunk forms Y = K S, D = V - Y, U' = T D, then S += K^T U';
//     it publishes U' and the next chunk's S as bf16 operand fragments in LDS;
//   * output wave c reads those fragments and forms Z = Q S, its share of
//     P = tril(Q K^T) (rows split between the output waves, shared via LDS)
//     and O = Z + P U'; the output waves also stream the chunk inputs into
//     the three-slot LDS ring by DMA (the scheme of recurrence_v4.h).
// Per chunk: barrier A (chunk n and S_n visible) -> chain: Y, U' | output: Z, P
// -> barrier B (U', P visible) -> chain: S update, publish S_{n+1} | output: O.
// On a 1.3B-shaped layer this keeps all four SIMDs of a CU busy, where one
// wavefront per tile could use only half of them.
#pragma once

#include "recurrence_v4.h"

namespace efla {

// s_waitcnt lgkmcnt(0) only: this wave's LDS writes are complete.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14)); }

template <int DK, int C, int BV>
struct V5Shape {
  static constexpr int NT = BV / 16;          // chain waves = output waves = value tiles
  static constexpr int THREADS = 2 * NT * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;
  // P fragments (row tile rt, k-unit ku) with 32 ku <= 16 rt + 15, in a flat list
  static constexpr int NPF = (NRT == 4) ? 6 : 2;
  using Dma = ChunkDma<DK, C, BV, NT>;  // issued by the NT output waves
  static constexpr int DMA_PER_WAVE = Dma::COUNT;
  static constexpr int STORES_PER_WAVE = NRT;
};

// index of P fragment (rt, ku) in the flat list (row tiles 0..NRT-1, ku <= rt/2)
__device__ __forceinline__ constexpr int pf_index(int rt, int ku) {
  // rt=0:(0,0)->0 rt=1:(1,0)->1 rt=2:(2,0)->2,(2,1)->3 rt=3:(3,0)->4,(3,1)->5
  return rt < 2 ? rt : 2 + 2 * (rt - 2) + ku;
}

template <int DK, int C, int BV>
__global__ __launch_bounds__(8 * BV) void recurrence_v5_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ tws, const float* __restrict__ s0, uint16_t* __restrict__ o,
    float* __restrict__ sfin, int H, int64_t L, int NC, int DV, int NVB, int remap) {
  using S = V5Shape<DK, C, BV>;
  constexpr int NT = S::NT, NRT = S::NRT, NDT = S::NDT, NKU_D = S::NKU_D, NKU_C = S::NKU_C;
  constexpr int NPF = S::NPF;
  __shared__ __align__(1024) uint16_t slot0[S::SLOT];
  __shared__ __align__(1024) uint16_t slot1[S::SLOT];
  __shared__ __align__(1024) uint16_t slot2[S::SLOT];
  __shared__ __align__(16) bf16x8 bS_buf[NT][NKU_D][kWave];  // S_n as B fragments, per tile
  __shared__ __align__(16) bf16x8 bU_buf[NT][NKU_C][kWave];  // U'_n as B fragments, per tile
  __shared__ __align__(16) bf16x8 P_buf[NPF][kWave];         // P_n as A fragments

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
  const bool chain = w < NT;
  const int tile = chain ? w : w - NT;  // value tile of this wave
  const int col = v0 + 16 * tile + li;

  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;
  auto chunk_valid = [&](int n) { return int(L - int64_t(n) * C < C ? L - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (b * L + int64_t(n) * C) * H + h; };
  typename S::Dma dma;  // used by the output waves
  dma.init(qk_stride, v_stride, lane, tile);
  auto chunk_src = [&](int n) {  // clamped to the last chunk (fixed transfer count)
    const int nn = n < NC ? n : NC - 1;
    const int64_t r0 = row_of(nn);
    using U = const uint16_t*;
    return typename S::Dma::Src{(U)uniform_ptr(q + r0 * DK), (U)uniform_ptr(k + r0 * DK),
                                (U)uniform_ptr(tws + (int64_t(bh) * NC + nn) * C * C),
                                (U)uniform_ptr(v + r0 * DV + v0), chunk_valid(nn)};
  };

  // chain waves: the state tile (fp32) and its bf16 operand fragments
  f32x4 St[NDT];
  Frag<uint16_t> bS[NKU_D];
  if (chain) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        St[dt][qq] = s0 != nullptr ? s0[(int64_t(bh) * DK + 16 * dt + 4 * g + qq) * DV + col] : 0.0f;
#pragma unroll
    for (int ku = 0; ku < NKU_D; ++ku) {
      bS[ku] = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);
      bS_buf[tile][ku][lane] = bS[ku].v;
    }
  } else if (NC > 0) {
    dma.issue_part(0, 1, lds_addr_of(slot0), chunk_src(0));
    dma.issue_part(0, 1, lds_addr_of(slot1), chunk_src(1));
  }

  constexpr int D = S::DMA_PER_WAVE, ST = S::STORES_PER_WAVE;
  auto chunk_step = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ fill, int n) {
    const uint16_t* Qs = cur + S::QOFF;
    const uint16_t* Ks = cur + S::KOFF;
    const uint16_t* Ts = cur + S::TOFF;
    const uint16_t* Vs = cur + S::VOFF;
    if (!chain) {
      // this wave's transfers of chunk n are complete once at most the
      // operations issued after them are outstanding
      if (n == 0) wait_vmcnt<D>();
      else if (n == 1) wait_vmcnt<D + ST>();
      else wait_vmcnt<D + 2 * ST>();
    }
    wait_lgkm0();
    barrier_nowait();  // A: chunk n and S_n visible; U', P buffers free

    if (chain) {
      // ---- chain phase 1: Y = K S, D = V - Y, U' = T D -> publish U'
      bf16x4 Vt[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int j = lane & 15;
        Vt[rt] = lds_read_tr(Vs + swz_off<BV>(16 * rt + 4 * g + (j >> 2), 16 * tile + 4 * (j & 3)));
      }
      Frag<uint16_t> Tf[NRT][NKU_C];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15) Tf[rt][ku] = sw_frag<C>(Ts, 16 * rt + li, ku, g);
      f32x4 Y[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Y[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        Frag<uint16_t> Kf[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Kf[rt] = sw_frag<DK>(Ks, 16 * rt + li, ku, g);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mma(Y[rt], Kf[rt], bS[ku]);
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) Y[rt][qq] = static_cast<float>(Vt[rt][qq]) - Y[rt][qq];
      Frag<uint16_t> bD[NKU_C];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        bD[ku] = acc_frag<uint16_t>(Y[2 * ku], 2 * ku + 1 < NRT ? Y[(2 * ku + 1) % NRT] : zero4());
      f32x4 U[2 * NKU_C];
#pragma unroll
      for (int rt = 0; rt < 2 * NKU_C; ++rt) {
        U[rt] = zero4();
        if (rt < NRT) {
#pragma unroll
          for (int ku = 0; ku < NKU_C; ++ku)
            if (32 * ku <= 16 * rt + 15) mma(U[rt], Tf[rt][ku], bD[ku]);
        }
      }
      Frag<uint16_t> bU[NKU_C];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) {
        bU[ku] = acc_frag<uint16_t>(U[2 * ku], U[2 * ku + 1]);
        bU_buf[tile][ku][lane] = bU[ku].v;
      }
      // K^T fragments for the update: the first half is fetched before the
      // barrier, the second half right after it.
      constexpr int NH = (NDT + 1) / 2;
      Frag<uint16_t> KTa[NH][NKU_C], KTb[NH][NKU_C];
#pragma unroll
      for (int dt = 0; dt < NH; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) KTa[dt][kt] = sw_frag_tr<DK>(Ks, 16 * dt, kt, lane);

      wait_lgkm0();
      barrier_nowait();  // B: U' and P visible

      // ---- chain phase 2: S += K^T U', publish S_{n+1}
#pragma unroll
      for (int dt = NH; dt < NDT; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) KTb[dt - NH][kt] = sw_frag_tr<DK>(Ks, 16 * dt, kt, lane);
#pragma unroll
      for (int dt = 0; dt < NH; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) mma(St[dt], KTa[dt][kt], bU[kt]);
#pragma unroll
      for (int dt = NH; dt < NDT; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) mma(St[dt], KTb[dt - NH][kt], bU[kt]);
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        bS[ku] = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);
        bS_buf[tile][ku][lane] = bS[ku].v;
      }
    } else {
      // ---- output phase 1: Z = Q S with chunk n+2's transfers issued between
      // the products, then this wave's rows of P
      const auto nsrc = chunk_src(n + 2);
      const uint32_t fill_addr = lds_addr_of(fill);
      // Z is formed transposed (Z^T = S^T Q^T, operands swapped), so that lane
      // (li, g) holds Z[16 rt + li][16 tile + 4g .. 4g + 3].
      f32x4 Z[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Z[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        Frag<uint16_t> bSo, Qf[NRT];
        bSo.v = bS_buf[tile][ku][lane];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Qf[rt] = sw_frag<DK>(Qs, 16 * rt + li, ku, g);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mma(Z[rt], bSo, Qf[rt]);
        dma.issue_part(ku, NKU_D, fill_addr, nsrc);
      }
      __builtin_amdgcn_sched_barrier(0);
      // P rows of this output wave, one row tile at a time: with four row
      // tiles and two output waves the rows are {0,3} and {1,2} (five P^T
      // tiles each); a single output wave does all rows.
#pragma unroll
      for (int r = 0; r < NRT; ++r) {
        const bool mine = (NT == 1) || (r == tile) || (r == NRT - 1 - tile);
        if (!mine) continue;
        f32x4 Pr[NRT];
#pragma unroll
        for (int c = 0; c <= r; ++c) Pr[c] = zero4();
#pragma unroll
        for (int ku = 0; ku < NKU_D; ++ku) {
          const Frag<uint16_t> Qr = sw_frag<DK>(Qs, 16 * r + li, ku, g);
          Frag<uint16_t> Kc[NRT];
#pragma unroll
          for (int c = 0; c <= r; ++c) Kc[c] = sw_frag<DK>(Ks, 16 * c + li, ku, g);
#pragma unroll
          for (int c = 0; c <= r; ++c) mma(Pr[c], Kc[c], Qr);
        }
        // Pr[c][qq] = P[16r + li][16c + 4g + qq]; zero above the diagonal
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (4 * g + qq > li) Pr[r][qq] = 0.0f;
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * r + 15) {
            const f32x4 phi = (2 * ku + 1 <= r) ? Pr[(2 * ku + 1) % NRT] : zero4();
            P_buf[pf_index(r, ku)][lane] = acc_frag<uint16_t>(Pr[2 * ku], phi).v;
          }
        __builtin_amdgcn_sched_barrier(0);
      }

      wait_lgkm0();
      barrier_nowait();  // B: U' and P visible

      // ---- output phase 2: O^T = Z^T + U'^T P^T (operands swapped), which
      // leaves 4 consecutive columns of one output row per lane: one 8-byte
      // store per lane and row tile
      const int valid = chunk_valid(n);
      const int64_t row0 = row_of(n);
      Frag<uint16_t> bUo[NKU_C];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) bUo[ku].v = bU_buf[tile][ku][lane];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        f32x4 acc = Z[rt];
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15) {
            Frag<uint16_t> pf;
            pf.v = P_buf[pf_index(rt, ku)][lane];
            mma(acc, bUo[ku], pf);
          }
        const int t = 16 * rt + li;
        bf16x4 ov;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) ov[qq] = static_cast<__bf16>(acc[qq]);
        if (t < valid)
          *reinterpret_cast<bf16x4*>(o + (row0 + int64_t(t) * H) * DV + v0 + 16 * tile + 4 * g) = ov;
      }
    }
  };

  for (int n = 0; n < NC; n += 3) {
    chunk_step(slot0, slot2, n);
    if (n + 1 < NC) chunk_step(slot1, slot0, n + 1);
    if (n + 2 < NC) chunk_step(slot2, slot1, n + 2);
  }
  wait_vmcnt<0>();  // drain the DMA of the clamped chunks past the end

  if (chain && sfin != nullptr) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sfin[(int64_t(bh) * DK + 16 * dt + 4 * g + qq) * DV + col] = St[dt][qq];
  }
}

// Shapes: d_k in {32, 64, 128}, chunk in {32, 64}, value block 32 (two
// value tiles: one wavefront pair per tile).
inline bool v5_supported(int DK, int C, int BV) {
  return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64) && BV == 32;
}

template <int DK, int C, int BV>
hipError_t recurrence_v5_launch_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DV, hipStream_t stream) {
  using S = V5Shape<DK, C, BV>;
  const int NC = int((L + C - 1) / C);
  const int BH = B * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((recurrence_v5_kernel<DK, C, BV>), dim3(unsigned(nwg)), dim3(S::THREADS), 0, stream, q,
                     k, v, tws, s0, o, sfin, H, L, NC, DV, NVB, remap);
  return hipGetLastError();
}

template <int DK, int C>
hipError_t recurrence_v5_bv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* tws,
                            const float* s0, uint16_t* o, float* sfin, int B, int H, int64_t L, int DV,
                            int BV, hipStream_t s) {
  if (BV == 32) return recurrence_v5_launch_impl<DK, C, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
  return hipErrorInvalidValue;
}

inline hipError_t launch_recurrence_v5(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       hipStream_t s) {
  if (C == 32) {
    switch (DK) {
      case 32: return recurrence_v5_bv<32, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_v5_bv<64, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_v5_bv<128, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return recurrence_v5_bv<32, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_v5_bv<64, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_v5_bv<128, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
