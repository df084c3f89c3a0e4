// recurrence_tile.h -- the sequential chunk pass for bf16 inputs: one
// wavefront per 16-column tile of the state, chunk inputs streamed into LDS by
// DMA.  (The default bf16 kernel is recurrence_roles.h; this one also serves
// 64-column value blocks.)
//
// Algebra (per chunk of C tokens with start state S; T from the UT transform):
//     Y = K S,  Z = Q S,  P = tril(Q K^T)
//     U' = T (V - Y),   O = Z + P U',   S <- S + K^T U'
// Layout on gfx950:
//   * wave w owns value columns v0 + 16w .. +15 and all key dims of S
//     (d_k/16 fp32 accumulator tiles), so the chain S -> Y -> U' -> S stays in
//     one wavefront;
//   * the chunk inputs (Q, K, T, V block) go straight from global memory into
//     LDS with global_load_lds_dwordx4 (no register staging), into a ring of
//     three slots, issued two chunks ahead, in pieces between the first
//     products of the step that frees the slot.  Each wave waits
//     (s_waitcnt vmcnt) for its own transfers and one s_barrier per chunk
//     publishes the slot;
//   * LDS rows are unpadded (a DMA instruction fills 1 KiB contiguously) and
//     16-byte chunks are XOR-swizzled per row so that both the row-fragment
//     reads (16 rows x 8 B) and the transposing reads (4 rows x 32 B) of
//     ds_read_b64_tr_b16 are free of bank conflicts;
//   * K^T and the V tile come from ds_read_b64_tr_b16; P stays in registers;
//   * Q S and O are formed transposed (operands of the same fragments
//     swapped), which leaves 4 consecutive output columns per lane: one
//     8-byte store per lane and row tile, no staging.
#pragma once

#include "lds_ring.h"

namespace efla {

template <int DK, int C, int BV>
struct TileShape {
  static constexpr int NW = BV / 16, THREADS = NW * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;  // elements, a multiple of 512
  using Dma = ChunkDma<DK, C, BV, NW>;
  static constexpr int DMA_PER_WAVE = Dma::COUNT;
  static constexpr int STORES_PER_WAVE = NRT;  // one 8-byte O store per row tile
};

template <int DK, int C, int BV>
__global__ __launch_bounds__(4 * BV) void recurrence_tile_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ tws, const float* s0, uint16_t* __restrict__ o,
    float* sfin, int H, int64_t L, int NC, int DV, int NVB, int remap) {
  using S = TileShape<DK, C, BV>;
  constexpr int NRT = S::NRT, NDT = S::NDT, NKU_D = S::NKU_D, NKU_C = S::NKU_C, NW = S::NW;
  // Three separate arrays (not one indexed ring) so that alias analysis can
  // tell the slot being filled by DMA from the slot being read: the compiler
  // then leaves the in-flight transfers alone instead of waiting for them.
  __shared__ __align__(1024) uint16_t slot0[S::SLOT];
  __shared__ __align__(1024) uint16_t slot1[S::SLOT];
  __shared__ __align__(1024) uint16_t slot2[S::SLOT];

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

  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;
  auto chunk_valid = [&](int n) { return int(L - int64_t(n) * C < C ? L - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (b * L + int64_t(n) * C) * H + h; };
  // Issue the DMA of chunk n (clamped to the last chunk, so every wave always
  // issues the same number of transfers) into `slot`.
  typename S::Dma dma;
  dma.init(qk_stride, v_stride, lane, w);
  // Sources of chunk n, clamped to the last chunk so that every wave always
  // issues the same number of transfers.
  auto chunk_src = [&](int n) {
    const int nn = n < NC ? n : NC - 1;
    const int64_t r0 = row_of(nn);
    using U = const uint16_t*;
    return typename S::Dma::Src{(U)uniform_ptr(q + r0 * DK), (U)uniform_ptr(k + r0 * DK),
                                (U)uniform_ptr(tws + (int64_t(bh) * NC + nn) * C * C),
                                (U)uniform_ptr(v + r0 * DV + v0), chunk_valid(nn)};
  };

  f32x4 St[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      St[dt][qq] = s0 != nullptr ? s0[(int64_t(bh) * DK + 16 * dt + 4 * g + qq) * DV + col] : 0.0f;

  if (NC > 0) {
    // all earlier global loads (the initial state) are done before counting
    wait_vmcnt<0>();
    dma.issue_part(0, 1, lds_addr_of(slot0), chunk_src(0));
    dma.issue_part(0, 1, lds_addr_of(slot1), chunk_src(1));
  }

  constexpr int D = S::DMA_PER_WAVE, ST = S::STORES_PER_WAVE;
  // One chunk: `cur` holds chunk n; chunk n + 2 is sent to `fill`.
  auto chunk_step = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ fill, int n) {
    // This wave's transfers for chunk n (issued during step n-2) are done once
    // at most the operations issued after them are outstanding: the output
    // stores of steps n-2 and n-1 and the transfers of chunk n+1.
    if (n == 0) wait_vmcnt<D>();
    else if (n == 1) wait_vmcnt<D + ST>();
    else wait_vmcnt<D + 2 * ST>();
    barrier_nowait();  // chunk n visible to all waves; `fill` no longer read
    const auto nsrc = chunk_src(n + 2);
    const uint32_t fill_addr = lds_addr_of(fill);

    const uint16_t* Qs = cur + S::QOFF;
    const uint16_t* Ks = cur + S::KOFF;
    const uint16_t* Ts = cur + S::TOFF;
    const uint16_t* Vs = cur + S::VOFF;
    const int valid = chunk_valid(n);
    const int64_t row0 = row_of(n);

    // Operands that only depend on this chunk's LDS data are fetched first, so
    // their latency hides behind the first products: the V tile (for D) and
    // T (for U').
    bf16x4 Vt[NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int j = lane & 15;
      Vt[rt] = lds_read_tr(Vs + swz_off<BV>(16 * rt + 4 * g + (j >> 2), 16 * w + 4 * (j & 3)));
    }
    Frag<uint16_t> Tf[NRT][NKU_C];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku <= 16 * rt + 15) Tf[rt][ku] = sw_frag<C>(Ts, 16 * rt + li, ku, g);

    // Y = K S, Z = Q S and the P^T tiles, k-unit by k-unit: the eight K and Q
    // fragments of one k-unit feed 2*NRT + NRT(NRT+1)/2 independent products.
    // Pt[r][c][qq] = P[16r + li][16c + 4g + qq] (c <= r; masked on the diagonal)
    // Z is formed transposed (Z^T = S^T Q^T: the same two fragments with the
    // operands swapped) so that each lane ends up holding 4 consecutive
    // columns of one output row: Zt[rt][qq] = Z[16 rt + li][16 w + 4 g + qq].
    f32x4 Y[NRT], Zt[NRT], Pt[NRT][NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      Y[rt] = zero4();
      Zt[rt] = zero4();
#pragma unroll
      for (int c = 0; c < NRT; ++c) Pt[rt][c] = zero4();
    }
#pragma unroll
    for (int ku = 0; ku < NKU_D; ++ku) {
      const Frag<uint16_t> bS = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);
      Frag<uint16_t> Kf[NRT], Qf[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        Kf[rt] = sw_frag<DK>(Ks, 16 * rt + li, ku, g);
        Qf[rt] = sw_frag<DK>(Qs, 16 * rt + li, ku, g);
      }
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        mma(Y[rt], Kf[rt], bS);
        mma(Zt[rt], bS, Qf[rt]);
#pragma unroll
        for (int c = 0; c <= rt; ++c) mma(Pt[rt][c], Kf[c], Qf[rt]);
      }
      // a share of chunk n+2's transfers, issued between the products
      dma.issue_part(ku, NKU_D, fill_addr, nsrc);
    }
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        if (4 * g + qq > li) Pt[rt][rt][qq] = 0.0f;

    // K^T fragments for the state update (transposing reads), fetched while
    // U' is formed.
    Frag<uint16_t> KTf[NDT][NKU_C];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kt = 0; kt < NKU_C; ++kt) KTf[dt][kt] = sw_frag_tr<DK>(Ks, 16 * dt, kt, lane);

    // D = V - Y, then U' = T D
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
    for (int ku = 0; ku < NKU_C; ++ku) bU[ku] = acc_frag<uint16_t>(U[2 * ku], U[2 * ku + 1]);

    // S += K^T U'
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int kt = 0; kt < NKU_C; ++kt) mma(St[dt], KTf[dt][kt], bU[kt]);

    // O^T = Z^T + U'^T P^T, again by swapping the operands of the same
    // fragments: lane (li, g) holds O[16 rt + li][16 w + 4g .. 4g + 3] and
    // stores it as one 8-byte write.
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 acc = Zt[rt];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku <= 16 * rt + 15) {
          const f32x4 phi = (2 * ku + 1 <= rt) ? Pt[rt][(2 * ku + 1) % NRT] : zero4();
          mma(acc, bU[ku], acc_frag<uint16_t>(Pt[rt][2 * ku], phi));
        }
      const int t = 16 * rt + li;
      bf16x4 ov;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ov[qq] = static_cast<__bf16>(acc[qq]);
      if (t < valid)
        *reinterpret_cast<bf16x4*>(o + (row0 + int64_t(t) * H) * DV + v0 + 16 * w + 4 * g) = ov;
    }
  };

  // the ring rotates through the three slots with a period of three chunks
  for (int n = 0; n < NC; n += 3) {
    chunk_step(slot0, slot2, n);
    if (n + 1 < NC) chunk_step(slot1, slot0, n + 1);
    if (n + 2 < NC) chunk_step(slot2, slot1, n + 2);
  }
  wait_vmcnt<0>();  // drain the DMA of the clamped chunks past the end

  if (sfin != nullptr) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) sfin[(int64_t(bh) * DK + 16 * dt + 4 * g + qq) * DV + col] = St[dt][qq];
  }
}

inline bool tile_supported(int DK, int C, int BV) {
  return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64) && (BV == 16 || BV == 32 || BV == 64);
}

template <int DK, int C, int BV>
hipError_t recurrence_tile_launch_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DV, hipStream_t stream) {
  using S = TileShape<DK, C, BV>;
  const int NC = int((L + C - 1) / C);
  const int BH = B * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((recurrence_tile_kernel<DK, C, BV>), dim3(unsigned(nwg)), dim3(S::THREADS), 0, stream, q,
                     k, v, tws, s0, o, sfin, H, L, NC, DV, NVB, remap);
  return hipGetLastError();
}

template <int DK, int C>
hipError_t recurrence_tile_bv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* tws,
                            const float* s0, uint16_t* o, float* sfin, int B, int H, int64_t L, int DV,
                            int BV, hipStream_t s) {
  switch (BV) {
    case 16: return recurrence_tile_launch_impl<DK, C, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
    case 32: return recurrence_tile_launch_impl<DK, C, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
    case 64: return recurrence_tile_launch_impl<DK, C, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
  }
  return hipErrorInvalidValue;
}

inline hipError_t launch_recurrence_tile(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       hipStream_t s) {
  if (C == 32) {
    switch (DK) {
      case 32: return recurrence_tile_bv<32, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_tile_bv<64, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_tile_bv<128, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return recurrence_tile_bv<32, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_tile_bv<64, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_tile_bv<128, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
