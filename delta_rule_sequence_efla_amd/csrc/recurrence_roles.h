// recurrence_roles.h -- the sequential chunk pass for bf16 inputs with one role
// per wavefront and one chain wavefront per 16-column state tile.
//
// Per chunk (start state S, T from the UT transform):
//     U' = T (V - K S),   S <- S + K^T U',   O = Q S + tril(Q K^T) U'
// A workgroup owns BV value columns of one (b, h); its wavefronts:
//   * chain c (one per 16-column tile): keeps its tile of S in fp32 registers
//     and forms Y = K S, U' = T (V - Y) and S += K^T U' (38 matrix-core ops
//     per chunk), publishing U' and the new S as bf16 operand fragments;
//   * output: Z^T = S^T Q^T and O^T = Z^T + U'^T P^T for all BV columns
//     (operands of the same fragments swapped, so each lane stores 4
//     consecutive columns);
//   * P: P = tril(Q K^T), published through LDS; half of the key dimension
//     is summed one step early, after barrier B of the step before, where
//     this wave would otherwise wait (the DMA wave completes chunk n+1 by
//     then);
//   * DMA: streams Q, K, T and V into a three-slot LDS ring two chunks ahead
//     with global_load_lds_dwordx4.  Moving data into LDS runs at well under
//     64 B/clock per CU and an issuing wavefront stalls while the queue is
//     full, so the transfers get a wavefront of their own.
// Q and K row fragments are 16-byte reads under the key-dimension
// relabeling of lds_ring.h.  Wavefronts: P, chain 0 .. BV/16-1, output, DMA
// (five for BV = 32; the DMA wave, which mostly waits, shares a SIMD with the
// P wave).
// Two barriers per chunk:
//   A (chunk n in LDS, S_n fragments published)
//     chains: Y, U' -> publish U'   | output: Z^T        | P: finish P_n -> publish | DMA: half of chunk n+2
//   B (U' and P published, chunk n+1 in LDS)
//     chains: S update -> publish S | output: O^T, store | P: start P_{n+1}        | DMA: other half
#pragma once

#include "lds_ring.h"

namespace efla {

template <int DK, int C, int BV>
struct RolesShape {
  static constexpr int NT = BV / 16;  // state tiles of the workgroup = chain wavefronts
  static constexpr int NWAVES = NT + 3, THREADS = NWAVES * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;
  static constexpr int NPF = (NRT == 4) ? 6 : 2;  // P fragments (rt, ku) with 32 ku <= 16 rt + 15
  using Dma = ChunkDma<DK, C, BV, 1, true>;       // every transfer from the DMA wave
  static constexpr int DMA_COUNT = Dma::COUNT;
  // wave 0 is the P wave, waves 1..NT the chains, then output and DMA
  static constexpr int kP = 0, kChain0 = 1, kOut = NT + 1, kDma = NT + 2;
};

// Instances (MODE):
//   kFwd     the forward pass: output and final state.
//   kStates  for the backward pass: writes the state at the start of every
//            chunk (the bf16 operand fragments the chains publish, i.e. the
//            values the forward's products use) to `states`, and no output;
//            the output wavefront copies the fragments.
//   kFinal   the final state only (no output).
//   kTrans   the chunk transition: V = 0 and the identity as the initial
//            state, final state only, so that it ends as the product of the
//            chunks' (I - K^T T K) over the value columns' rows of I.
// Without output the P wavefront (and in kFinal / kTrans the output
// wavefront) only keeps the barriers.
enum RolesMode { kFwd = 0, kStates = 1, kFinal = 2, kTrans = 3 };
template <int DK, int C, int BV, int MODE>
__global__ __launch_bounds__(64 * (BV / 16 + 3)) void recurrence_roles_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ tws, const float* s0, uint16_t* __restrict__ o,
    float* sfin, int H, int64_t L, int NC, int DV, int NVB, int remap,
    const int32_t* __restrict__ cu, uint16_t* __restrict__ states, const int32_t* __restrict__ order, int nseq) {
  using S = RolesShape<DK, C, BV>;
  constexpr bool ST = MODE == kStates, NOOUT = MODE != kFwd, VZERO = MODE == kTrans;
  constexpr int NT = S::NT, NRT = S::NRT, NDT = S::NDT, NKU_D = S::NKU_D, NKU_C = S::NKU_C;
  constexpr int NPF = S::NPF;
  __shared__ __align__(1024) uint16_t slot0[S::SLOT];
  __shared__ __align__(1024) uint16_t slot1[S::SLOT];
  __shared__ __align__(1024) uint16_t slot2[S::SLOT];
  __shared__ __align__(16) bf16x8 bS_buf[NT][NKU_D][kWave];  // S_n as operand fragments
  __shared__ __align__(16) bf16x8 bU_buf[NT][NKU_C][kWave];  // U'_n as operand fragments
  __shared__ __align__(16) bf16x8 P_buf[NPF][kWave];         // P_n as operand fragments

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
  if (order != nullptr) bh = seq_of_rank(order, bh / H, nseq) * H + bh % H;  // packed: longest first
  const int64_t h = bh % H;
  const SeqSpan sp = seq_span<C>(cu, bh / H, h, H, L, NC);  // sequence bh / H
  const int nc = sp.nc;
  const int v0 = vb * BV;
  const int lane = threadIdx.x & 63, role = wave_id(), li = lane & 15, g = lane >> 4;
  auto chunk_valid = [&](int n) { return int(sp.len - int64_t(n) * C < C ? sp.len - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (sp.bos + int64_t(n) * C) * H + h; };
  auto sync = [&]() {  // this wave's LDS writes done, then the workgroup barrier
    wait_lgkm0();
    barrier_nowait();
  };
  // The DMA wave writes LDS only through global_load_lds, whose completion it
  // tracks with vmcnt; an lgkmcnt drain there would wait for transfers still
  // in flight (they count against it too), so it passes the barriers directly.
  auto sync_dma = [&]() { barrier_nowait(); };

  if (role == S::kDma) {
    // ---------------------------------------------------------------- DMA
    typename S::Dma dma;
    dma.init(int64_t(H) * DK, int64_t(H) * DV, lane, 0);
    auto chunk_src = [&](int n) {
      const int64_t r0 = row_of(n);
      using U = const uint16_t*;
      return typename S::Dma::Src{(U)uniform_ptr(q + r0 * DK), (U)uniform_ptr(k + r0 * DK),
                                  (U)uniform_ptr(tws + (sp.slot0 + n) * C * C),
                                  (U)uniform_ptr(v + r0 * DV + v0), chunk_valid(n)};
    };
    constexpr int D = S::DMA_COUNT, D0 = S::DMA_COUNT / 2;  // D0: transfers of part 0
    if (nc > 0) dma.issue_part(0, 1, lds_addr_of(slot0), chunk_src(0));
    if (nc > 1) dma.issue_part(0, 1, lds_addr_of(slot1), chunk_src(1));
    auto step = [&](uint16_t* fill, int n) {
      // chunk n is complete once at most chunk n+1's transfers are outstanding
      // (already true since barrier B of the step before)
      if (n + 1 < nc) wait_vmcnt<D>();
      else wait_vmcnt<0>();
      sync_dma();  // A
      const bool more = n + 2 < nc;
      const auto src = chunk_src(more ? n + 2 : n);
      const uint32_t fa = lds_addr_of(fill);
      if (more) dma.issue_part(0, 2, fa, src);
      // chunk n+1 complete before barrier B: the P wave starts on it there
      if (more) wait_vmcnt<D0>();
      else wait_vmcnt<0>();
      sync_dma();  // B
      if (more) dma.issue_part(1, 2, fa, src);
    };
    for (int n = 0; n < nc; n += 3) {
      step(slot2, n);
      if (n + 1 < nc) step(slot0, n + 1);
      if (n + 2 < nc) step(slot1, n + 2);
    }
    wait_vmcnt<0>();
  } else if (role >= S::kChain0 && role < S::kChain0 + NT) {
    // -------------------------------------------------------------- chain
    const int ct = role - S::kChain0;  // this wave's state tile
    const int col = v0 + 16 * ct + li;
    // St[dt][qq] = S[key_phys(16 dt + 4 g + qq)][col]
    f32x4 St[NDT];
    Frag<uint16_t> bS[NKU_D];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        St[dt][qq] = VZERO ? (key_phys(16 * dt + 4 * g + qq) == col ? 1.0f : 0.0f)
                   : s0 != nullptr ? s0[(int64_t(bh) * DK + key_phys(16 * dt + 4 * g + qq)) * DV + col] : 0.0f;
#pragma unroll
    for (int ku = 0; ku < NKU_D; ++ku) {
      bS[ku] = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);
      bS_buf[ct][ku][lane] = bS[ku].v;
    }
    auto step = [&](const uint16_t* __restrict__ cur) {
      const uint16_t* Ks = cur + S::KOFF;
      const uint16_t* Ts = cur + S::TOFF;
      const uint16_t* Vs = cur + S::VOFF;
      sync();  // A
      // operands that only depend on the chunk: this tile's V columns and T
      bf16x4 Vt[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) {
        const int j = lane & 15;
        Vt[rt] = lds_read_tr(Vs + swz_off<BV>(16 * rt + 4 * g + (j >> 2), 16 * ct + 4 * (j & 3)));
      }
      Frag<uint16_t> Tf[NRT][NKU_C];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15) Tf[rt][ku] = sw_frag<C>(Ts, 16 * rt + li, ku, g);
      // Y = K S
      f32x4 Y[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Y[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        Frag<uint16_t> Kf[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Kf[rt] = wide_frag<DK>(Ks, 16 * rt + li, ku, g);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mma(Y[rt], Kf[rt], bS[ku]);
      }
      // D = V - Y, U' = T D, published for the output wave
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) Y[rt][qq] = (VZERO ? 0.0f : static_cast<float>(Vt[rt][qq])) - Y[rt][qq];
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
        bU_buf[ct][ku][lane] = bU[ku].v;
      }
      sync();  // B
      // S += K^T U' (the K^T fragments are read after the barrier, where the
      // LDS is less busy), then publish S_{n+1}
      Frag<uint16_t> KT[NDT][NKU_C];
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) KT[dt][kt] = wide_frag_tr<DK>(Ks, dt, kt, lane);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) mma(St[dt], KT[dt][kt], bU[kt]);
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        bS[ku] = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);
        bS_buf[ct][ku][lane] = bS[ku].v;
      }
    };
    for (int n = 0; n < nc; n += 3) {
      step(slot0);
      if (n + 1 < nc) step(slot1);
      if (n + 2 < nc) step(slot2);
    }
    if (sfin != nullptr) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          sfin[(int64_t(bh) * DK + key_phys(16 * dt + 4 * g + qq)) * DV + col] = St[dt][qq];
    }
  } else if (ST && role == S::kOut) {
    // S_n fragments of tile ct, k-unit ku: element e of lane (li, g) is state
    // row key_phys(32 ku + 16 (e / 4) + 4 g + e % 4) = 32 ku + 8 g + e, column
    // v0 + 16 ct + li.  So columns 8 j .. 8 j + 7 of row r are element r % 8
    // of eight neighbouring lanes' fragments: the wave gathers them with 2-byte
    // LDS reads and writes each (row, 8 columns) unit with one 16-byte store
    // (eight stores per lane per chunk instead of 64 2-byte ones).
    const uint16_t* frag = reinterpret_cast<const uint16_t*>(&bS_buf[0][0][0]);
    for (int n = 0; n < nc; ++n) {
      sync();  // A: S_n published
      uint16_t* dst = states + (sp.slot0 + n) * DK * DV + v0;
#pragma unroll 1
      for (int u = lane; u < DK * (BV / 8); u += kWave) {
        const int r = u / (BV / 8), cg = u % (BV / 8);
        const int ct = cg / 2, l0 = 8 * (cg % 2), ku = r / 32, gr = (r % 32) / 8, e = r % 8;
        const uint16_t* src = frag + ((ct * NKU_D + ku) * kWave + 16 * gr + l0) * 8 + e;
        union {
          u32x4 u;
          uint16_t e16[8];
        } f;
#pragma unroll
        for (int c = 0; c < 8; ++c) f.e16[c] = src[8 * c];
        *reinterpret_cast<u32x4*>(dst + r * DV + 8 * cg) = f.u;
      }
      sync();  // B
    }
  } else if (!NOOUT && role == S::kOut) {
    // ------------------------------------------------------------- output
    auto step = [&](const uint16_t* __restrict__ cur, int n) {
      const uint16_t* Qs = cur + S::QOFF;
      sync();  // A
      // Zt[ct][rt][qq] = Z[16 rt + li][16 ct + 4 g + qq]  (Z^T = S^T Q^T)
      f32x4 Zt[NT][NRT];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Zt[ct][rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        Frag<uint16_t> bSo[NT], Qf[NRT];
#pragma unroll
        for (int ct = 0; ct < NT; ++ct) bSo[ct].v = bS_buf[ct][ku][lane];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Qf[rt] = wide_frag<DK>(Qs, 16 * rt + li, ku, g);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int ct = 0; ct < NT; ++ct) mma(Zt[ct][rt], bSo[ct], Qf[rt]);
      }
      sync();  // B
      // O^T = Z^T + U'^T P^T; lane (li, g) stores O[16 rt + li][16 ct + 4g .. 4g + 3]
      const int valid = chunk_valid(n);
      const int64_t row0 = row_of(n);
      Frag<uint16_t> pf[NPF];
#pragma unroll
      for (int i = 0; i < NPF; ++i) pf[i].v = P_buf[i][lane];
#pragma unroll
      for (int ct = 0; ct < NT; ++ct) {
        Frag<uint16_t> bUo[NKU_C];
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku) bUo[ku].v = bU_buf[ct][ku][lane];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          f32x4 acc = Zt[ct][rt];
#pragma unroll
          for (int ku = 0; ku < NKU_C; ++ku)
            if (32 * ku <= 16 * rt + 15) mma(acc, bUo[ku], pf[pf_index(rt, ku)]);
          const int t = 16 * rt + li;
          bf16x4 ov;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) ov[qq] = static_cast<__bf16>(acc[qq]);
          if (t < valid)
            *reinterpret_cast<bf16x4*>(o + (row0 + int64_t(t) * H) * DV + v0 + 16 * ct + 4 * g) = ov;
        }
      }
    };
    for (int n = 0; n < nc; n += 3) {
      step(slot0, n);
      if (n + 1 < nc) step(slot1, n + 1);
      if (n + 2 < nc) step(slot2, n + 2);
    }
  } else if (NOOUT && (role == S::kP || role == S::kOut)) {
    for (int n = 0; n < nc; ++n) {
      sync();
      sync();
    }
  } else if (!NOOUT && role == S::kP) {
    // ------------------------------------------------------------------ P
    // P_n = tril(Q K^T) of chunk n, split over the key dimension: k-units
    // 0 .. KH-1 after barrier B of step n-1 (chunk n is complete there, and
    // this wave would otherwise idle), the rest after barrier A of step n.
    constexpr int KH = NKU_D / 2;
    // Pt[r][c][qq] = P[16 r + li][16 c + 4 g + qq] for c <= r
    f32x4 Pt[NRT][NRT];
    auto accumulate = [&](const uint16_t* __restrict__ cur, int ku0, int ku1) {
      const uint16_t* Qs = cur + S::QOFF;
      const uint16_t* Ks = cur + S::KOFF;
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        if (ku < ku0 || ku >= ku1) continue;
        Frag<uint16_t> Qf[NRT], Kf[NRT];
#pragma unroll
        for (int r = 0; r < NRT; ++r) {
          Qf[r] = wide_frag<DK>(Qs, 16 * r + li, ku, g);
          Kf[r] = wide_frag<DK>(Ks, 16 * r + li, ku, g);
        }
#pragma unroll
        for (int r = 0; r < NRT; ++r)
#pragma unroll
          for (int c = 0; c <= r; ++c) mma(Pt[r][c], Kf[c], Qf[r]);
      }
    };
    auto clear = [&]() {
#pragma unroll
      for (int r = 0; r < NRT; ++r)
#pragma unroll
        for (int c = 0; c < NRT; ++c) Pt[r][c] = zero4();
    };
    clear();
    auto step = [&](const uint16_t* __restrict__ cur, const uint16_t* __restrict__ nxt, int n) {
      sync();  // A
      if (n == 0) accumulate(cur, 0, KH);
      accumulate(cur, KH, NKU_D);
#pragma unroll
      for (int r = 0; r < NRT; ++r) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          if (4 * g + qq > li) Pt[r][r][qq] = 0.0f;
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * r + 15) {
            const f32x4 phi = (2 * ku + 1 <= r) ? Pt[r][(2 * ku + 1) % NRT] : zero4();
            P_buf[pf_index(r, ku)][lane] = acc_frag<uint16_t>(Pt[r][2 * ku], phi).v;
          }
      }
      sync();  // B
      clear();
      if (n + 1 < nc) accumulate(nxt, 0, KH);
    };
    for (int n = 0; n < nc; n += 3) {
      step(slot0, slot1, n);
      if (n + 1 < nc) step(slot1, slot2, n + 1);
      if (n + 2 < nc) step(slot2, slot0, n + 2);
    }
  }
}

// Shapes: d_k in {32, 64, 128}, chunk in {32, 64}, value block 16 or 32.
inline bool roles_supported(int DK, int C, int BV) {
  return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64) && (BV == 16 || BV == 32);
}

template <int DK, int C, int BV>
hipError_t recurrence_roles_launch_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DV, const int32_t* cu, int N,
                                     uint16_t* states, bool trans, const int32_t* order, hipStream_t stream) {
  const int NC = cu == nullptr ? int((L + C - 1) / C) : int(L / C) + N;  // chunk slots per sequence / head
  const int BH = (cu == nullptr ? B : N) * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  if (cu == nullptr) order = nullptr;  // dense batches keep their order
  const int remap = (BH % 8 == 0) ? 1 : 0;
  const int mode = states != nullptr ? kStates : trans ? kTrans : o == nullptr ? kFinal : kFwd;
  const dim3 grid{unsigned(nwg)}, block{unsigned(RolesShape<DK, C, BV>::THREADS)};
  switch (mode) {
    case kFwd:
      hipLaunchKernelGGL((recurrence_roles_kernel<DK, C, BV, kFwd>), grid, block, 0, stream, q, k, v, tws, s0, o,
                         sfin, H, L, NC, DV, NVB, remap, cu, states, order, N);
      break;
    case kStates:
      hipLaunchKernelGGL((recurrence_roles_kernel<DK, C, BV, kStates>), grid, block, 0, stream, q, k, v, tws, s0, o,
                         sfin, H, L, NC, DV, NVB, remap, cu, states, order, N);
      break;
    case kFinal:
      hipLaunchKernelGGL((recurrence_roles_kernel<DK, C, BV, kFinal>), grid, block, 0, stream, q, k, v, tws, s0, o,
                         sfin, H, L, NC, DV, NVB, remap, cu, states, order, N);
      break;
    default:
      hipLaunchKernelGGL((recurrence_roles_kernel<DK, C, BV, kTrans>), grid, block, 0, stream, q, k, v, tws, s0, o,
                         sfin, H, L, NC, DV, NVB, remap, cu, states, order, N);
  }
  return hipGetLastError();
}

template <int DK, int C>
hipError_t recurrence_roles_bv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* tws,
                            const float* s0, uint16_t* o, float* sfin, int B, int H, int64_t L, int DV,
                            int BV, const int32_t* cu, int N, uint16_t* states, bool trans, const int32_t* order,
                            hipStream_t s) {
  switch (BV) {
    case 16: return recurrence_roles_launch_impl<DK, C, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, states, trans, order, s);
    case 32: return recurrence_roles_launch_impl<DK, C, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, states, trans, order, s);
  }
  return hipErrorInvalidValue;
}

inline hipError_t launch_recurrence_roles(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       const int32_t* cu, int N, uint16_t* states, bool trans, const int32_t* order,
                                       hipStream_t s) {
  if (C == 32) {
    switch (DK) {
      case 32: return recurrence_roles_bv<32, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, states, trans, order, s);
      case 64: return recurrence_roles_bv<64, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, states, trans, order, s);
      case 128: return recurrence_roles_bv<128, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, states, trans, order, s);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return recurrence_roles_bv<32, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, states, trans, order, s);
      case 64: return recurrence_roles_bv<64, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, states, trans, order, s);
      case 128: return recurrence_roles_bv<128, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, cu, N, states, trans, order, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
