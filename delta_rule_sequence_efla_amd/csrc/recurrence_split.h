// recurrence_split.h -- the sequential chunk pass for bf16 inputs with each
// chunk's work spread over nine wavefronts.
//
// Per chunk (start state S, T from the UT transform):
//     U' = T (V - K S),   S <- S + K^T U',   O = Q S + tril(Q K^T) U'
// A workgroup owns BV = 32 value columns (two 16-column state tiles) of one
// (b, h).  A wavefront's time per chunk is close to the sum of its own LDS
// reads (tens of cycles each, whatever their width) and matrix-core
// products, so the work of the one-role-per-wavefront kernel
// (recurrence_roles.h) is cut finer here:
//   * Y wave per tile: Y = K S_tile, D = V - Y, U' = T D, publishes U'.  The
//     chunk's K, T and V fragments are read in the other phase, right after
//     the chunk lands, so only the products sit between S and U'.
//   * S wave per half of the key dimension: keeps those 64 rows of S (both
//     tiles) in fp32 registers, reads its K^T fragments while the Y waves
//     work, then forms S += K^T U' and publishes its rows of S as bf16
//     operand fragments.  Splitting the key dimension (not the columns)
//     halves each S wave's K^T reads.
//   * output wave per half of the chunk's rows, both tiles: Z^T = S^T Q^T,
//     then O^T = Z^T + U'^T P^T for its 32 rows; the next chunk's Q
//     fragments (of those rows only) are read once its output is staged.
//     Split by rows, each reads half of Q (split by tiles, each read all).
//   * two P waves: P = tril(Q K^T), row tiles 0-2 and row tile 3; half of the
//     key dimension is summed in the phase before.
//   * DMA wave: streams Q, K, T and V into a three-slot LDS ring two chunks
//     ahead (as in recurrence_roles.h).
// Wavefront w runs on SIMD w % 4; each SIMD holds one Y or S wave, and the
// lighter roles fill in.
// Two barriers per chunk:
//   A (chunk n in LDS, S_n published)
//     Y: products -> publish U'_n | S: read K^T_n | O: Z^T | P: finish P_n -> publish | DMA: half of chunk n+2
//   B (U'_n and P_n published, chunk n+1 in LDS)
//     Y: read K, T, V of chunk n+1 | S: S += K^T U' -> publish S_{n+1} | O: O^T -> stage, read Q_{n+1}
//     | P: start P_{n+1} | DMA: other half
// The output of chunk n is staged in LDS and stored after barrier A of step
// n+1 (after one last barrier for the final chunk).
// Every exchange buffer is written in one phase and read in the other, so
// one copy of each suffices.
#pragma once

#include <type_traits>

#include "lds_ring.h"

namespace efla {

template <int DK, int C, int BV, int NDMA = 1>
struct SplitShape {
  static_assert(C == 64 && BV == 32 && (DK == 64 || DK == 128), "shapes of the split recurrence");
  static constexpr int NT = BV / 16;  // state tiles of the workgroup
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int KH = NKU_D / 2;  // key k-units per S wave (and per P half)
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;
  static constexpr int NPF = 6;  // P fragments (rt, ku) with 32 ku <= 16 rt + 15
  static constexpr int OP = BV + 8;  // pitch of the output staging rows (80 bytes: 8-byte writes conflict-free)
  using Dma = ChunkDma<DK, C, BV, 1, true>;
  static constexpr int DMA_COUNT = Dma::COUNT;
  // roles by wavefront index (SIMD = index % 4):
  //   SIMD 0: P rows 0-47 (0), S rows 64-127 (4), DMA (8)
  //   SIMD 1: Y tile 0 (1), output rows 0-31 (5)
  //   SIMD 2: Y tile 1 (2), output rows 32-63 (6)
  //   SIMD 3: S rows 0-63 (3), P rows 48-63 (7)[, second DMA wave (9)]
  // With NDMA = 2 two DMA waves share each chunk's transfers, one streaming
  // Q and T, the other K and V.
  static constexpr int kP0 = 0, kY0 = 1, kY1 = 2, kS0 = 3, kS1 = 4, kO0 = 5, kO1 = 6, kP1 = 7, kDma = 8, kDma2 = 9;
  __host__ __device__ static constexpr bool is_output(int w) { return w == kO0 || w == kO1; }
  static constexpr int NWAVES = 8 + NDMA, THREADS = NWAVES * kWave;
};

inline bool split_supported(int DK, int C, int BV) { return C == 64 && BV == 32 && (DK == 64 || DK == 128); }

// SAVE: the S wavefronts also store the state at the start of every chunk, as
// the bf16 operand values the products use, transposed ([slots][DV][DK], the
// layout of the backward's state-only pass), so that a training step's
// backward pass need not recompute them.
template <int DK, int C, int BV, int NDMA, bool SAVE = false>
__global__ __launch_bounds__(64 * (8 + NDMA)) void recurrence_split_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ tws, const float* s0, uint16_t* __restrict__ o, float* sfin, int H, int64_t L,
    int NC, int DV, int NVB, int remap, const int32_t* __restrict__ cu, const int32_t* __restrict__ order,
    int nseq, uint16_t* __restrict__ statesT = nullptr) {
  using S = SplitShape<DK, C, BV, NDMA>;
  constexpr int NT = S::NT, NRT = S::NRT, NKU_D = S::NKU_D, NKU_C = S::NKU_C, KH = S::KH, NPF = S::NPF;
  __shared__ __align__(1024) uint16_t ring[3 * S::SLOT];  // three chunk slots of 44 KiB
  uint16_t* const slot0 = ring;
  uint16_t* const slot1 = ring + S::SLOT;
  uint16_t* const slot2 = ring + 2 * S::SLOT;
  __shared__ __align__(16) bf16x8 bS_buf[NT][NKU_D][kWave];  // S_n as operand fragments
  __shared__ __align__(16) bf16x8 bU_buf[NT][NKU_C][kWave];  // U'_n as operand fragments
  __shared__ __align__(16) bf16x8 P_buf[NPF][kWave];         // P_n as operand fragments
  __shared__ __align__(16) uint16_t O_st[C][S::OP];          // O_n, staged for 64-byte row stores

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
  const SeqSpan sp = seq_span<C>(cu, bh / H, h, H, L, NC);
  const int nc = sp.nc;
  const int v0 = vb * BV;
  const int lane = threadIdx.x & 63, role = wave_id(), li = lane & 15, g = lane >> 4;
  auto chunk_valid = [&](int n) { return int(sp.len - int64_t(n) * C < C ? sp.len - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (sp.bos + int64_t(n) * C) * H + h; };
  auto sync = [&]() {  // this wave's LDS accesses done, then the workgroup barrier
    wait_lgkm0();
    barrier_nowait();
  };
  // Output of chunk n from the staging tile: output wave `half` stores rows
  // 32 half .. 32 half + 31, one 16-byte piece per lane, so every row's 64
  // bytes leave in one instruction, as nontemporal stores.  (Eight
  // 32-byte pieces of each 256-byte row of o, from eight wavefronts, slowed
  // the whole pass and most of all the heads whose rows sit at 256 mod 1024
  // bytes; with ordinary stores of whole 64-byte pieces those heads still
  // trailed the others by ~15 %, with nontemporal ones they do not.)
  auto store_staged = [&](int n, int half) {
    const int valid = chunk_valid(n);
    const int64_t row0 = row_of(n);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 32 * half + 16 * i + (lane >> 2), piece = lane & 3;
      const u32x4 val = *reinterpret_cast<const u32x4*>(&O_st[r][8 * piece]);
      if (r < valid)
        __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(o + (row0 + int64_t(r) * H) * DV + v0 + 8 * piece));
    }
  };
  const int o_rh = role == S::kO1 ? 1 : 0;  // output waves: row half
  // Steps of three chunks keep the ring slots compile-time addresses.
  auto run = [&](auto&& step) {
    for (int n = 0; n < nc; n += 3) {
      step(slot0, slot1, n);
      if (n + 1 < nc) step(slot1, slot2, n + 1);
      if (n + 2 < nc) step(slot2, slot0, n + 2);
    }
  };

  auto dma_role = [&](auto setc) {
    // ---------------------------------------------------------------- DMA
    // Every reader of chunk n is done with its slot by barrier B of step n
    // (the next chunk's fragments are read after that barrier, K^T and the
    // second half of P before it), so chunk n+3 goes into that slot right
    // away: half after barrier B of step n, half after barrier A of step n+1,
    // and it is first needed after barrier B of step n+2 -- one and a half to
    // two chunk periods to land.  At most 63 transfers can be outstanding per
    // wave, so the waits are expressed against one chunk's (chunk n+1 is
    // complete once only chunk n+2's transfers remain).  SET < 0: this wave
    // issues every transfer; else transfer set SET of two.  The DMA waves
    // write LDS only through global_load_lds, whose completion they track
    // with vmcnt; they pass the barriers without an lgkmcnt drain.
    constexpr int SET = decltype(setc)::value;
    constexpr int D = SET < 0 ? S::DMA_COUNT : SET == 0 ? S::Dma::SET0 : S::Dma::SET1;
    static_assert(D < 64, "one chunk's transfers fit the vmcnt counter");
    typename S::Dma dma;
    dma.init(int64_t(H) * DK, int64_t(H) * DV, lane, 0);
    auto issue = [&](int m, int part, int parts) {
      const int64_t r0 = row_of(m);
      using U = const uint16_t*;
      const typename S::Dma::Src src{(U)uniform_ptr(q + r0 * DK), (U)uniform_ptr(k + r0 * DK),
                                     (U)uniform_ptr(tws + (sp.slot0 + m) * C * C),
                                     (U)uniform_ptr(v + r0 * DV + v0), chunk_valid(m)};
      const uint32_t addr = lds_addr_of(ring + (m % 3) * S::SLOT);
      if constexpr (SET < 0) dma.issue_part(part, parts, addr, src);
      else dma.template issue_set<SET>(part, parts, addr, src);
    };
    if (nc > 0) issue(0, 0, 1);
    if (nc > 1) {
      issue(1, 0, 1);
      wait_vmcnt<D>();  // chunk 0 complete
    } else {
      wait_vmcnt<0>();
    }
    if (nc > 2) issue(2, 0, 2);
    for (int n = 0; n < nc; ++n) {
      barrier_nowait();  // A
      if (n + 2 < nc) issue(n + 2, 1, 2);
      if (n + 2 < nc) wait_vmcnt<D>();  // chunk n+1 complete: only chunk n+2's transfers remain
      else wait_vmcnt<0>();
      barrier_nowait();  // B
      if (n + 3 < nc) issue(n + 3, 0, 2);
    }
    wait_vmcnt<0>();
  };

  if (role == S::kDma || role == S::kDma2) {
    if constexpr (NDMA == 1) dma_role(std::integral_constant<int, -1>{});
    else if (role == S::kDma) dma_role(std::integral_constant<int, 0>{});
    else dma_role(std::integral_constant<int, 1>{});
  } else if (role == S::kY0 || role == S::kY1) {
    // ----------------------------------------------------------------- Y
    const int ct = role == S::kY1 ? 1 : 0;
    Frag<uint16_t> Kf[NRT][NKU_D];
    Frag<uint16_t> Tf[NRT][NKU_C];
    bf16x4 Vt[NRT];
    auto load = [&](const uint16_t* __restrict__ cur) {  // this chunk's K, T and this tile's V
      const uint16_t* Ks = cur + S::KOFF;
      const uint16_t* Ts = cur + S::TOFF;
      const uint16_t* Vs = cur + S::VOFF;
      const int j = lane & 15;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
        Vt[rt] = lds_read_tr(Vs + swz_off<BV>(16 * rt + 4 * g + (j >> 2), 16 * ct + 4 * (j & 3)));
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15) Tf[rt][ku] = sw_frag<C>(Ts, 16 * rt + li, ku, g);
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Kf[rt][ku] = wide_frag<DK>(Ks, 16 * rt + li, ku, g);
    };
    // The slot is computed at run time here: with the three slots unrolled
    // the fragment addresses of all three stay live and the held K, T and V
    // fragments no longer fit the registers.
    for (int n = 0; n < nc; ++n) {
      const int sn = n % 3;
      sync();  // A
      if (n == 0) load(ring);
      Frag<uint16_t> bS[NKU_D];
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) bS[ku].v = bS_buf[ct][ku][lane];
      f32x4 Y[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) Y[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mma(Y[rt], Kf[rt][ku], bS[ku]);
      // D = V - Y, U' = T D, published for the S and output waves
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) Y[rt][qq] = static_cast<float>(Vt[rt][qq]) - Y[rt][qq];
      Frag<uint16_t> bD[NKU_C];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) bD[ku] = acc_frag<uint16_t>(Y[2 * ku], Y[2 * ku + 1]);
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) {
        f32x4 U0 = zero4(), U1 = zero4();
#pragma unroll
        for (int kk = 0; kk < NKU_C; ++kk) {
          if (32 * kk <= 32 * ku + 15) mma(U0, Tf[2 * ku][kk], bD[kk]);
          if (32 * kk <= 32 * ku + 31) mma(U1, Tf[2 * ku + 1][kk], bD[kk]);
        }
        bU_buf[ct][ku][lane] = acc_frag<uint16_t>(U0, U1).v;
      }
      sync();  // B
      if (n + 1 < nc) load(ring + (sn == 2 ? 0 : (sn + 1) * S::SLOT));
    }
  } else if (role == S::kS0 || role == S::kS1) {
    // ----------------------------------------------------------------- S
    // rows: logical key dims 64 hh .. 64 hh + 63 (k-units KH hh .. KH hh + KH - 1)
    const int hh = role == S::kS1 ? 1 : 0, dt0 = 2 * KH * hh, ku0 = KH * hh;
    // St[d][c][qq] = S[key_phys(16 (dt0 + d) + 4 g + qq)][v0 + 16 c + li]
    f32x4 St[2 * KH][NT];
#pragma unroll
    for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq)
          St[d][c][qq] = s0 != nullptr
                             ? s0[(int64_t(bh) * DK + key_phys(16 * (dt0 + d) + 4 * g + qq)) * DV + v0 + 16 * c + li]
                             : 0.0f;
    // S_m as operand fragments: fragment (u, c) = key dims 32 (ku0 + u) +
    // 8 g .. + 7 of column v0 + 16 c + li
    auto publish = [&]() {
#pragma unroll
      for (int u = 0; u < KH; ++u)
#pragma unroll
        for (int c = 0; c < NT; ++c) bS_buf[c][ku0 + u][lane] = acc_frag<uint16_t>(St[2 * u][c], St[2 * u + 1][c]).v;
    };
    // SAVE: chunk n's start state, from the fragments both S wavefronts
    // published: this wavefront stores rows v0 + 16 hh .. + 15 of S^T, each
    // instruction 8 rows x 128 contiguous bytes (each 16-lane read group
    // takes 8 rows x 2 pieces: two lanes per bank)
    auto save = [&](int n) {
      constexpr int PR = DK / 8;  // 16-byte pieces per row
#pragma unroll
      for (int j = 0; j < PR / 4; ++j) {
        const int rr = 8 * (j / (PR / 8)) + (lane & 7);
        const int p = 8 * (j % (PR / 8)) + 2 * (lane >> 4) + ((lane >> 3) & 1);
        const bf16x8 f = bS_buf[hh][p >> 2][16 * (p & 3) + rr];
        __builtin_nontemporal_store(
            f, reinterpret_cast<bf16x8*>(statesT + ((sp.slot0 + n) * DV + v0 + 16 * hh + rr) * DK + 8 * p));
      }
    };
    publish();
    run([&](const uint16_t* __restrict__ cur, const uint16_t*, int n) {
      sync();  // A
      Frag<uint16_t> KT[2 * KH][NKU_C];
#pragma unroll
      for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) KT[d][kt] = wide_frag_tr<DK>(cur + S::KOFF, dt0 + d, kt, lane);
      if constexpr (SAVE) save(n);
      sync();  // B
      Frag<uint16_t> bU[NT][NKU_C];
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) bU[c][kt].v = bU_buf[c][kt][lane];
#pragma unroll
      for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int kt = 0; kt < NKU_C; ++kt) mma(St[d][c], KT[d][kt], bU[c][kt]);
      publish();
    });
    if (sfin != nullptr) {
#pragma unroll
      for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            sfin[(int64_t(bh) * DK + key_phys(16 * (dt0 + d) + 4 * g + qq)) * DV + v0 + 16 * c + li] = St[d][c][qq];
    }
  } else if (S::is_output(role)) {
    // ------------------------------------------------------------- output
    // row tiles 2 rh and 2 rh + 1, both state tiles
    const int rt0 = 2 * o_rh;
    Frag<uint16_t> Qf[2][NKU_D];
    auto load = [&](const uint16_t* __restrict__ cur) {
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
#pragma unroll
        for (int r = 0; r < 2; ++r) Qf[r][ku] = wide_frag<DK>(cur + S::QOFF, 16 * (rt0 + r) + li, ku, g);
    };
    run([&](const uint16_t* __restrict__ cur, const uint16_t* __restrict__ nxt, int n) {
      sync();  // A
      if (n == 0) load(cur);
      else store_staged(n - 1, o_rh);  // both output waves staged chunk n-1 before barrier A
      // Zt[c][r][qq] = Z[16 (rt0 + r) + li][16 c + 4 g + qq]  (Z^T = S^T Q^T)
      f32x4 Zt[NT][2];
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int r = 0; r < 2; ++r) Zt[c][r] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          Frag<uint16_t> bSo;
          bSo.v = bS_buf[c][ku][lane];
#pragma unroll
          for (int r = 0; r < 2; ++r) mma(Zt[c][r], bSo, Qf[r][ku]);
        }
      sync();  // B
      // O^T = Z^T + U'^T P^T; lane (li, g) stages O[16 rt + li][16 c + 4g .. 4g + 3]
      Frag<uint16_t> bUo[NT][NKU_C];
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku) bUo[c][ku].v = bU_buf[c][ku][lane];
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int rt = rt0 + r;
        Frag<uint16_t> pf[NKU_C];
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku <= 16 * rt + 15) pf[ku].v = P_buf[pf_index(rt, ku)][lane];
#pragma unroll
        for (int c = 0; c < NT; ++c) {
          f32x4 acc = Zt[c][r];
#pragma unroll
          for (int ku = 0; ku < NKU_C; ++ku)
            if (32 * ku <= 16 * rt + 15) mma(acc, bUo[c][ku], pf[ku]);
          bf16x4 ov;
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) ov[qq] = static_cast<__bf16>(acc[qq]);
          *reinterpret_cast<bf16x4*>(&O_st[16 * rt + li][16 * c + 4 * g]) = ov;
        }
      }
      if (n + 1 < nc) load(nxt);
    });
  } else {
    // ----------------------------------------------------------------- P
    // P_n = tril(Q K^T) of chunk n for row tiles R0 .. R1-1, split over the
    // key dimension: k-units 0 .. KH-1 after barrier B of step n-1 (chunk n
    // is complete there), the rest after barrier A of step n.
    auto prole = [&](auto r0, auto r1) {
      constexpr int R0 = decltype(r0)::value, R1 = decltype(r1)::value;
      // Pt[r - R0][c][qq] = P[16 r + li][16 c + 4 g + qq] for c <= r
      f32x4 Pt[R1 - R0][R1];
      auto clear = [&]() {
#pragma unroll
        for (int r = R0; r < R1; ++r)
#pragma unroll
          for (int c = 0; c < R1; ++c) Pt[r - R0][c] = zero4();
      };
      auto accumulate = [&](const uint16_t* __restrict__ cur, int ku0, int ku1) {
#pragma unroll
        for (int ku = 0; ku < NKU_D; ++ku) {
          if (ku < ku0 || ku >= ku1) continue;
          Frag<uint16_t> Qf[R1 - R0], Kf[R1];
#pragma unroll
          for (int r = R0; r < R1; ++r) Qf[r - R0] = wide_frag<DK>(cur + S::QOFF, 16 * r + li, ku, g);
#pragma unroll
          for (int c = 0; c < R1; ++c) Kf[c] = wide_frag<DK>(cur + S::KOFF, 16 * c + li, ku, g);
#pragma unroll
          for (int r = R0; r < R1; ++r)
#pragma unroll
            for (int c = 0; c <= r; ++c) mma(Pt[r - R0][c], Kf[c], Qf[r - R0]);
        }
      };
      clear();
      run([&](const uint16_t* __restrict__ cur, const uint16_t* __restrict__ nxt, int n) {
        sync();  // A
        if (n == 0) accumulate(cur, 0, KH);
        accumulate(cur, KH, NKU_D);
#pragma unroll
        for (int r = R0; r < R1; ++r) {
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            if (4 * g + qq > li) Pt[r - R0][r][qq] = 0.0f;
#pragma unroll
          for (int ku = 0; ku < NKU_C; ++ku)
            if (32 * ku <= 16 * r + 15) {
              const f32x4 phi = (2 * ku + 1 <= r) ? Pt[r - R0][2 * ku + 1] : zero4();
              P_buf[pf_index(r, ku)][lane] = acc_frag<uint16_t>(Pt[r - R0][2 * ku], phi).v;
            }
        }
        sync();  // B
        clear();
        if (n + 1 < nc) accumulate(nxt, 0, KH);
      });
    };
    if (role == S::kP0) prole(std::integral_constant<int, 0>{}, std::integral_constant<int, NRT - 1>{});
    else prole(std::integral_constant<int, NRT - 1>{}, std::integral_constant<int, NRT>{});
  }
  // the last chunk's output: staged by every output wave before this barrier
  sync();
  if (nc > 0 && S::is_output(role)) store_staged(nc - 1, o_rh);
}

template <int DK, int C, int BV, int NDMA>
hipError_t recurrence_split_launch_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* tws, const float* s0, uint16_t* o, float* sfin, int B,
                                        int H, int64_t L, int DV, const int32_t* cu, int N, const int32_t* order,
                                        hipStream_t stream, uint16_t* statesT = nullptr) {
  const int NC = cu == nullptr ? int((L + C - 1) / C) : int(L / C) + N;  // chunk slots per sequence / head
  const int BH = (cu == nullptr ? B : N) * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  if (cu == nullptr) order = nullptr;  // dense batches keep their order
  const int remap = (BH % 8 == 0) ? 1 : 0;
  if constexpr (NDMA == 1) {
    if (statesT != nullptr) {
      hipLaunchKernelGGL((recurrence_split_kernel<DK, C, BV, NDMA, true>), dim3(unsigned(nwg)),
                         dim3(unsigned(SplitShape<DK, C, BV, NDMA>::THREADS)), 0, stream, q, k, v, tws, s0, o, sfin, H, L,
                         NC, DV, NVB, remap, cu, order, N, statesT);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((recurrence_split_kernel<DK, C, BV, NDMA>), dim3(unsigned(nwg)),
                     dim3(unsigned(SplitShape<DK, C, BV, NDMA>::THREADS)), 0, stream, q, k, v, tws, s0, o, sfin, H, L, NC,
                     DV, NVB, remap, cu, order, N);
  return hipGetLastError();
}

// ndma: DMA wavefronts per workgroup (1 or 2); statesT (non-null: one DMA
// wavefront) receives the chunk start states.
inline hipError_t launch_recurrence_split(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                          const uint16_t* tws, const float* s0, uint16_t* o, float* sfin, int B,
                                          int H, int64_t L, int DK, int DV, int C, int BV, const int32_t* cu, int N,
                                          const int32_t* order, int ndma, hipStream_t s, uint16_t* statesT = nullptr) {
  if (statesT != nullptr) ndma = 1;
  if (C == 64 && BV == 32) {
    if (DK == 64) {
      if (ndma == 2) return recurrence_split_launch_impl<64, 64, 32, 2>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, order, s);
      return recurrence_split_launch_impl<64, 64, 32, 1>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, order, s, statesT);
    }
    if (DK == 128) {
      if (ndma == 2) return recurrence_split_launch_impl<128, 64, 32, 2>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, order, s);
      return recurrence_split_launch_impl<128, 64, 32, 1>(q, k, v, tws, s0, o, sfin, B, H, L, DV, cu, N, order, s, statesT);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
