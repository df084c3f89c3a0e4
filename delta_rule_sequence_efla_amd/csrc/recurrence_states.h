// recurrence_states.h -- the state-only chunk pass of the segment scan.
//
// Over a run of chunks the recurrence is affine in its start state,
//     S_end = M S_start + N,
// where N is the state the run reaches from zero with the true values and M,
// the product of the chunk transitions (I - K^T T K), is the state it reaches
// from the identity with V = 0 (d_k "value" columns).  This kernel forms both
// in one pass: a workgroup owns 32 columns of N and 32 columns of M of one
// (segment, head), so each chunk's K and T cross HBM and the LDS ring once
// for the two.  There is no Q and no output, so a chunk is 28 transfers of
// 1 KiB (d_k = 128) instead of the forward pass's 44.
//   * Y wave per chain and 16-column tile: Y = K S, D = V - Y (N) or -Y (M),
//     U' = T D, published as operand fragments.  The next chunk's K, T (and
//     V) fragments are read in the other phase.
//   * S wave per chain and half of the key dimension: holds those 64 rows of
//     its chain's state in fp32 registers, reads its K^T fragments in the
//     phase before, then S += K^T U' and publishes its rows as bf16 fragments.
//   * DMA wave: streams K, T and V into a three-slot ring two chunks ahead.
// The four Y waves sit on four different SIMDs, and so do the four S waves,
// so the two chains' products never share a matrix core.  Two barriers per
// chunk:
//   A (chunk n in LDS, S_n published)
//     Y: products -> publish U'_n | S: read K^T_n | DMA: half of chunk n+2
//   B (U'_n published, chunk n+1 in LDS)
//     Y: read K, T, V of chunk n+1 | S: S += K^T U' -> publish S_{n+1}
//     | DMA: other half
// Every exchange buffer is written in one phase and read in the other.
//
// The same kernel with BWD set runs one chain, the true recurrence from the
// initial state, for the backward pass: it writes the state at the start of
// every chunk, as the bf16 values the forward products use, transposed
// ([d_v][d_k] per chunk slot): each S wave's published operand fragment is
// eight consecutive key dims of one value column, one 16-byte store.  Five
// wavefronts: Y tiles 0 and 1, S halves 0 and 1, DMA.
#pragma once

#include <type_traits>

#include "lds_ring.h"

namespace efla {

template <int DK, int C, int BV, bool BWD = false>
struct StatesShape {
  static_assert(C == 64 && BV == 32 && (DK == 64 || DK == 128), "shapes of the state-only pass");
  static constexpr int NT = BV / 16;  // state tiles per chain
  static constexpr int NRT = C / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int KH = NKU_D / 2;  // key k-units per S wave
  static constexpr int KOFF = 0, TOFF = C * DK, VOFF = C * DK + C * C;
  static constexpr int SLOT = C * DK + C * C + C * BV;
  using TK = DmaTile<C, DK, 1, true>;  // 16-byte-fragment swizzle, as wide_frag reads it
  using TT = DmaTile<C, C, 1>;
  using TV = DmaTile<C, BV, 1>;
  static constexpr int PK = TK::PER_WAVE, PT = TT::PER_WAVE, PV = TV::PER_WAVE;
  static constexpr int COUNT = PK + PT + PV;  // transfers per chunk
  // waves: Y (chain 0 tiles 0-1[, chain 1 tiles 0-1]), S (same order), DMA
  static constexpr int NCH = BWD ? 1 : 2;  // chains
  static constexpr int kY0 = 0, kS0 = 2 * NCH, kDma = 4 * NCH, NWAVES = 4 * NCH + 1, THREADS = NWAVES * kWave;
};

inline bool states_supported(int DK, int C, int BV) { return C == 64 && BV == 32 && (DK == 64 || DK == 128); }

// N [nseq * H, DK, DV] and M [nseq * H, DK, DK], fp32, rows indexed by key
// dim.  NVB = max(DV, DK) / BV workgroups per (sequence, head); the first
// NVB_N = DV / BV of them write N, the first NVB_M = DK / BV write M.
// BWD: chain 0 starts from s0 (NULL: zeros) and NVB = NVB_N; statesT gets
// the bf16 start state of every chunk slot, [slots][DV][DK]; nout and mout
// are not used.
template <int DK, int C, int BV, bool BWD>
__global__ __launch_bounds__((64 * StatesShape<DK, C, BV, BWD>::NWAVES)) void recurrence_states_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const uint16_t* __restrict__ tws,
    float* __restrict__ nout, float* __restrict__ mout, int H, int64_t L, int NC, int DV, int NVB, int NVB_N,
    int NVB_M, int remap, const int32_t* __restrict__ cu, const float* __restrict__ s0,
    uint16_t* __restrict__ statesT) {
  using S = StatesShape<DK, C, BV, BWD>;
  constexpr int NT = S::NT, NRT = S::NRT, NKU_D = S::NKU_D, NKU_C = S::NKU_C, KH = S::KH;
  __shared__ __align__(1024) uint16_t ring[3 * S::SLOT];
  uint16_t* const slot0 = ring;
  uint16_t* const slot1 = ring + S::SLOT;
  uint16_t* const slot2 = ring + 2 * S::SLOT;
  __shared__ __align__(16) bf16x8 bS_buf[S::NCH][NT][NKU_D][kWave];  // S_n of each chain as operand fragments
  __shared__ __align__(16) bf16x8 bU_buf[S::NCH][NT][NKU_C][kWave];  // U'_n of each chain

  const int x = blockIdx.x;
  int bh, vb;
  if (remap) {  // all column blocks of one (sequence, head) on one XCD (same blockIdx % 8)
    const int slot = x >> 3;
    vb = slot % NVB;
    bh = (slot / NVB) * 8 + (x & 7);
  } else {
    bh = x / NVB;
    vb = x % NVB;
  }
  const int64_t h = bh % H;
  const SeqSpan sp = seq_span<C>(cu, bh / H, h, H, L, NC);
  const int nc = sp.nc;
  // chain 0 (N) reads value columns vn0..; a block past d_v repeats the last
  // one and stores nothing (likewise chain 1 past d_k)
  const int vn0 = (vb < NVB_N ? vb : NVB_N - 1) * BV, m0 = vb * BV;
  const int lane = threadIdx.x & 63, role = wave_id(), li = lane & 15, g = lane >> 4;
  auto chunk_valid = [&](int n) { return int(sp.len - int64_t(n) * C < C ? sp.len - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (sp.bos + int64_t(n) * C) * H + h; };
  auto sync = [&]() {
    wait_lgkm0();
    barrier_nowait();
  };
  auto run = [&](auto&& step) {
    for (int n = 0; n < nc; n += 3) {
      step(slot0, n);
      if (n + 1 < nc) step(slot1, n + 1);
      if (n + 2 < nc) step(slot2, n + 2);
    }
  };

  if (role == S::kDma) {
    // ---------------------------------------------------------------- DMA
    // Same schedule as the split forward pass: chunk n+3 goes into chunk n's
    // slot half after barrier B of step n and half after barrier A of step
    // n+1; before barrier B of step n only chunk n+2's transfers may remain.
    constexpr int D = S::COUNT;
    static_assert(2 * D < 64, "two chunks' transfers fit the vmcnt counter");
    typename S::TK tk;
    typename S::TT tt;
    typename S::TV tv;
    tk.init(int64_t(H) * DK, lane, 0);
    tt.init(C, lane, 0);
    tv.init(int64_t(H) * DV, lane, 0);
    auto issue = [&](int m, int part, int parts) {
      const int64_t r0 = row_of(m);
      const auto* ks = static_cast<const uint16_t*>(uniform_ptr(k + r0 * DK));
      const auto* ts = static_cast<const uint16_t*>(uniform_ptr(tws + (sp.slot0 + m) * C * C));
      const auto* vs = static_cast<const uint16_t*>(uniform_ptr(v + r0 * DV + vn0));
      const int valid = chunk_valid(m);
      const uint32_t addr = lds_addr_of(ring + (m % 3) * S::SLOT);
      auto body = [&](auto ragged) {
        constexpr bool R = decltype(ragged)::value;
#pragma unroll
        for (int j = 0; j < D; ++j) {
          if (j < part * D / parts || j >= (part + 1) * D / parts) continue;
          if (j < S::PK) tk.template issue<R>(j, addr + 2 * S::KOFF, ks, valid);
          else if (j < S::PK + S::PT) tt.template issue<false>(j - S::PK, addr + 2 * S::TOFF, ts, C);
          else tv.template issue<R>(j - S::PK - S::PT, addr + 2 * S::VOFF, vs, valid);
        }
      };
      if (valid == C) body(std::false_type{});
      else body(std::true_type{});
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
      if (n + 2 < nc) wait_vmcnt<D>();  // chunk n+1 complete
      else wait_vmcnt<0>();
      barrier_nowait();  // B
      if (n + 3 < nc) issue(n + 3, 0, 2);
    }
    wait_vmcnt<0>();
  } else if (role < S::kS0) {
    // ----------------------------------------------------------------- Y
    auto yrole = [&](auto chain) {
      constexpr int CH = decltype(chain)::value;
      const int ct = role & 1;
      Frag<uint16_t> Kf[NRT][NKU_D];
      Frag<uint16_t> Tf[NRT][NKU_C];
      bf16x4 Vt[NRT];
      auto load = [&](const uint16_t* __restrict__ cur) {
        const uint16_t* Ks = cur + S::KOFF;
        const uint16_t* Ts = cur + S::TOFF;
        if constexpr (CH == 0) {
          const uint16_t* Vs = cur + S::VOFF;
          const int j = lane & 15;
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt)
            Vt[rt] = lds_read_tr(Vs + swz_off<BV>(16 * rt + 4 * g + (j >> 2), 16 * ct + 4 * (j & 3)));
        }
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
      for (int n = 0; n < nc; ++n) {
        const int sn = n % 3;
        sync();  // A
        if (n == 0) load(ring);
        Frag<uint16_t> bS[NKU_D];
#pragma unroll
        for (int ku = 0; ku < NKU_D; ++ku) bS[ku].v = bS_buf[CH][ct][ku][lane];
        f32x4 Y[NRT];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) Y[rt] = zero4();
#pragma unroll
        for (int ku = 0; ku < NKU_D; ++ku)
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) mma(Y[rt], Kf[rt][ku], bS[ku]);
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            if constexpr (CH == 0) Y[rt][qq] = static_cast<float>(Vt[rt][qq]) - Y[rt][qq];
            else Y[rt][qq] = -Y[rt][qq];
          }
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
          bU_buf[CH][ct][ku][lane] = acc_frag<uint16_t>(U0, U1).v;
        }
        sync();  // B
        if (n + 1 < nc) load(ring + (sn == 2 ? 0 : (sn + 1) * S::SLOT));
      }
    };
    if constexpr (BWD) {
      yrole(std::integral_constant<int, 0>{});
    } else {
      if (role < S::kY0 + 2) yrole(std::integral_constant<int, 0>{});
      else yrole(std::integral_constant<int, 1>{});
    }
  } else {
    // ----------------------------------------------------------------- S
    // rows: logical key dims 64 hh .. 64 hh + 63 of chain ch's state
    const int ch = (role - S::kS0) >> 1, hh = (role - S::kS0) & 1, dt0 = 2 * KH * hh, ku0 = KH * hh;
    // St[d][c][qq] = S[key_phys(16 (dt0 + d) + 4 g + qq)][col0 + 16 c + li]
    const int col0 = ch == 0 ? vn0 : m0;
    f32x4 St[2 * KH][NT];
#pragma unroll
    for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int key = key_phys(16 * (dt0 + d) + 4 * g + qq);
          if constexpr (BWD)
            St[d][c][qq] = s0 != nullptr ? s0[(int64_t(bh) * DK + key) * DV + col0 + 16 * c + li] : 0.0f;
          else
            St[d][c][qq] = (ch == 1 && key == col0 + 16 * c + li) ? 1.0f : 0.0f;
        }
    // S_m as operand fragments: fragment (u, c) holds key dims 32 (ku0 + u)
    // + 8 g .. + 7 of column col0 + 16 c + li
    auto publish = [&]() {
#pragma unroll
      for (int u = 0; u < KH; ++u)
#pragma unroll
        for (int c = 0; c < NT; ++c)
          bS_buf[ch][c][ku0 + u][lane] = acc_frag<uint16_t>(St[2 * u][c], St[2 * u + 1][c]).v;
    };
    // BWD: the start state of chunk n, from the fragments both S wavefronts
    // published: this wavefront stores rows col0 + 16 hh .. + 15 of S^T, each
    // instruction 8 rows x 128 contiguous bytes (each 16-lane read group
    // takes 8 rows x 2 pieces: two lanes per bank), nontemporal (plain stores
    // stalled this wave's LDS reads: 1.4x longer pass).  Stored so, every
    // row is written whole (from the registers, 64-byte pieces from two
    // wavefronts wrote 1.3x the bytes).
    auto save = [&](int n) {
      constexpr int PR = DK / 8;  // 16-byte pieces per row
#pragma unroll
      for (int j = 0; j < PR / 4; ++j) {
        const int rr = 8 * (j / (PR / 8)) + (lane & 7);
        const int p = 8 * (j % (PR / 8)) + 2 * (lane >> 4) + ((lane >> 3) & 1);
        const bf16x8 f = bS_buf[ch][hh][p >> 2][16 * (p & 3) + rr];
        __builtin_nontemporal_store(
            f, reinterpret_cast<bf16x8*>(statesT + ((sp.slot0 + n) * DV + col0 + 16 * hh + rr) * DK + 8 * p));
      }
    };
    publish();
    run([&](const uint16_t* __restrict__ cur, int n) {
      sync();  // A
      Frag<uint16_t> KT[2 * KH][NKU_C];
#pragma unroll
      for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) KT[d][kt] = wide_frag_tr<DK>(cur + S::KOFF, dt0 + d, kt, lane);
      if constexpr (BWD) save(n);
      sync();  // B
      Frag<uint16_t> bU[NT][NKU_C];
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) bU[c][kt].v = bU_buf[ch][c][kt][lane];
#pragma unroll
      for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int kt = 0; kt < NKU_C; ++kt) mma(St[d][c], KT[d][kt], bU[c][kt]);
      publish();
    });
    const bool owner = !BWD && (ch == 0 ? vb < NVB_N : vb < NVB_M);
    float* const out = ch == 0 ? nout : mout;
    const int pitch = ch == 0 ? DV : DK;
    if (owner) {
#pragma unroll
      for (int d = 0; d < 2 * KH; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            out[(int64_t(bh) * DK + key_phys(16 * (dt0 + d) + 4 * g + qq)) * pitch + col0 + 16 * c + li] =
                St[d][c][qq];
    }
  }
}

template <int DK, int C, int BV, bool BWD>
hipError_t recurrence_states_launch_impl(const uint16_t* k, const uint16_t* v, const uint16_t* tws, float* nout,
                                         float* mout, int B, int H, int64_t L, int DV, const int32_t* cu, int N,
                                         const float* s0, uint16_t* statesT, hipStream_t stream) {
  const int NC = cu == nullptr ? int((L + C - 1) / C) : int(L / C) + N;
  const int BH = (cu == nullptr ? B : N) * H;
  const int NVB_N = DV / BV, NVB_M = BWD ? 0 : DK / BV;
  const int NVB = NVB_N > NVB_M ? NVB_N : NVB_M;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((recurrence_states_kernel<DK, C, BV, BWD>), dim3(unsigned(nwg)),
                     dim3(unsigned(StatesShape<DK, C, BV, BWD>::THREADS)), 0, stream, k, v, tws, nout, mout, H, L,
                     NC, DV, NVB, NVB_N, NVB_M, remap, cu, s0, statesT);
  return hipGetLastError();
}

}  // namespace efla
