// recurrence_reverse.h -- the reverse pass over the chunks of the backward,
// in the form of the forward's state-only pass (recurrence_states.h).
//
// Per chunk, last to first, with dS' the loss gradient with respect to the
// state at the chunk's end and Qe = Q - P T K the chunk's effective queries
// (written by the backward instance of the UT transform):
//     dstates[n] = dS'
//     E = K dS',   F = T^T E
//     dS = dS' + Qe^T dO - K^T F      (the gradient at the chunk's start)
// This is the plain reverse step dS = dS' + Q^T dO - K^T T^T (P^T dO + K dS')
// with the two terms in dO gathered into Qe^T dO, so the chain needs no P and
// a chunk moves the same 44 KiB through the ring as the forward pass (K, Qe,
// T and a 32-column block of dO instead of Q, K, T and V).
//
// A workgroup owns 32 value columns (two 16-column tiles) of one (b, h):
//   * Y wave per tile: E = K dS'_tile (16 products), F = T^T E (6), publishes
//     -F as operand fragments; it reads the next chunk's K and T^T fragments
//     in the other phase.
//   * S wave per 32 key dims: holds those rows of dS (both tiles) in fp32
//     registers.  Phase A: reads its K^T, Qe^T and dO fragments of the chunk
//     and adds Qe^T dO (8 products); phase B: adds K^T (-F) (8 products),
//     publishes its rows as bf16 fragments for the next chunk and stores them,
//     eight consecutive key dims of one value column per 16-byte store, so
//     dstates is kept transposed, [slots][d_v][d_k].
//   * DMA wave: K, Qe, T and the dO block into a three-slot ring, two chunks
//     ahead, on the schedule of the forward pass.
// Two barriers per chunk; every exchange buffer is written in one phase and
// read in the other:
//   A (chunk n in LDS, dS'_n published)
//     Y: products -> publish -F_n | S: read K^T, Qe^T, dO; dS += Qe^T dO
//     | DMA: half of chunk n+2
//   B (-F_n published, chunk n+1 in LDS)
//     Y: read K, T^T of chunk n+1 | S: dS += K^T (-F) -> publish, store
//     | DMA: other half
// Tokens past the end of the last chunk: the ring's K and dO rows there
// repeat row 0, but Qe's rows there are zero (its workspace slot has C rows)
// and so are T's rows and columns, so they add nothing.
#pragma once

#include <type_traits>

#include "lds_ring.h"

namespace efla {

template <int DK, int C, int BV>
struct ReverseShape {
  static_assert(C == 64 && BV == 32 && (DK == 64 || DK == 128), "shapes of the reverse pass");
  static constexpr int NT = BV / 16;  // dS tiles per workgroup
  static constexpr int NRT = C / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int NSW = NKU_D;  // S waves, 32 key dims each
  static constexpr int KOFF = 0, QOFF = C * DK, TOFF = 2 * C * DK, OOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;
  using TK = DmaTile<C, DK, 1, true>;  // K and Qe: 16-byte-fragment swizzle
  using TT = DmaTile<C, C, 1>;
  using TO = DmaTile<C, BV, 1>;
  static constexpr int PK = TK::PER_WAVE, PT = TT::PER_WAVE, PO = TO::PER_WAVE;
  static constexpr int COUNT = 2 * PK + PT + PO;  // transfers per chunk
  static constexpr int kY0 = 0, kS0 = 2, kDma = 2 + NSW, NWAVES = 3 + NSW, THREADS = NWAVES * kWave;
};

inline bool reverse_supported(int DK, int DV, int C) {
  return C == 64 && DV % 32 == 0 && (DK == 64 || DK == 128);
}

// dense batch [B][L][H][*]; NVB = DV / BV workgroups per (b, h).  qe and tws
// are per chunk slot ((b H + h) NC + n): [slots][C][DK] and [slots][C][C].
// dsf: gradient with respect to the final state, fp32 [B H][DK][DV] (NULL:
// zero); ds0: the gradient with respect to the initial state, same layout.
template <int DK, int C, int BV>
__global__ __launch_bounds__((64 * ReverseShape<DK, C, BV>::NWAVES)) void reverse_states_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ qe, const uint16_t* __restrict__ tws,
    const uint16_t* __restrict__ dout, const float* __restrict__ dsf, float* __restrict__ ds0,
    uint16_t* __restrict__ dstatesT, int H, int64_t L, int NC, int DV, int NVB, int remap) {
  using S = ReverseShape<DK, C, BV>;
  constexpr int NT = S::NT, NRT = S::NRT, NKU_D = S::NKU_D, NKU_C = S::NKU_C;
  __shared__ __align__(1024) uint16_t ring[3 * S::SLOT];
  uint16_t* const slot0 = ring;
  uint16_t* const slot1 = ring + S::SLOT;
  uint16_t* const slot2 = ring + 2 * S::SLOT;
  __shared__ __align__(16) bf16x8 bS_buf[NT][NKU_D][kWave];  // dS' as operand fragments
  __shared__ __align__(16) bf16x8 bF_buf[NT][NKU_C][kWave];  // -F as operand fragments

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
  const int64_t h = bh % H;
  const SeqSpan sp = seq_span<C>(nullptr, bh / H, h, H, L, NC);
  const int nc = sp.nc;
  const int v0 = vb * BV;
  const int lane = threadIdx.x & 63, role = wave_id(), li = lane & 15, g = lane >> 4;
  // step n processes chunk nc - 1 - n
  auto chunk_of = [&](int n) { return nc - 1 - n; };
  auto chunk_valid = [&](int m) { return int(sp.len - int64_t(m) * C < C ? sp.len - int64_t(m) * C : C); };
  auto row_of = [&](int m) { return (sp.bos + int64_t(m) * C) * H + h; };
  auto sync = [&]() {
    wait_lgkm0();
    barrier_nowait();
  };
  auto run = [&](auto&& step) {  // steps of three keep the ring slots compile-time addresses
    for (int n = 0; n < nc; n += 3) {
      step(slot0, n);
      if (n + 1 < nc) step(slot1, n + 1);
      if (n + 2 < nc) step(slot2, n + 2);
    }
  };

  if (role == S::kDma) {
    // ---------------------------------------------------------------- DMA
    // The forward pass's schedule (recurrence_split.h): step n+3's chunk goes
    // into step n's slot half after barrier B of step n and half after
    // barrier A of step n+1; before barrier B of step n only step n+2's
    // transfers may remain (waits counted against one chunk's transfers).
    constexpr int D = S::COUNT;
    static_assert(D < 64, "one chunk's transfers fit the vmcnt counter");
    typename S::TK tk, tq;
    typename S::TT tt;
    typename S::TO to;
    tk.init(int64_t(H) * DK, lane, 0);
    tq.init(DK, lane, 0);
    tt.init(C, lane, 0);
    to.init(int64_t(H) * DV, lane, 0);
    auto issue = [&](int n, int part, int parts) {
      const int m = chunk_of(n);
      const int64_t r0 = row_of(m);
      const auto* ks = static_cast<const uint16_t*>(uniform_ptr(k + r0 * DK));
      const auto* qs = static_cast<const uint16_t*>(uniform_ptr(qe + (sp.slot0 + m) * C * DK));
      const auto* ts = static_cast<const uint16_t*>(uniform_ptr(tws + (sp.slot0 + m) * C * C));
      const auto* os = static_cast<const uint16_t*>(uniform_ptr(dout + r0 * DV + v0));
      const int valid = chunk_valid(m);
      const uint32_t addr = lds_addr_of(ring + (n % 3) * S::SLOT);
      auto body = [&](auto ragged) {
        constexpr bool R = decltype(ragged)::value;
#pragma unroll
        for (int j = 0; j < D; ++j) {
          if (j < part * D / parts || j >= (part + 1) * D / parts) continue;
          if (j < S::PK) tk.template issue<R>(j, addr + 2 * S::KOFF, ks, valid);
          else if (j < 2 * S::PK) tq.template issue<false>(j - S::PK, addr + 2 * S::QOFF, qs, C);
          else if (j < 2 * S::PK + S::PT) tt.template issue<false>(j - 2 * S::PK, addr + 2 * S::TOFF, ts, C);
          else to.template issue<R>(j - 2 * S::PK - S::PT, addr + 2 * S::OOFF, os, valid);
        }
      };
      if (valid == C) body(std::false_type{});
      else body(std::true_type{});
    };
    if (nc > 0) issue(0, 0, 1);
    if (nc > 1) {
      issue(1, 0, 1);
      wait_vmcnt<D>();  // step 0's chunk complete
    } else {
      wait_vmcnt<0>();
    }
    if (nc > 2) issue(2, 0, 2);
    for (int n = 0; n < nc; ++n) {
      barrier_nowait();  // A
      if (n + 2 < nc) issue(n + 2, 1, 2);
      if (n + 2 < nc) wait_vmcnt<D>();  // step n+1's chunk complete
      else wait_vmcnt<0>();
      barrier_nowait();  // B
      if (n + 3 < nc) issue(n + 3, 0, 2);
    }
    wait_vmcnt<0>();
  } else if (role < S::kS0) {
    // ----------------------------------------------------------------- Y
    const int ct = role - S::kY0;
    Frag<uint16_t> Kf[NRT][NKU_D];
    Frag<uint16_t> Tf[NRT][NKU_C];  // T^T: row tile rt, k-unit ku (T^T is upper triangular: ku >= rt / 2)
    auto load = [&](const uint16_t* __restrict__ cur) {
      const uint16_t* Ks = cur + S::KOFF;
      const uint16_t* Ts = cur + S::TOFF;
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ku = 0; ku < NKU_C; ++ku)
          if (32 * ku + 31 >= 16 * rt) Tf[rt][ku] = sw_frag_tr<C>(Ts, 16 * rt, ku, lane);
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
      for (int ku = 0; ku < NKU_D; ++ku) bS[ku].v = bS_buf[ct][ku][lane];
      f32x4 E[NRT];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt) E[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) mma(E[rt], Kf[rt][ku], bS[ku]);
      Frag<uint16_t> bE[NKU_C];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) bE[ku] = acc_frag<uint16_t>(E[2 * ku], E[2 * ku + 1]);
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) {
        f32x4 F0 = zero4(), F1 = zero4();
#pragma unroll
        for (int kk = ku; kk < NKU_C; ++kk) {
          mma(F0, Tf[2 * ku][kk], bE[kk]);
          mma(F1, Tf[2 * ku + 1][kk], bE[kk]);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          F0[qq] = -F0[qq];
          F1[qq] = -F1[qq];
        }
        bF_buf[ct][ku][lane] = acc_frag<uint16_t>(F0, F1).v;
      }
      sync();  // B
      if (n + 1 < nc) load(ring + (sn == 2 ? 0 : (sn + 1) * S::SLOT));
    }
  } else {
    // ----------------------------------------------------------------- S
    // rows: logical key dims 32 s .. 32 s + 31 of dS
    const int sw = role - S::kS0, col0 = v0;
    // St[d][c][qq] = dS[key_phys(16 (2 sw + d) + 4 g + qq)][col0 + 16 c + li]
    f32x4 St[2][NT];
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int key = key_phys(16 * (2 * sw + d) + 4 * g + qq);
          St[d][c][qq] = dsf != nullptr ? dsf[(int64_t(bh) * DK + key) * DV + col0 + 16 * c + li] : 0.0f;
        }
    // dS' as operand fragments: fragment c holds key dims 32 sw + 8 g .. + 7
    // of column col0 + 16 c + li
    auto publish = [&]() {
#pragma unroll
      for (int c = 0; c < NT; ++c) bS_buf[c][sw][lane] = acc_frag<uint16_t>(St[0][c], St[1][c]).v;
    };
    // dstates[m] (m: the chunk of this step, whose end-gradient the buffer
    // holds), from the fragments every S wavefront published: this wavefront
    // stores its share of the rows of dS'^T (8 with d_k 128, 16 with d_k 64),
    // each instruction 8 rows x 128 contiguous bytes (two lanes per bank in
    // each 16-lane read group), nontemporal; every row is written whole
    // (from the registers, 64-byte pieces from several wavefronts wrote 1.16x
    // the bytes)
    auto save = [&](int m) {
      constexpr int PR = DK / 8, RW = BV / NKU_D;  // 16-byte pieces per row, rows per S wavefront
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = RW * sw + 8 * (PR == 16 ? 0 : j) + (lane & 7);
        const int p = 8 * (PR == 16 ? j : 0) + 2 * (lane >> 4) + ((lane >> 3) & 1);
        const bf16x8 f = bS_buf[r >> 4][p >> 2][16 * (p & 3) + (r & 15)];
        __builtin_nontemporal_store(
            f, reinterpret_cast<bf16x8*>(dstatesT + ((sp.slot0 + m) * DV + col0 + r) * DK + 8 * p));
      }
    };
    publish();
    run([&](const uint16_t* __restrict__ cur, int n) {
      sync();  // A
      save(chunk_of(n));
      Frag<uint16_t> KT[2][NKU_C], QT[2][NKU_C], dOf[NT][NKU_C];
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) {
          KT[d][kt] = wide_frag_tr<DK>(cur + S::KOFF, 2 * sw + d, kt, lane);
          QT[d][kt] = wide_frag_tr<DK>(cur + S::QOFF, 2 * sw + d, kt, lane);
        }
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) dOf[c][kt] = sw_frag_tr<BV>(cur + S::OOFF, 16 * c, kt, lane);
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int kt = 0; kt < NKU_C; ++kt) mma(St[d][c], QT[d][kt], dOf[c][kt]);
      sync();  // B
      Frag<uint16_t> bF[NT][NKU_C];
#pragma unroll
      for (int c = 0; c < NT; ++c)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt) bF[c][kt].v = bF_buf[c][kt][lane];
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int kt = 0; kt < NKU_C; ++kt) mma(St[d][c], KT[d][kt], bF[c][kt]);
      publish();
    });
    if (ds0 != nullptr) {
#pragma unroll
      for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int c = 0; c < NT; ++c)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq)
            ds0[(int64_t(bh) * DK + key_phys(16 * (2 * sw + d) + 4 * g + qq)) * DV + col0 + 16 * c + li] =
                St[d][c][qq];
    }
  }
}

template <int DK, int C, int BV>
hipError_t reverse_states_launch_impl(const uint16_t* k, const uint16_t* qe, const uint16_t* tws,
                                      const uint16_t* dout, const float* dsf, float* ds0, uint16_t* dstatesT, int B,
                                      int H, int64_t L, int DV, hipStream_t stream) {
  const int NC = int((L + C - 1) / C);
  const int BH = B * H, NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((reverse_states_kernel<DK, C, BV>), dim3(unsigned(nwg)),
                     dim3(unsigned(ReverseShape<DK, C, BV>::THREADS)), 0, stream, k, qe, tws, dout, dsf, ds0,
                     dstatesT, H, L, NC, DV, NVB, remap);
  return hipGetLastError();
}

}  // namespace efla
