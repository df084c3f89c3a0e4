// bwd_chunk_tr.h -- the per-chunk gradients of the backward pass for bf16
// inputs in ~76 KiB of LDS, so that two workgroups share a compute unit and
// one's loads and barriers overlap the other's products.
//
// Same formulas, value blocks and roundings as bwd_chunk_bf16_kernel
// (bwd_bf16.h):
//     D = V - K S      dU = P^T dO + K dS'      U = T D      dD = T^T dU (= dV)
//     dQ += dO S^T     dK += U dS'^T - dD S^T   dP += dO U^T  dT += dU D^T
// per block of 32 value columns, then the UT-transform part
//     dQ += dP K;  dK += dP^T Q;  dX = dT diag(a);  da_j = sum_i dT_ij X_ij;
//     W = X^T dX;  dA = -W X^T (strictly lower);  da_i += sum_{j<i} dA_ij G_ij;
//     dG = diag(a) dA;  dbeta, dlambda;  dK += (dG + dG^T) K + 2 diag(dlambda) K.
// What differs is the layout: every operand is held once, as a swizzled bf16
// tile, and read in whichever orientation a product needs -- rows as 16- or
// 8-byte fragments, columns by transposing reads (ds_read_b64_tr_b16) --
// instead of in both layouts; the fp32 C x C arrays of the UT-transform part
// take the space of the value-block arrays, and W and dA share one.  K, the
// states S and dS' come in the key-dimension order of the recurrence kernels
// (lds_ring.h), so the products over the key dimension pair them as stored,
// and dQ, dK come out with logical key columns, mapped back when stored.  The
// states and dS' are read transposed, [slots][d_v][d_k], as the state-only
// passes write them.  Eight wavefronts; the VGPRs stay at most 128 so that
// two workgroups fit a SIMD's register file.
#pragma once

#include <type_traits>

#include "bwd_kernels.h"
#include "lds_ring.h"

namespace efla {

constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <int DK, int C>
struct BwdTrShape {
  static_assert(C == 64 && (DK == 64 || DK == 128), "shapes of the two-workgroup per-chunk kernel");
  static constexpr int BV = 32, NWV = 8, NTH = NWV * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int NQ = NRT * NDT / NWV;  // dQ / dK tiles per wavefront
  static constexpr int NP = NRT * NRT / NWV;  // dP / dT (and C x C) tiles per wavefront
  static constexpr int CPF = C + 4;           // pitch (floats) of the fp32 C x C arrays
  // byte offsets; the loop's arrays
  static constexpr int KT = 0;                 // K [C][DK] (stays to the end)
  static constexpr int TT = KT + C * DK * 2;   // T [C][C]
  static constexpr int PT = TT + C * C * 2;    // P [C][C]
  static constexpr int ST = PT + C * C * 2;    // S^T of the value block [BV][DK]
  static constexpr int DST = ST + BV * DK * 2;  // dS'^T [BV][DK]
  static constexpr int VT = DST + BV * DK * 2;  // V block [C][BV]
  static constexpr int DOT = VT + C * BV * 2;   // dO block
  static constexpr int DT = DOT + C * BV * 2;   // D
  static constexpr int DUT = DT + C * BV * 2;   // dU
  static constexpr int UT = DUT + C * BV * 2;   // U
  static constexpr int DDT = UT + C * BV * 2;   // dD
  static constexpr int LOOP_END = DDT + C * BV * 2;
  // the UT-transform part's arrays, in three regions after K:
  //   R1: Q [C][DK] and dP [C][C] (bf16), then dX (bf16 high and low parts),
  //       then dA (fp32 [C][CPF]), then dK staged for the stores ([C][DK + 8])
  //   A0: dT (fp32 [C][CPF]), then W (bf16 high and low parts), then dQ staged
  //   XF: X (bf16 high and low parts), then dG + dG^T (bf16)
  static constexpr int CPG = DK + 8;            // pitch of the staged dQ, dK rows
  static constexpr int QT = TT;
  static constexpr int DPT = QT + C * DK * 2;
  static constexpr int DXH = TT, DXL = DXH + C * C * 2, DAF = TT, DKS = TT;
  static constexpr int R1_BYTES = cmax(cmax(C * DK * 2 + C * C * 2, C * CPF * 4), cmax(4 * C * C, C * CPG * 2));
  static constexpr int A0 = TT + R1_BYTES;
  static constexpr int WH = A0, WL = A0 + C * C * 2, DQS = A0;
  static constexpr int A0_BYTES = cmax(C * CPF * 4, C * CPG * 2);
  static constexpr int XF = A0 + A0_BYTES;
  static constexpr int XH = XF, XL = XF + C * C * 2, EB = XF;
  static constexpr int RED = XF + 4 * C * C;    // partial sums, one per thread
  using TS = DmaTile<BV, DK, NWV, true>;  // a value block's S^T or dS'^T rows (16-byte-fragment swizzle)
  using TV = DmaTile<C, BV, NWV>;         // its V or dO rows
  using TK = DmaTile<C, DK, NWV, true>;   // K, Q
  using TC = DmaTile<C, C, NWV>;          // T, P
  static constexpr int TAIL_END = RED + NTH * 4;
  static constexpr int BYTES = LOOP_END > TAIL_END ? LOOP_END : TAIL_END;
};

inline bool bwd_chunk_tr_supported(int DK, int DV, int C) {
  return C == 64 && (DK == 64 || DK == 128) && DV % 32 == 0;
}

// `states` and `dstates`: [slots][DV][DK] bf16 (the chunk's start state and the
// loss gradient at its end, transposed).
template <int DK, int C>
__global__ __launch_bounds__((BwdTrShape<DK, C>::NTH)) __attribute__((amdgpu_waves_per_eu(4, 4))) void bwd_chunk_tr_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ beta, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ tws,
    const float* __restrict__ xws, const float* __restrict__ aws, const uint16_t* __restrict__ pws,
    const uint16_t* __restrict__ states, const uint16_t* __restrict__ dstates, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, uint16_t* __restrict__ dbeta, int H, int64_t L, int NC,
    int DV, int rule) {
  using S = BwdTrShape<DK, C>;
  constexpr int BV = S::BV, NRT = S::NRT, NDT = S::NDT, NKU_D = S::NKU_D, NKU_C = S::NKU_C, NWV = S::NWV;
  constexpr int NTH = S::NTH, NQ = S::NQ, NP = S::NP, CPF = S::CPF;
  __shared__ __align__(1024) unsigned char lds[S::BYTES];
  __shared__ float as[C], das[C], dls[C], lam[C];
  auto b16 = [&](int off) { return reinterpret_cast<uint16_t*>(lds + off); };
  auto f32p = [&](int off) { return reinterpret_cast<float*>(lds + off); };
  uint16_t *Kt = b16(S::KT), *Tt = b16(S::TT), *Pt = b16(S::PT), *St = b16(S::ST), *dSt = b16(S::DST);
  uint16_t *Vt = b16(S::VT), *dOt = b16(S::DOT), *Dt = b16(S::DT), *dUt = b16(S::DUT), *Ut = b16(S::UT);
  uint16_t* dDt = b16(S::DDT);

  const int64_t slot = blockIdx.x;
  const int n = int(slot % NC);
  const int64_t bh = slot / NC, h = bh % H;
  const SeqSpan sp = seq_span<C>(nullptr, int(bh / H), h, H, L, NC);
  const int64_t t0 = int64_t(n) * C;
  const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
  const int64_t row0 = (sp.bos + t0) * H + h;
  const int tid = threadIdx.x, lane0 = tid & 63, w = wave_id(), li0 = lane0 & 15, g0 = lane0 >> 4;
  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;
  auto ld16 = [](const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); };
  auto st16 = [](uint16_t* p, const u32x4& x) { *reinterpret_cast<u32x4*>(p) = x; };
  constexpr u32x4 Z{0u, 0u, 0u, 0u};

  // ---- the chunk's K, T, P: direct global -> LDS transfers, issued with the
  // first value block's (rows of K past the end of the sequence re-read row 0
  // and are cleared with the block's)
  constexpr int UK = C * DK / 8;  // 16-byte units of a [C][DK] tile
  static_assert(UK % NTH == 0, "whole units per thread");
  typename S::TK dma_k;
  typename S::TC dma_c;
  dma_k.init(qk_stride, lane0, w);
  dma_c.init(C, lane0, w);
  {
    const auto* ks = static_cast<const uint16_t*>(uniform_ptr(k + row0 * DK));
    const auto* ts = static_cast<const uint16_t*>(uniform_ptr(tws + slot * C * C));
    const auto* ps = static_cast<const uint16_t*>(uniform_ptr(pws + slot * C * C));
#pragma unroll
    for (int i = 0; i < S::TK::PER_WAVE; ++i) {
      if (valid == C) dma_k.template issue<false>(i, lds_addr_of(Kt), ks, C);
      else dma_k.template issue<true>(i, lds_addr_of(Kt), ks, valid);
    }
#pragma unroll
    for (int i = 0; i < S::TC::PER_WAVE; ++i) {
      dma_c.template issue<false>(i, lds_addr_of(Tt), ts, C);
      dma_c.template issue<false>(i, lds_addr_of(Pt), ps, C);
    }
  }
  if (tid < C) as[tid] = aws[slot * C + tid];

  // ---- one value block's S^T, dS'^T, V and dO: direct global -> LDS
  // transfers spread over the wavefronts, so nothing is held in registers
  // across a block (register staging cost ~16 VGPRs over the 128 two
  // workgroups per compute unit allow).  Rows of V and dO past the end of the
  // sequence are cleared after the transfers (they re-read row 0).
  typename S::TS dma_s;
  typename S::TV dma_v;
  dma_s.init(DK, lane0, w);
  dma_v.init(v_stride, lane0, w);
  // one [C][BV] tile (V or dO) of the block at v0
  auto dma_rows = [&](uint16_t* dst, const uint16_t* src, int v0) {
    const auto* sp_ = static_cast<const uint16_t*>(uniform_ptr(src + row0 * DV + v0));
#pragma unroll
    for (int i = 0; i < S::TV::PER_WAVE; ++i) {
      if (valid == C) dma_v.template issue<false>(i, lds_addr_of(dst), sp_, C);
      else dma_v.template issue<true>(i, lds_addr_of(dst), sp_, valid);
    }
  };
  // the block's S^T, dS'^T and dO (with V: the first block)
  auto dma_block = [&](int v0, bool with_v) {
    const auto* sb = static_cast<const uint16_t*>(uniform_ptr(states + (slot * DV + v0) * DK));
    const auto* db = static_cast<const uint16_t*>(uniform_ptr(dstates + (slot * DV + v0) * DK));
#pragma unroll
    for (int i = 0; i < S::TS::PER_WAVE; ++i) {
      dma_s.template issue<false>(i, lds_addr_of(St), sb, BV);
      dma_s.template issue<false>(i, lds_addr_of(dSt), db, BV);
    }
    dma_rows(dOt, dout, v0);
    if (with_v) dma_rows(Vt, v, v0);
  };
  // an accumulator tile (rows 16 rt + 4 g + qq, column 16 c + li) into a [C][BV] tile
  auto put = [&](uint16_t* X, const f32x4& a, int rt, int c, int li, int g) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) X[swz_off<BV>(16 * rt + 4 * g + qq, 16 * c + li)] = from_f32<uint16_t>(a[qq]);
  };

  f32x4 dQa[NQ], dKa[NQ], dPa[NP], dTa[NP];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dQa[i] = dKa[i] = zero4();
#pragma unroll
  for (int i = 0; i < NP; ++i) dPa[i] = dTa[i] = zero4();

  // the tail's X
  constexpr int UX = C * C / 4;  // 16-byte units of fp32 X
  u32x4 rx[UX / NTH];
  static_assert(UX % NTH == 0, "whole units per thread");

  dma_block(0, true);
  // one value block; the last one (LAST) also requests the tail's X after
  // its first phase, so that the load overlaps the block's other two phases
  // (requested after the block, the tail waited for it; before the first
  // phase, the held registers spilled more)
  auto block = [&](const int v0, auto lastc) {
    constexpr bool LAST = decltype(lastc)::value;
    // the lane indices as values the compiler cannot see to be the same in
    // every block, so that the fragment addresses built from them are formed
    // here rather than held in registers across the loop
    int li = li0, g = g0, lane = lane0, tidv = tid;
    asm volatile("" : "+v"(li), "+v"(g), "+v"(lane), "+v"(tidv));
    wait_vmcnt<0>();  // this wavefront's transfers of the block
    if (valid < C) {
      __syncthreads();  // every wavefront's transfers landed
      for (int i = tidv; i < 2 * (C - valid) * (BV / 8); i += NTH) {
        const int r = valid + (i >> 1) / (BV / 8), ch = (i >> 1) % (BV / 8);
        st16(((i & 1) ? dOt : Vt) + swz_off<BV>(r, 8 * ch), Z);
      }
      if (v0 == 0)
        for (int i = tidv; i < (C - valid) * (DK / 8); i += NTH)
          st16(Kt + swzw_off<DK>(valid + i / (DK / 8), 8 * (i % (DK / 8))), Z);
    }
    __syncthreads();  // the block's operands in place (and the chunk's K, T, P)
    // D = V - K S and dU = P^T dO + K dS': tile (rt, c) of each, wavefront w = 2 rt + c
    {
      const int rt = w >> 1, c = w & 1;
      f32x4 d = zero4(), du = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        const Frag<uint16_t> a = wide_frag<DK>(Kt, 16 * rt + li, ku, g);
        mma(d, a, wide_frag<DK>(St, 16 * c + li, ku, g));
        mma(du, a, wide_frag<DK>(dSt, 16 * c + li, ku, g));
      }
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku + 31 >= 16 * rt) mma(du, sw_frag_tr<C>(Pt, 16 * rt, ku, lane), sw_frag_tr<BV>(dOt, 16 * c, ku, lane));
      const bf16x4 vv = lds_read_tr(Vt + swz_off<BV>(16 * rt + 4 * g + (li >> 2), 16 * c + 4 * (li & 3)));
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) d[qq] = static_cast<float>(vv[qq]) - d[qq];
      put(Dt, d, rt, c, li, g);
      put(dUt, du, rt, c, li, g);
    }
    __syncthreads();
    if (v0 + BV < DV) dma_rows(Vt, v, v0 + BV);  // V is read only in the phase above
    if constexpr (LAST) {
#pragma unroll
      for (int i = 0; i < UX / NTH; ++i) {
        const int u = tidv + NTH * i, r = u / (C / 4), ch = u % (C / 4);
        rx[i] = *reinterpret_cast<const u32x4*>(xws + slot * C * C + r * C + 4 * ch);
      }
    }
    // U = T D and dD = T^T dU (= dV)
    {
      const int rt = w >> 1, c = w & 1;
      f32x4 u = zero4(), dd = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku) {
        if (32 * ku <= 16 * rt + 15) mma(u, sw_frag<C>(Tt, 16 * rt + li, ku, g), sw_frag_tr<BV>(Dt, 16 * c, ku, lane));
        if (32 * ku + 31 >= 16 * rt)
          mma(dd, sw_frag_tr<C>(Tt, 16 * rt, ku, lane), sw_frag_tr<BV>(dUt, 16 * c, ku, lane));
      }
      put(Ut, u, rt, c, li, g);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) dd[qq] = -dd[qq];
      put(dDt, dd, rt, c, li, g);  // as -dD
    }
    __syncthreads();
    // dv = dD of the block from its staged tile, as whole 64-byte row pieces
    // (four lanes a row; bf16 negation is exact): stored from the product
    // tiles, as 32-byte pieces of two wavefronts, each 64-byte line was
    // written in parts
    if (tidv < 4 * C) {
      const int r = tidv >> 2, p = tidv & 3;
      if (r < valid) {
        u32x4 x = *reinterpret_cast<const u32x4*>(dDt + r * BV + 8 * (p ^ swz_row<BV / 8>(r)));
        x ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
        __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(dv + row0 * DV + r * v_stride + v0 + 8 * p));
      }
    }
    if (v0 + BV >= DV) {  // the tail's Q, during the last block (over T and P, done with)
      const auto* qs = static_cast<const uint16_t*>(uniform_ptr(q + row0 * DK));
#pragma unroll
      for (int i = 0; i < S::TK::PER_WAVE; ++i) {
        if (valid == C) dma_k.template issue<false>(i, lds_addr_of(b16(S::QT)), qs, C);
        else dma_k.template issue<true>(i, lds_addr_of(b16(S::QT)), qs, valid);
      }
    }
    // dQ += dO S^T;  dK += U dS'^T - dD S^T  (tiles (rt, dt), logical key columns);
    // dP += dO U^T;  dT += dU D^T  (lower tiles)
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int t = w + NWV * i, rt = t / NDT, dt = t % NDT;
      const Frag<uint16_t> bS = wide_frag_tr<DK>(St, dt, 0, lane);
      mma(dQa[i], sw_frag<BV>(dOt, 16 * rt + li, 0, g), bS);
      mma(dKa[i], sw_frag<BV>(Ut, 16 * rt + li, 0, g), wide_frag_tr<DK>(dSt, dt, 0, lane));
      mma(dKa[i], sw_frag<BV>(dDt, 16 * rt + li, 0, g), bS);

    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = w + NWV * i, rt = t / NRT, jt = t % NRT;
      if (jt <= rt) {
        mma(dPa[i], sw_frag<BV>(dOt, 16 * rt + li, 0, g), sw_frag<BV>(Ut, 16 * jt + li, 0, g));
        mma(dTa[i], sw_frag<BV>(dUt, 16 * rt + li, 0, g), sw_frag<BV>(Dt, 16 * jt + li, 0, g));
      }
    }
    if (v0 + BV < DV) {
      __syncthreads();  // every read of this block's operands done
      dma_block(v0 + BV, false);
    }
  };
  for (int v0 = 0; v0 + BV < DV; v0 += BV) block(v0, std::false_type{});
  block(DV - BV, std::true_type{});
  wait_vmcnt<0>();   // Q's transfers and X
  __syncthreads();  // done with the loop's arrays (K stays); Q in place

  // ---- the UT-transform part -----------------------------------------------
  // Its C x C x C products W = X^T dX and dA = -W X^T run on bf16 matrix cores
  // in three passes over a split of each fp32 operand into bf16 high and low
  // parts (hi hi + hi lo + lo hi: ~16 significant bits, beside the single bf16
  // rounding of the other operands), with every fragment one LDS read.
  const int li = li0, g = g0, lane = lane0;
  uint16_t *Qt = b16(S::QT), *dPt = b16(S::DPT), *dXh = b16(S::DXH), *dXl = b16(S::DXL);
  uint16_t *Wh = b16(S::WH), *Wl = b16(S::WL), *Xh = b16(S::XH), *Xl = b16(S::XL), *Eb = b16(S::EB);
  uint16_t *dQs = b16(S::DQS), *dKs = b16(S::DKS);
  float *A0 = f32p(S::A0), *dAf = f32p(S::DAF), *red = f32p(S::RED);
  constexpr int CPG = S::CPG;
  constexpr int NPART = NTH / C, RPP = C / NPART;
  const int cr = tid % C, prt = tid / C;
  auto split = [](float x, uint16_t& hi, uint16_t& lo) {
    hi = from_f32<uint16_t>(x);
    lo = from_f32<uint16_t>(x - to_f32(hi));
  };
  // three-pass product acc += A B over one 32-deep slice
  auto mma3 = [](f32x4& acc, const Frag<uint16_t>& ah, const Frag<uint16_t>& al, const Frag<uint16_t>& bh,
                 const Frag<uint16_t>& bl) {
    mma(acc, ah, bh);
    mma(acc, ah, bl);
    mma(acc, al, bh);
  };
  // dP (lower, diagonal included) as bf16, dT (lower) fp32; Q; X as high and low parts
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + NWV * i, rt = t / NRT, jt = t % NRT;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 16 * rt + 4 * g + qq, c = 16 * jt + li;
      dPt[swz_off<C>(r, c)] = from_f32<uint16_t>(c <= r ? dPa[i][qq] : 0.0f);
      A0[r * CPF + c] = c <= r ? dTa[i][qq] : 0.0f;
    }
  }
  for (int i = tid; i < (C - valid) * (DK / 8); i += NTH)  // Q's rows past the end re-read row 0
    st16(Qt + swzw_off<DK>(valid + i / (DK / 8), 8 * (i % (DK / 8))), Z);
#pragma unroll
  for (int i = 0; i < UX / NTH; ++i) {
    const int u = tid + NTH * i, r = u / (C / 4), ch = u % (C / 4);
    union {
      u32x4 u;
      float f[4];
    } x;
    x.u = rx[i];
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) split(x.f[e], hi[e], lo[e]);
    *reinterpret_cast<uint2*>(Xh + swz_off<C>(r, 4 * ch)) = *reinterpret_cast<const uint2*>(hi);
    *reinterpret_cast<uint2*>(Xl + swz_off<C>(r, 4 * ch)) = *reinterpret_cast<const uint2*>(lo);
  }
  __syncthreads();
  // dQ += dP K;  dK += dP^T Q;  da_j = sum_i dT_ij X_ij (partial sums)
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int t = w + NWV * i, rt = t / NDT, dt = t % NDT;
#pragma unroll
    for (int ku = 0; ku < NKU_C; ++ku) {
      if (32 * ku <= 16 * rt + 15)
        mma(dQa[i], sw_frag<C>(dPt, 16 * rt + li, ku, g), wide_frag_tr<DK>(Kt, dt, ku, lane));
      if (32 * ku + 31 >= 16 * rt)
        mma(dKa[i], sw_frag_tr<C>(dPt, 16 * rt, ku, lane), wide_frag_tr<DK>(Qt, dt, ku, lane));
    }
  }
  {
    float s = 0.0f;
#pragma unroll
    for (int r = prt * RPP; r < (prt + 1) * RPP; ++r)
      s = fmaf(A0[r * CPF + cr], to_f32(Xh[swz_off<C>(r, cr)]) + to_f32(Xl[swz_off<C>(r, cr)]), s);
    red[prt * C + cr] = s;
  }
  __syncthreads();
  // dX = dT diag(a), as high and low parts (over Q)
  if (tid < C) {
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < NPART; ++p) s += red[p * C + tid];
    das[tid] = s;
  }
  for (int i = tid; i < C * C; i += NTH) {
    const int r = i / C, c = i % C;
    uint16_t hi, lo;
    split(A0[r * CPF + c] * as[c], hi, lo);
    dXh[swz_off<C>(r, c)] = hi;
    dXl[swz_off<C>(r, c)] = lo;
  }
  __syncthreads();
  // W = X^T dX, as high and low parts (over dT)
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + NWV * i, rt = t / NRT, jt = t % NRT;
    f32x4 acc = zero4();
#pragma unroll
    for (int ku = 0; ku < NKU_C; ++ku)
      if (32 * ku + 31 >= 16 * rt && 32 * ku + 31 >= 16 * jt)  // X and dT are lower triangular
        mma3(acc, sw_frag_tr<C>(Xh, 16 * rt, ku, lane), sw_frag_tr<C>(Xl, 16 * rt, ku, lane),
             sw_frag_tr<C>(dXh, 16 * jt, ku, lane), sw_frag_tr<C>(dXl, 16 * jt, ku, lane));
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 16 * rt + 4 * g + qq, c = 16 * jt + li;
      uint16_t hi, lo;
      split(acc[qq], hi, lo);
      Wh[swz_off<C>(r, c)] = hi;
      Wl[swz_off<C>(r, c)] = lo;
    }
  }
  __syncthreads();
  // dA = -W X^T (strictly lower, fp32, over dX);  G = K K^T on the lower tiles:
  // lambda (its diagonal) and the row sums of dA G, tile column by tile column
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + NWV * i, rt = t / NRT, jt = t % NRT;
    f32x4 acc = zero4(), gg = zero4();
    if (jt <= rt) {
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku <= 16 * jt + 15)  // X^T's rows of this tile are zero past column 16 jt + 15
          mma3(acc, sw_frag<C>(Wh, 16 * rt + li, ku, g), sw_frag<C>(Wl, 16 * rt + li, ku, g),
               sw_frag<C>(Xh, 16 * jt + li, ku, g), sw_frag<C>(Xl, 16 * jt + li, ku, g));
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku)
        mma(gg, wide_frag<DK>(Kt, 16 * rt + li, ku, g), wide_frag<DK>(Kt, 16 * jt + li, ku, g));
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 16 * rt + 4 * g + qq, c = 16 * jt + li;
      const float da = c < r ? -acc[qq] : 0.0f;
      dAf[r * CPF + c] = da;
      if (c == r) lam[r] = gg[qq];
      float s = da * gg[qq];
      // over the 16 columns of the tile: rotations within each 16-lane row
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x121, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x122, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x124, 0xF, 0xF, false));
      s += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s), 0x128, 0xF, 0xF, false));
      if (li == 0) red[jt * C + r] = s;
    }
  }
  __syncthreads();
  // da_i += sum_{j<i} dA_ij G_ij, then dbeta and dlambda;  dG + dG^T with
  // dG = diag(a) dA, as bf16 (over X)
  if (tid < C) {
    float s = das[tid];
#pragma unroll
    for (int jt = 0; jt < NRT; ++jt) s += red[jt * C + tid];
    float dl = 0.0f;
    if (tid < valid) {
      const float bt = to_f32(beta[row0 + int64_t(tid) * H]);
      float da_db, da_dl;
      efla_alpha_grad(bt, lam[tid], rule, da_db, da_dl);
      dl = s * da_dl;
      dbeta[row0 + int64_t(tid) * H] = from_f32<uint16_t>(s * da_db);
    }
    dls[tid] = dl;
  }
  for (int i = tid; i < C * C; i += NTH) {
    const int r = i / C, c = i % C;
    Eb[swz_off<C>(r, c)] = from_f32<uint16_t>(as[r] * dAf[r * CPF + c] + as[c] * dAf[c * CPF + r]);
  }
  __syncthreads();
  // dK += (dG + dG^T) K + 2 diag(dlambda) K;  dQ and dK staged as bf16 rows
  // (physical key columns) over W and dA
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int t = w + NWV * i, rt = t / NDT, dt = t % NDT;
#pragma unroll
    for (int ku = 0; ku < NKU_C; ++ku)
      mma(dKa[i], sw_frag<C>(Eb, 16 * rt + li, ku, g), wide_frag_tr<DK>(Kt, dt, ku, lane));
    const int cp = key_phys(16 * dt + li);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = 16 * rt + 4 * g + qq;
      const float kv = to_f32(Kt[swzw_off<DK>(r, cp)]);
      dQs[r * CPG + cp] = from_f32<uint16_t>(dQa[i][qq]);
      dKs[r * CPG + cp] = from_f32<uint16_t>(dKa[i][qq] + 2.0f * dls[r] * kv);
    }
  }
  __syncthreads();
  // dq, dk: 16-byte row pieces
  const int64_t qk_row = row0 * DK;
#pragma unroll
  for (int i = 0; i < UK / NTH; ++i) {
    const int u = tid + NTH * i, r = u / (DK / 8), ch = u % (DK / 8);
    if (r < valid) {
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(dQs + r * CPG + 8 * ch),
                                  reinterpret_cast<u32x4*>(dq + qk_row + r * qk_stride + 8 * ch));
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(dKs + r * CPG + 8 * ch),
                                  reinterpret_cast<u32x4*>(dk + qk_row + r * qk_stride + 8 * ch));
    }
  }
}

}  // namespace efla
