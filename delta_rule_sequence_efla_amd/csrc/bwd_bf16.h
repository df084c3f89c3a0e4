// bwd_bf16.h -- the per-chunk gradients of the backward pass for bf16 inputs,
// with the value-block products on bf16 matrix cores.
//
// Same formulas and work split as bwd_chunk_kernel (bwd_kernels.h): one
// workgroup per (b, h, chunk), value columns streamed in blocks, dQ, dK, dP and
// dT accumulated in fp32 registers, then the UT-transform part.  What differs
// is where the products run: every product with a value block, Q or K is one
// v_mfma_f32_16x16x32_bf16 per 32-deep slice on bf16 operands in LDS.  The
// operands that are not bf16 already (P, the intermediates D = V - K S,
// dU, U, dD, and dP, dG + dG^T) are rounded to bf16 once, like the states the
// forward products use; X, W = X^T dX, dA and the coefficient gradients stay
// fp32 (fp32 matrix cores and VALU).
//
// Every product is written acc += A B with A read as rows of an [M][K] array
// and B as rows of an [N][K] array (B's transpose), so each operand fragment is
// one 16-byte LDS read (lane (li, g) takes k = 32 ku + 8 g .. +7).  Arrays that
// serve as B with the other orientation too are kept in both layouts:
//     D = V - K S          A = K [C][DK]      B^T = S^T [BV][DK]
//     dU = P^T dO + K dS'  A = P^T, K         B^T = dO^T [BV][C], dS'^T [BV][DK]
//     U = T D              A = T              B^T = D^T [BV][C]
//     dD = T^T dU          A = T^T            B^T = dU^T [BV][C]
//     dQ += dO S^T         A = dO [C][BV]     B^T = S [DK][BV]
//     dK += U dS'^T - dD S^T, dP += dO U^T, dT += dU D^T  (likewise, K = BV)
#pragma once

#include "bwd_kernels.h"

namespace efla {

constexpr int kBwdBV = 32;  // value columns per block

template <int DK, int C>
struct BwdBf16Shape {
  static constexpr int BV = kBwdBV;
  static constexpr int KBP = DK + 8;   // pitch (elements) of [*][DK] arrays
  static constexpr int TBP = C + 8;    // pitch of [*][C] arrays
  static constexpr int VBP = BV + 8;   // pitch of [*][BV] arrays
  // byte offsets of the loop-phase arrays (all bf16, 16-byte aligned)
  static constexpr int KB = 0;
  static constexpr int TB = KB + C * KBP * 2;
  static constexpr int TBT = TB + C * TBP * 2;
  static constexpr int PBT = TBT + C * TBP * 2;
  static constexpr int SV = PBT + C * TBP * 2;
  static constexpr int DSV = SV + DK * VBP * 2;
  static constexpr int SVT = DSV + DK * VBP * 2;
  static constexpr int DSVT = SVT + BV * KBP * 2;
  static constexpr int DOV = DSVT + BV * KBP * 2;
  static constexpr int VV = DOV + C * VBP * 2;
  static constexpr int DV_ = VV + C * VBP * 2;
  static constexpr int DUV = DV_ + C * VBP * 2;
  static constexpr int UV = DUV + C * VBP * 2;
  static constexpr int DDV = UV + C * VBP * 2;
  static constexpr int DOVT = DDV + C * VBP * 2;
  static constexpr int DVT = DOVT + BV * TBP * 2;
  static constexpr int DUVT = DVT + BV * TBP * 2;
  static constexpr int LOOP_BYTES = DUVT + BV * TBP * 2;
  // the tail's arrays (K stays where the loop had it): fp32 [C][CPP] for dT
  // (then dX, then G), X, W and dA; bf16 K^T, Q^T [DK][TBP] and dP, dP^T,
  // dG + dG^T [C][TBP]
  static constexpr int CPP = C + 4;
  static constexpr int TA0 = TB;
  static constexpr int TX = TA0 + C * CPP * 4;
  static constexpr int TW = TX + C * CPP * 4;
  static constexpr int TDA = TW + C * CPP * 4;
  static constexpr int TKBT = TDA + C * CPP * 4;
  static constexpr int TQBT = TKBT + DK * TBP * 2;
  static constexpr int TDPB = TQBT + DK * TBP * 2;
  static constexpr int TDPBT = TDPB + C * TBP * 2;
  static constexpr int TEB = TDPBT + C * TBP * 2;
  // sixteen, eight or four wavefronts: the most over which every tile loop
  // splits evenly
  static constexpr bool splits(int n) {
    return (C / 16) * (DK / 16) % n == 0 && (C / 16) * (C / 16) % n == 0 && 2 * (C / 16) * (BV / 16) % n == 0;
  }
  static constexpr int NWV = splits(16) ? 16 : splits(8) ? 8 : 4;
  static constexpr int NTH = NWV * kWave;
  static constexpr int NQ = (C / 16) * (DK / 16) / NWV;  // dQ / dK tiles per wavefront
  static constexpr int NP = (C / 16) * (C / 16) / NWV;   // dP / dT tiles per wavefront
  static constexpr int TRED = TEB + C * TBP * 2;  // fp32 partial sums, one per thread
  static constexpr int TAIL_BYTES = TRED + NTH * 4;
  static constexpr int BYTES = LOOP_BYTES > TAIL_BYTES ? LOOP_BYTES : TAIL_BYTES;
};

inline bool bwd_bf16_supported(int DK, int DV, int C) {
  return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64) && DV % kBwdBV == 0;
}

// One 16-byte operand fragment: row `row` of an [*][K] bf16 array, k-slice ku.
__device__ __forceinline__ Frag<uint16_t> row8(const uint16_t* X, int pitch, int row, int ku, int g) {
  Frag<uint16_t> f;
  f.v = *reinterpret_cast<const bf16x8*>(X + row * pitch + 32 * ku + 8 * g);
  return f;
}

// acc (16x16 tile, rows r0.., columns c0..) += A B over k < K (K % 32 == 0):
// A rows from A [M][K], B columns from Bt [N][K].
template <int K>
__device__ __forceinline__ void tile_bf(f32x4& acc, const uint16_t* A, int lda, const uint16_t* Bt, int ldb, int r0,
                                        int c0, int li, int g) {
#pragma unroll
  for (int ku = 0; ku < K / 32; ++ku) mma(acc, row8(A, lda, r0 + li, ku, g), row8(Bt, ldb, c0 + li, ku, g));
}

// An accumulator tile (rows r0 + 4 g + q, column c0 + li) stored as bf16 into
// X [rows][pitch] (four 2-byte writes) and, if XT, into XT [cols][pitchT]
// (one 8-byte write: the four rows are consecutive there).
__device__ __forceinline__ void put_tile(uint16_t* X, int pitch, uint16_t* XT, int pitchT, const f32x4& a, int r0,
                                         int c0, int li, int g) {
#pragma unroll
  for (int q = 0; q < 4; ++q) X[(r0 + 4 * g + q) * pitch + c0 + li] = from_f32<uint16_t>(a[q]);
  if (XT != nullptr) st4(XT + (c0 + li) * pitchT + r0 + 4 * g, a);
}

// A ROWS x COLS tile of a bf16 or fp32 array in global memory or LDS (rows `stride`
// elements apart, rows at or past `valid` read as zero), staged through
// registers into bf16 LDS: load() issues 16-byte loads, store() writes the
// tile as rows (dst [ROWS][pitch]) and, if dstT, as its transpose
// (dstT [COLS][pitchT], pitchT even).  Each thread takes two consecutive rows
// of one 16-byte column slice, and consecutive threads consecutive row pairs:
// a transposed store then writes both rows' halfwords of one column as one
// 4-byte word, and a wavefront's such stores land on consecutive words
// (conflict-free).
template <typename S, int ROWS, int COLS, int NTH = kThreads>  // NTH: threads of the workgroup
struct Bf16Stager {
  static constexpr int VN = 16 / int(sizeof(S)), RP = ROWS / 2, TOT = RP * (COLS / VN), CNT = cdiv(TOT, NTH);
  static_assert(COLS % VN == 0 && ROWS % 2 == 0, "whole 16-byte vectors per row, row pairs");
  u32x4 r[CNT][2];
  __device__ __forceinline__ void load(const S* src, int64_t stride, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      const int t = 2 * (idx % RP), c = (idx / RP) * VN;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        r[i][h] = u32x4{0u, 0u, 0u, 0u};
        if (idx < TOT && t + h < valid) r[i][h] = *reinterpret_cast<const u32x4*>(src + (t + h) * stride + c);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int pitch, uint16_t* dstT, int pitchT, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      if (idx >= TOT) continue;
      const int t = 2 * (idx % RP), c = (idx / RP) * VN;
      uint16_t hv[2][VN];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        union {
          u32x4 u;
          S e[VN];
        } x;
        x.u = r[i][h];
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          if constexpr (sizeof(S) == 2) hv[h][e] = x.e[e];
          else hv[h][e] = from_f32<uint16_t>(x.e[e]);
        }
        if (dst != nullptr) {
          if constexpr (VN == 8) {
            *reinterpret_cast<u32x4*>(dst + (t + h) * pitch + c) = *reinterpret_cast<const u32x4*>(hv[h]);
          } else {
            *reinterpret_cast<uint2*>(dst + (t + h) * pitch + c) = *reinterpret_cast<const uint2*>(hv[h]);
          }
        }
      }
      if (dstT != nullptr) {
#pragma unroll
        for (int e = 0; e < VN; ++e)
          *reinterpret_cast<uint32_t*>(dstT + (c + e) * pitchT + t) = uint32_t(hv[0][e]) | (uint32_t(hv[1][e]) << 16);
      }
    }
  }
};

// One value block's four operands staged through one set of registers: S and
// dS' (bf16 [DK][BV]), V and dO (bf16 [C][BV]), their 16-byte units numbered
// in that order and dealt to the workgroup's threads, so a thread holds
// cdiv(units, NTH) row pairs instead of one per operand (with 32 value
// columns every operand boundary falls on a whole wavefront).
// Each unit is two consecutive rows of one 16-byte column slice, written as
// in Bf16Stager: rows, and transposed as 4-byte words of the two rows.  STT:
// S comes transposed (rows of d_k per value column), so its rows land in
// S^T and its transpose in S; DSTT likewise for dS'.
template <int DK, int C, int BV, int NTH, bool STT, bool DSTT>
struct BlockStager {
  static constexpr int U0 = (DK / 2) * (BV / 8), U1 = U0, U2 = (C / 2) * (BV / 8);
  static constexpr int TOT = U0 + U1 + 2 * U2, CNT = cdiv(TOT, NTH);
  u32x4 r[CNT][2];
  // operand of unit idx, and its index within that operand
  __device__ __forceinline__ static int which(int idx, int& j) {
    if (idx < U0) { j = idx; return 0; }
    if (idx < U0 + U1) { j = idx - U0; return 1; }
    if (idx < U0 + U1 + U2) { j = idx - U0 - U1; return 2; }
    j = idx - U0 - U1 - U2;
    return 3;
  }
  __device__ __forceinline__ void load(const uint16_t* st, const uint16_t* dst, const uint16_t* vv,
                                       const uint16_t* dov, int DV, int64_t v_stride, int valid, int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      r[i][0] = r[i][1] = u32x4{0u, 0u, 0u, 0u};
      if (idx >= TOT) continue;
      int j;
      const int op = which(idx, j);
      if ((op == 0 && STT) || (op == 1 && DSTT)) {  // S^T or dS'^T rows: BV rows, stride DK
        const int t = 2 * (j % (BV / 2)), c = (j / (BV / 2)) * 8;
        const uint16_t* src = op == 0 ? st : dst;
#pragma unroll
        for (int h = 0; h < 2; ++h) r[i][h] = *reinterpret_cast<const u32x4*>(src + (t + h) * DK + c);
      } else if (op <= 1) {  // S or dS' rows: DK rows, stride DV
        const int t = 2 * (j % (DK / 2)), c = (j / (DK / 2)) * 8;
        const uint16_t* src = op == 0 ? st : dst;
#pragma unroll
        for (int h = 0; h < 2; ++h) r[i][h] = *reinterpret_cast<const u32x4*>(src + (t + h) * int64_t(DV) + c);
      } else {  // V or dO: C token rows, rows at or past `valid` read as zero
        const uint16_t* src = op == 2 ? vv : dov;
        const int t = 2 * (j % (C / 2)), c = (j / (C / 2)) * 8;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          if (t + h < valid) r[i][h] = *reinterpret_cast<const u32x4*>(src + (t + h) * v_stride + c);
      }
    }
  }
  // Sv [DK][VBP] + SvT [BV][KBP]; dSv + dSvT likewise; Vv [C][VBP]; dOv [C][VBP] + dOvT [BV][TBP]
  __device__ __forceinline__ void store(uint16_t* Sv, uint16_t* SvT, uint16_t* dSv, uint16_t* dSvT, uint16_t* Vv,
                                        uint16_t* dOv, uint16_t* dOvT, int VBP, int KBP, int TBP, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      if (idx >= TOT) continue;
      int j;
      const int op = which(idx, j);
      {  // eight bf16 columns
        const bool tr = (STT && op == 0) || (DSTT && op == 1);
        const int rows = tr ? BV : op <= 1 ? DK : C;
        const int t = 2 * (j % (rows / 2)), c = (j / (rows / 2)) * 8;
        uint16_t* X = tr ? (op == 0 ? SvT : dSvT) : op == 0 ? Sv : op == 1 ? dSv : op == 2 ? Vv : dOv;
        uint16_t* XT = tr ? (op == 0 ? Sv : dSv) : op == 0 ? SvT : op == 1 ? dSvT : op == 2 ? nullptr : dOvT;
        const int pitch = tr ? KBP : VBP;
        const int pitchT = tr ? VBP : op <= 1 ? KBP : TBP;
#pragma unroll
        for (int h = 0; h < 2; ++h) *reinterpret_cast<u32x4*>(X + (t + h) * pitch + c) = r[i][h];
        if (XT != nullptr) {
          union {
            u32x4 u;
            uint16_t e[8];
          } x0, x1;
          x0.u = r[i][0];
          x1.u = r[i][1];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            *reinterpret_cast<uint32_t*>(XT + (c + e) * pitchT + t) = uint32_t(x0.e[e]) | (uint32_t(x1.e[e]) << 16);
        }
      }
    }
  }
};

// STT: `states` holds each chunk's start state transposed, [slots][DV][DK]
// (else [slots][DK][DV]); DSTT: `dstates` likewise.
template <int DK, int C, bool STT, bool DSTT>
__global__ __launch_bounds__((BwdBf16Shape<DK, C>::NTH)) void bwd_chunk_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ beta, const uint16_t* __restrict__ dout, const uint16_t* __restrict__ tws,
    const float* __restrict__ xws, const float* __restrict__ aws, const uint16_t* __restrict__ pws,
    const uint16_t* __restrict__ states, const uint16_t* __restrict__ dstates, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, uint16_t* __restrict__ dbeta, int H, int64_t L, int NC,
    int DV, int rule) {
  using S = BwdBf16Shape<DK, C>;
  using F = BwdChunkShape<uint16_t, DK, C>;
  constexpr int KBP = S::KBP, TBP = S::TBP, VBP = S::VBP, BV = S::BV;
  constexpr int NQ = S::NQ, NP = S::NP, NCQ = DK / 16, NCP = C / 16, NRT = C / 16;
  constexpr int NWV = S::NWV, NTH = S::NTH;
  static_assert(F::CP == C && F::DKP == DK, "bf16 kernel: DK and C are multiples of 32");
  __shared__ __align__(16) unsigned char lds[S::BYTES];
  __shared__ float as[C], das[C], dls[C];
  auto arr = [&](int off) { return reinterpret_cast<uint16_t*>(lds + off); };
  uint16_t *Kb = arr(S::KB), *Tb = arr(S::TB), *TbT = arr(S::TBT), *PbT = arr(S::PBT);
  uint16_t *Sv = arr(S::SV), *dSv = arr(S::DSV), *SvT = arr(S::SVT), *dSvT = arr(S::DSVT);
  uint16_t *dOv = arr(S::DOV), *Vv = arr(S::VV), *Dv = arr(S::DV_), *dUv = arr(S::DUV), *Uv = arr(S::UV);
  uint16_t *dDv = arr(S::DDV), *dOvT = arr(S::DOVT), *DvT = arr(S::DVT), *dUvT = arr(S::DUVT);

  const int64_t slot = blockIdx.x;
  const int n = int(slot % NC);
  const int64_t bh = slot / NC, h = bh % H;
  const SeqSpan sp = seq_span<C>(nullptr, int(bh / H), h, H, L, NC);
  const int64_t t0 = int64_t(n) * C;
  const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
  const int64_t row0 = (sp.bos + t0) * H + h;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;

  // chunk operands: K, T, T^T, P^T as bf16 for the loop (the tail loads Q
  // and transposes K from these rows)
  {
    Bf16Stager<uint16_t, C, DK, NTH> sk;
    sk.load(k + row0 * DK, qk_stride, valid, tid);
    Bf16Stager<uint16_t, C, C, NTH> st;
    Bf16Stager<uint16_t, C, C, NTH> spp;
    st.load(tws + slot * C * C, C, C, tid);
    spp.load(pws + slot * C * C, C, C, tid);
    sk.store(Kb, KBP, nullptr, 0, tid);
    st.store(Tb, TBP, TbT, TBP, tid);
    spp.store(nullptr, 0, PbT, TBP, tid);
  }
  if (tid < C) as[tid] = aws[slot * C + tid];

  f32x4 dQa[NQ], dKa[NQ], dPa[NP], dTa[NP];
#pragma unroll
  for (int i = 0; i < NQ; ++i) dQa[i] = dKa[i] = zero4();
#pragma unroll
  for (int i = 0; i < NP; ++i) dPa[i] = dTa[i] = zero4();

  const uint16_t* st = states + slot * DK * DV;
  const uint16_t* dst = dstates + slot * DK * DV;
  // one value block's operands, staged through registers one block ahead
  BlockStager<DK, C, BV, NTH, STT, DSTT> sb;
  auto load_block = [&](int v0) {
    sb.load(st + (STT ? v0 * DK : v0), dst + (DSTT ? v0 * DK : v0), v + row0 * DV + v0, dout + row0 * DV + v0, DV, v_stride, valid,
            tid);
  };
  load_block(0);
  for (int v0 = 0; v0 < DV; v0 += BV) {
    __syncthreads();  // the previous block's buffers are free (and the chunk operands are in place)
    sb.store(Sv, SvT, dSv, dSvT, Vv, dOv, dOvT, VBP, KBP, TBP, tid);
    if (v0 + BV < DV) load_block(v0 + BV);  // in flight during this block
    __syncthreads();
    // D = V - K S,  dU = P^T dO + K dS'   (tiles of [C][BV])
    for (int t = w; t < 2 * NRT * (BV / 16); t += NWV) {
      const int tt = t % (NRT * (BV / 16)), r0 = 16 * (tt / (BV / 16)), c0 = 16 * (tt % (BV / 16));
      f32x4 acc = zero4();
      if (t < NRT * (BV / 16)) {
        tile_bf<DK>(acc, Kb, KBP, SvT, KBP, r0, c0, li, g);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) acc[qq] = to_f32(Vv[(r0 + 4 * g + qq) * VBP + c0 + li]) - acc[qq];
        put_tile(Dv, VBP, DvT, TBP, acc, r0, c0, li, g);
      } else {
        tile_bf<C>(acc, PbT, TBP, dOvT, TBP, r0, c0, li, g);
        tile_bf<DK>(acc, Kb, KBP, dSvT, KBP, r0, c0, li, g);
        put_tile(dUv, VBP, dUvT, TBP, acc, r0, c0, li, g);
      }
    }
    __syncthreads();
    // U = T D,  dD = T^T dU (= dV)
    for (int t = w; t < 2 * NRT * (BV / 16); t += NWV) {
      const int tt = t % (NRT * (BV / 16)), r0 = 16 * (tt / (BV / 16)), c0 = 16 * (tt % (BV / 16));
      f32x4 acc = zero4();
      if (t < NRT * (BV / 16)) {
        tile_bf<C>(acc, Tb, TBP, DvT, TBP, r0, c0, li, g);
        put_tile(Uv, VBP, nullptr, 0, acc, r0, c0, li, g);
      } else {
        tile_bf<C>(acc, TbT, TBP, dUvT, TBP, r0, c0, li, g);
        put_tile(dDv, VBP, nullptr, 0, acc, r0, c0, li, g);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int r = r0 + 4 * g + qq;
          if (r < valid)
            __builtin_nontemporal_store(from_f32<uint16_t>(acc[qq]), dv + row0 * DV + r * v_stride + v0 + c0 + li);
        }
      }
    }
    __syncthreads();
    // dQ += dO S^T;  dK += U dS'^T - dD S^T;  dP += dO U^T;  dT += dU D^T   (K = BV)
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int t = w + NWV * i, r0 = 16 * (t / NCQ), c0 = 16 * (t % NCQ);
      tile_bf<BV>(dQa[i], dOv, VBP, Sv, VBP, r0, c0, li, g);
      tile_bf<BV>(dKa[i], Uv, VBP, dSv, VBP, r0, c0, li, g);
      f32x4 m = zero4();
      tile_bf<BV>(m, dDv, VBP, Sv, VBP, r0, c0, li, g);
      dKa[i] -= m;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int t = w + NWV * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
      tile_bf<BV>(dPa[i], dOv, VBP, Uv, VBP, r0, c0, li, g);
      tile_bf<BV>(dTa[i], dUv, VBP, Dv, VBP, r0, c0, li, g);
    }
  }
  __syncthreads();  // done with the loop's arrays (K stays): the tail's arrays take their place

  // The UT-transform part of the gradient:
  //   dQ += dP K;  dK += dP^T Q;  dX = dT diag(a);  da_j = sum_i dT_ij X_ij;
  //   W = X^T dX;  dA = -W X^T (strictly lower);  da_i += sum_{j<i} dA_ij G_ij;
  //   dG = diag(a) dA;  dbeta, dlambda;  dK += (dG + dG^T) K + 2 diag(dlambda) K.
  // The products with K and Q run on bf16 matrix cores (dP and dG + dG^T
  // rounded once); X, W, dA, G and the coefficient gradients stay fp32.
  constexpr int CPP = S::CPP;
  auto f32 = [&](int off) { return reinterpret_cast<float*>(lds + off); };
  float *A0 = f32(S::TA0), *X = f32(S::TX), *Wm = f32(S::TW), *dA = f32(S::TDA);
  uint16_t *KbT = arr(S::TKBT), *QbT = arr(S::TQBT), *dPb = arr(S::TDPB), *dPbT = arr(S::TDPBT), *Eb = arr(S::TEB);
  float* red = f32(S::TRED);
  // the sums over one index of a C x C product run on every thread: part
  // `prt` of column / row `cr` covers indices prt * RPP .. +RPP
  constexpr int NPART = NTH / C, RPP = C / NPART;
  const int cr = tid % C, prt = tid / C;
  const int64_t qk_row = row0 * DK;
  // dP (lower, diagonal included) as bf16 rows and transposed; dT (lower) -> A0; X; K^T, Q^T
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + NWV * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
    f32x4 p;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 4 * g + qq, c = c0 + li;
      p[qq] = c <= r ? dPa[i][qq] : 0.0f;
      A0[r * CPP + c] = c <= r ? dTa[i][qq] : 0.0f;
    }
    put_tile(dPb, TBP, dPbT, TBP, p, r0, c0, li, g);
  }
  {
    // X and Q from global memory (their latencies overlap); K^T from K's rows,
    // which stay in LDS
    F32Stager<float, C, C, NTH> sx;
    Bf16Stager<uint16_t, C, DK, NTH> sq, sk;
    sx.load(xws + slot * C * C, C, C, tid);
    sq.load(q + row0 * DK, qk_stride, valid, tid);
    sk.load(Kb, KBP, C, tid);
    sk.store(nullptr, 0, KbT, TBP, tid);
    sx.store(X, CPP, tid);
    sq.store(nullptr, 0, QbT, TBP, tid);
  }
  __syncthreads();
  // dQ += dP K;  dK += dP^T Q;  da_j = sum_i dT_ij X_ij
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int t = w + NWV * i, r0 = 16 * (t / NCQ), c0 = 16 * (t % NCQ);
    tile_bf<C>(dQa[i], dPb, TBP, KbT, TBP, r0, c0, li, g);
    tile_bf<C>(dKa[i], dPbT, TBP, QbT, TBP, r0, c0, li, g);
  }
  {
    float s = 0.0f;
#pragma unroll
    for (int r = prt * RPP; r < (prt + 1) * RPP; ++r) s = fmaf(A0[r * CPP + cr], X[r * CPP + cr], s);
    red[prt * C + cr] = s;
  }
  __syncthreads();
  if (tid < C) {
    float s = 0.0f;
#pragma unroll
    for (int p = 0; p < NPART; ++p) s += red[p * C + tid];
    das[tid] = s;
  }
  // dX = dT diag(a), in place
  for (int i = tid; i < C * C; i += NTH) {
    const int r = i / C, c = i % C;
    A0[r * CPP + c] *= as[c];
  }
  __syncthreads();
  // W = X^T dX
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + NWV * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
    f32x4 acc = zero4();
    tile_mma16<true, false>(acc, X, CPP, A0, CPP, r0, c0, C, li, g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) Wm[(r0 + 4 * g + qq) * CPP + c0 + li] = acc[qq];
  }
  __syncthreads();
  // dA = -W X^T (strictly lower);  G = K K^T -> A0
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int t = w + NWV * i, r0 = 16 * (t / NCP), c0 = 16 * (t % NCP);
    f32x4 acc = zero4(), gg = zero4();
    tile_mma16<false, true>(acc, Wm, CPP, X, CPP, r0, c0, C, li, g);
    tile_bf<DK>(gg, Kb, KBP, Kb, KBP, r0, c0, li, g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 4 * g + qq, c = c0 + li;
      dA[r * CPP + c] = c < r ? -acc[qq] : 0.0f;
      A0[r * CPP + c] = gg[qq];
    }
  }
  __syncthreads();
  // da_i += sum_{j<i} dA_ij G_ij;  dG + dG^T with dG = diag(a) dA, as bf16
  {
    float s = 0.0f;  // dA is zero on and above the diagonal
#pragma unroll
    for (int c = prt * RPP; c < (prt + 1) * RPP; ++c) s = fmaf(dA[cr * CPP + c], A0[cr * CPP + c], s);
    red[prt * C + cr] = s;
  }
  for (int i = tid; i < C * C; i += NTH) {
    const int r = i / C, c = i % C;
    Eb[r * TBP + c] = from_f32<uint16_t>(as[r] * dA[r * CPP + c] + as[c] * dA[c * CPP + r]);
  }
  __syncthreads();
  // dbeta, dlambda (lambda = G's diagonal)
  if (tid < C) {
#pragma unroll
    for (int p = 0; p < NPART; ++p) das[tid] += red[p * C + tid];
    float dl = 0.0f;
    if (tid < valid) {
      const float bt = to_f32(beta[row0 + int64_t(tid) * H]);
      float da_db, da_dl;
      efla_alpha_grad(bt, A0[tid * CPP + tid], rule, da_db, da_dl);
      dl = das[tid] * da_dl;
      dbeta[row0 + int64_t(tid) * H] = from_f32<uint16_t>(das[tid] * da_db);
    }
    dls[tid] = dl;
  }
  __syncthreads();
  // dK += (dG + dG^T) K + 2 diag(dlambda) K;  write dq, dk
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int t = w + NWV * i, r0 = 16 * (t / NCQ), c0 = 16 * (t % NCQ);
    tile_bf<C>(dKa[i], Eb, TBP, KbT, TBP, r0, c0, li, g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int r = r0 + 4 * g + qq, c = c0 + li;
      if (r < valid) {
        __builtin_nontemporal_store(from_f32<uint16_t>(dQa[i][qq]), dq + qk_row + r * qk_stride + c);
        __builtin_nontemporal_store(from_f32<uint16_t>(dKa[i][qq] + 2.0f * dls[r] * to_f32(Kb[r * KBP + c])),
                                    dk + qk_row + r * qk_stride + c);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The reverse sequential pass for bf16 inputs: one workgroup per (b, h, 32
// value columns), for chunk n = last .. 0:
//     dstates[n] = dS;   E = P^T dO + K dS;   F = T^T E;   dS += Q^T dO - K^T F
// as in bwd_state_kernel, with dS (d_k x 32) in fp32 registers (its 16x16
// tiles spread over the workgroup's wavefronts) and every
// product on bf16 matrix cores:
// dS, E and F enter the products as bf16 copies (dS^T, E^T, F^T in LDS), Q, K,
// T and P as bf16 in the layouts the products read (K rows; K^T, Q^T, T^T,
// P^T, dO^T).  The next chunk's operands are loaded while this one computes.
// ---------------------------------------------------------------------------
template <int DK, int C>
struct BwdStateBf16Shape {
  static constexpr int BV = kBwdBV;
  static constexpr int KBP = DK + 8, TBP = C + 8;
  static constexpr int KB = 0;                          // K      [C][KBP]
  static constexpr int KBT = KB + C * KBP * 2;          // K^T    [DK][TBP]
  static constexpr int QBT = KBT + DK * TBP * 2;        // Q^T    [DK][TBP]
  static constexpr int TBT = QBT + DK * TBP * 2;        // T^T    [C][TBP]
  static constexpr int PBT = TBT + C * TBP * 2;         // P^T    [C][TBP]
  static constexpr int DOT = PBT + C * TBP * 2;         // dO^T   [BV][TBP]
  static constexpr int DST = DOT + BV * TBP * 2;        // dS^T   [BV][KBP]
  static constexpr int ET = DST + BV * KBP * 2;         // E^T    [BV][TBP]
  static constexpr int FT = ET + BV * TBP * 2;          // F^T    [BV][TBP]
  static constexpr int BYTES = FT + BV * TBP * 2;
  // sixteen wavefronts where the dS tiles split over them (the E and F tiles
  // then take the first NEF), else eight where dS and E split evenly, else four
  static constexpr int NDS = (DK / 16) * (BV / 16), NEF = (C / 16) * (BV / 16);
  static constexpr int NWV = NDS % 16 == 0 ? 16 : (NDS % 8 == 0 && NEF % 8 == 0) ? 8 : 4, NTH = NWV * kWave;
  static constexpr int NS = NDS / NWV;  // dS tiles per wavefront
};

// The chunk operands of the reverse pass staged through one set of
// registers: K (rows and transposed), Q, T, P and the dO block (transposed),
// all bf16 with C token rows, their 16-byte units numbered in that order and
// dealt to the workgroup's threads (two consecutive rows of one column slice
// per unit, written as in Bf16Stager).
template <int DK, int C, int BV, int NTH>
struct StateStager {
  static constexpr int RP = C / 2;
  static constexpr int UK = RP * (DK / 8), UT = RP * (C / 8), UO = RP * (BV / 8);
  static constexpr int E1 = UK, E2 = 2 * UK, E3 = E2 + UT, E4 = E3 + UT, TOT = E4 + UO, CNT = cdiv(TOT, NTH);
  u32x4 r[CNT][2];
  __device__ __forceinline__ static int which(int idx, int& j) {
    if (idx < E1) { j = idx; return 0; }
    if (idx < E2) { j = idx - E1; return 1; }
    if (idx < E3) { j = idx - E2; return 2; }
    if (idx < E4) { j = idx - E3; return 3; }
    j = idx - E4;
    return 4;
  }
  __device__ __forceinline__ void load(const uint16_t* kk, const uint16_t* qq, int64_t qk_stride, const uint16_t* tt,
                                       const uint16_t* pp, const uint16_t* dov, int64_t v_stride, int valid,
                                       int tid) {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      r[i][0] = r[i][1] = u32x4{0u, 0u, 0u, 0u};
      if (idx >= TOT) continue;
      int j;
      const int op = which(idx, j);
      const int t = 2 * (j % RP), c = (j / RP) * 8;
      const uint16_t* src;
      int64_t stride;  // elements
      int lim = valid;
      if (op <= 1) {
        src = (op == 0 ? kk : qq) + c;
        stride = qk_stride;
      } else if (op <= 3) {  // T, P: whole C x C slots
        src = (op == 2 ? tt : pp) + c;
        stride = C;
        lim = C;
      } else {
        src = dov + c;
        stride = v_stride;
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (t + h < lim) r[i][h] = *reinterpret_cast<const u32x4*>(src + (t + h) * stride);
    }
  }
  __device__ __forceinline__ void store(uint16_t* Kb, int KBP, uint16_t* KbT, uint16_t* QbT, uint16_t* TbT,
                                        uint16_t* PbT, uint16_t* dOT, int TBP, int tid) const {
#pragma unroll
    for (int i = 0; i < CNT; ++i) {
      const int idx = tid + i * NTH;
      if (idx >= TOT) continue;
      int j;
      const int op = which(idx, j);
      const int t = 2 * (j % RP), c = (j / RP) * 8;
      if (op == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) *reinterpret_cast<u32x4*>(Kb + (t + h) * KBP + c) = r[i][h];
      }
      uint16_t* XT = op == 0 ? KbT : op == 1 ? QbT : op == 2 ? TbT : op == 3 ? PbT : dOT;
      union {
        u32x4 u;
        uint16_t e[8];
      } x0, x1;
      x0.u = r[i][0];
      x1.u = r[i][1];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        *reinterpret_cast<uint32_t*>(XT + (c + e) * TBP + t) = uint32_t(x0.e[e]) | (uint32_t(x1.e[e]) << 16);
    }
  }
};

template <int DK, int C>
__global__ __launch_bounds__((BwdStateBf16Shape<DK, C>::NTH)) void bwd_state_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ dout,
    const uint16_t* __restrict__ tws, const uint16_t* __restrict__ pws, const float* __restrict__ dsf,
    uint16_t* __restrict__ dstates, float* __restrict__ ds0, int H, int64_t L, int NC, int DV, int NVB, int remap) {
  using S = BwdStateBf16Shape<DK, C>;
  constexpr int KBP = S::KBP, TBP = S::TBP, BV = S::BV, NS = S::NS, NEF = S::NEF, NWV = S::NWV, NTH = S::NTH;
  static_assert(NS >= 1 && NEF >= 1, "d_k and the chunk are multiples of 32");
  __shared__ __align__(16) unsigned char lds[S::BYTES];
  auto arr = [&](int off) { return reinterpret_cast<uint16_t*>(lds + off); };
  uint16_t *Kb = arr(S::KB), *KbT = arr(S::KBT), *QbT = arr(S::QBT), *TbT = arr(S::TBT), *PbT = arr(S::PBT);
  uint16_t *dOT = arr(S::DOT), *dST = arr(S::DST), *ET = arr(S::ET), *FT = arr(S::FT);

  // Workgroup -> (b, h, value block).  With remap, the value blocks of one
  // (b, h), which read the same Q, K, T and P, get the same blockIdx % 8, i.e.
  // the same XCD and L2.
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
  const int64_t h = bh % H;
  const SeqSpan sp = seq_span<C>(nullptr, bh / H, h, H, L, NC);
  const int v0 = BV * vb;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;

  // dS tiles of this wavefront: tile t = w + NWV i covers dims 16 (t / 2) .., columns 16 (t % 2) ..
  f32x4 dS[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int t = w + NWV * i, d0 = 16 * (t / 2), c0 = 16 * (t % 2);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      dS[i][qq] = dsf != nullptr ? dsf[(int64_t(bh) * DK + d0 + 4 * g + qq) * DV + v0 + c0 + li] : 0.0f;
  }

  // chunk n's operands, staged through registers one chunk ahead
  StateStager<DK, C, BV, NTH> so;
  auto load = [&](int n) {
    const int64_t t0 = int64_t(n) * C;
    const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
    const int64_t row0 = (sp.bos + t0) * H + h;
    so.load(k + row0 * DK, q + row0 * DK, qk_stride, tws + (sp.slot0 + n) * C * C, pws + (sp.slot0 + n) * C * C,
            dout + row0 * DV + v0, v_stride, valid, tid);
  };
  if (sp.nc > 0) load(sp.nc - 1);

  for (int n = sp.nc - 1; n >= 0; --n) {
    __syncthreads();  // the previous chunk's products are done with every array
    // dstates[n] = dS and dS^T (LDS), both bf16: the per-chunk products use
    // dS only as a bf16 operand
    uint16_t* dst = dstates + (sp.slot0 + n) * DK * DV;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int t = w + NWV * i, d0 = 16 * (t / 2), c0 = 16 * (t % 2);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        __builtin_nontemporal_store(from_f32<uint16_t>(dS[i][qq]), dst + (d0 + 4 * g + qq) * DV + v0 + c0 + li);
      st4(dST + (c0 + li) * KBP + d0 + 4 * g, dS[i]);
    }
    so.store(Kb, KBP, KbT, QbT, TbT, PbT, dOT, TBP, tid);
    if (n > 0) load(n - 1);  // in flight during this chunk
    __syncthreads();
    // E = P^T dO + K dS   ([C][BV] tiles; stored as E^T)
#pragma unroll
    for (int t = w; t < NEF; t += NWV) {
      const int r0 = 16 * (t / 2), c0 = 16 * (t % 2);
      f32x4 acc = zero4();
      tile_bf<C>(acc, PbT, TBP, dOT, TBP, r0, c0, li, g);
      tile_bf<DK>(acc, Kb, KBP, dST, KBP, r0, c0, li, g);
      st4(ET + (c0 + li) * TBP + r0 + 4 * g, acc);
    }
    __syncthreads();
    // F = T^T E   (stored as F^T)
#pragma unroll
    for (int t = w; t < NEF; t += NWV) {
      const int r0 = 16 * (t / 2), c0 = 16 * (t % 2);
      f32x4 acc = zero4();
      tile_bf<C>(acc, TbT, TBP, ET, TBP, r0, c0, li, g);
      st4(FT + (c0 + li) * TBP + r0 + 4 * g, acc);
    }
    __syncthreads();
    // dS += Q^T dO - K^T F
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int t = w + NWV * i, d0 = 16 * (t / 2), c0 = 16 * (t % 2);
      f32x4 m = zero4();
      tile_bf<C>(dS[i], QbT, TBP, dOT, TBP, d0, c0, li, g);
      tile_bf<C>(m, KbT, TBP, FT, TBP, d0, c0, li, g);
      dS[i] -= m;
    }
  }
  if (ds0 != nullptr) {
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int t = w + NWV * i, d0 = 16 * (t / 2), c0 = 16 * (t % 2);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) ds0[(int64_t(bh) * DK + d0 + 4 * g + qq) * DV + v0 + c0 + li] = dS[i][qq];
    }
  }
}

}  // namespace efla
