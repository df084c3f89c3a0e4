// recurrence_v4.h -- the sequential chunk pass for bf16 inputs: one wavefront
// per 16-column tile of the state, chunk inputs streamed into LDS by DMA.
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

#include "recurrence_v3.h"

namespace efla {

typedef __attribute__((address_space(3))) void lds_void_t;

// Physical 16-byte chunk for logical chunk `c` of row `r` in a row of NCH
// chunks (NCH = row bytes / 16).  A 1 KiB DMA instruction covers RPI = 64/NCH
// rows, and the swizzle is f(r % RPI) ^ g(r / RPI): the lane-dependent part is
// the same for every instruction, the instruction-dependent part is uniform.
// It spreads any 16 consecutive rows over distinct bank groups (row-fragment
// reads, 16 rows x 8 B) and keeps the two chunks of any 4 consecutive rows
// apart (transposing reads, 4 rows x 32 B).  Rows share the 64 LDS banks
// 256 / (16 NCH) at a time.
template <int NCH>
__device__ __forceinline__ int swz_lane(int rr) {  // f: rr = r % RPI
  if constexpr (NCH >= 16) return 2 * (rr & 3);
  else if constexpr (NCH == 8) return 2 * ((rr >> 1) & 3);
  else if constexpr (NCH == 4) return (rr >> 2) & 3;
  else return 0;
}
template <int NCH>
__device__ __forceinline__ int swz_instr(int b) {  // g: b = r / RPI
  if constexpr (NCH >= 16) return (b & 1) | ((b & 2) << 2);
  else if constexpr (NCH == 8) return b & 1;
  else return 0;
}
template <int NCH>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  constexpr int RPI = 64 / NCH;
  return c ^ swz_lane<NCH>(r % RPI) ^ swz_instr<NCH>(r / RPI);
}

// A second swizzle, for tiles read with 16-byte row fragments (16 rows, one
// 16-byte chunk each) and with transposing reads of 4 rows x 4 consecutive
// chunks (8 bytes of each): s(r) = f(r % RPI) ^ g(r / RPI) with
//   16 chunks per row: s = 4 (r & 3) ^ ((r >> 2) & 3)
//    8 chunks per row: s = 4 ((r >> 1) & 1) ^ ((r >> 2) & 1) ^ 2 ((r >> 3) & 1)
//    4 chunks per row: s = (r >> 2) & 3
// Any 16 consecutive (16-aligned) rows then land on distinct bank groups, and
// so do the 16 (row, chunk) pairs of a transposing read.
template <int NCH>
__device__ __forceinline__ int swzw_lane(int rr) {  // rr = r % RPI
  if constexpr (NCH >= 16) return 4 * (rr & 3);
  else if constexpr (NCH == 8) return 4 * ((rr >> 1) & 1) + ((rr >> 2) & 1);
  else if constexpr (NCH == 4) return (rr >> 2) & 3;
  else return 0;
}
template <int NCH>
__device__ __forceinline__ int swzw_instr(int b) {  // b = r / RPI
  if constexpr (NCH >= 16) return b & 3;
  else if constexpr (NCH == 8) return 2 * (b & 1);
  else return 0;
}
template <int NCH, bool WIDE>
__device__ __forceinline__ int swz_lane_of(int rr) {
  if constexpr (WIDE) return swzw_lane<NCH>(rr);
  else return swz_lane<NCH>(rr);
}
template <int NCH, bool WIDE>
__device__ __forceinline__ int swz_instr_of(int b) {
  if constexpr (WIDE) return swzw_instr<NCH>(b);
  else return swz_instr<NCH>(b);
}
template <int ROWE>
__device__ __forceinline__ int swzw_off(int r, int col) {
  constexpr int NCH = ROWE / 8, RPI = 64 / NCH;
  return r * ROWE + (((col >> 3) ^ swzw_lane<NCH>(r % RPI) ^ swzw_instr<NCH>(r / RPI)) * 8) + (col & 7);
}

// Element offset of (r, col) in a swizzled bf16 tile with ROWE elements per row.
template <int ROWE>
__device__ __forceinline__ int swz_off(int r, int col) {
  constexpr int NCH = ROWE / 8;
  return r * ROWE + swz_chunk<NCH>(r, col >> 3) * 8 + (col & 7);
}

template <int ROWE>
__device__ __forceinline__ Frag<uint16_t> sw_frag(const uint16_t* X, int row, int ku, int g) {
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(X + swz_off<ROWE>(row, 32 * ku + 4 * g));
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(X + swz_off<ROWE>(row, 32 * ku + 16 + 4 * g));
  Frag<uint16_t> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// Transposed fragment (operand row = column m0 + li of X, k = rows of X).
template <int ROWE>
__device__ __forceinline__ Frag<uint16_t> sw_frag_tr(const uint16_t* X, int m0, int ku, int lane) {
  const int j = lane & 15, g = lane >> 4;
  const int r = 32 * ku + 4 * g + (j >> 2), c = m0 + 4 * (j & 3);
  const bf16x4 lo = lds_read_tr(X + swz_off<ROWE>(r, c));
  const bf16x4 hi = lds_read_tr(X + swz_off<ROWE>(r + 16, c));
  Frag<uint16_t> f;
  f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}

// One direct global -> LDS transfer of 16 bytes per lane: lane L reads
// sbase + voff (voff per lane) and its bytes land at LDS byte address
// lds_addr + 16 L (lds_addr wave-uniform, held in M0).  Issued through inline
// asm so the compiler's wait-count model, which cannot tell ring slots apart,
// does not add a drain of all transfers before every LDS read; the kernel
// waits for exactly the transfers it needs.  The asm is volatile, so it stays
// ordered with the kernel's waits and barriers (also volatile asm), but it
// has no memory clobber: it only writes an LDS slot nobody reads until the
// next barrier, so LDS reads and products may be scheduled around it.  M0 is
// saved and restored around the transfer, and s_nop covers the M0-write hazard.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      // readfirstlane: a no-op on a value already in a scalar register, and a
      // guard where the compiler keeps the (uniform) address in a vector one
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_addr)));
}

// A pointer the whole wavefront agrees on, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(u >> 32));
  return reinterpret_cast<const void*>((uint64_t(hi) << 32) | lo);
}

// LDS byte address of a __shared__ object, as a wave-uniform (scalar) value.
__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p))));
}

// DMA of ROWS x ROWE bf16 (row t at src + t*stride) into a swizzled LDS tile.
// The tile is a multiple of 1 KiB; wave w of NW issues instructions w, w + NW,
// ... and every wave issues exactly cdiv(ninstr, NW) of them (a wave past the
// end repeats its last one), so all waves issue the same count.  init()
// computes, once, each lane's byte offset for every instruction of a full
// tile; a ragged tile (rows at or past `valid` re-read row 0) takes the
// slower per-instruction path.
template <int ROWS, int ROWE, int NW, bool WIDE = false>
struct DmaTile {
  static constexpr int BYTES = ROWS * ROWE * 2, NINSTR = BYTES / 1024, PER_WAVE = cdiv(NINSTR, NW);
  static constexpr int NCH = ROWE / 8, RPI = 64 / NCH;
  static_assert(BYTES % 1024 == 0, "DMA tiles are whole KiB");
  uint32_t off[PER_WAVE];       // lane byte offset of each instruction, full tile
  uint32_t off_chunk;           // lane's swizzled chunk offset within its row
  int lrow, w;                  // lane's row within one instruction; wave index
  __device__ __forceinline__ static int instr(int w, int i) {
    const int ins = w + i * NW;
    return ins < NINSTR ? ins : NINSTR - 1;
  }
  __device__ __forceinline__ void init(int64_t stride, int lane, int wave) {
    w = __builtin_amdgcn_readfirstlane(wave);  // uniform: LDS addresses stay scalar
    lrow = lane / NCH;
    off_chunk = 16u * uint32_t((lane % NCH) ^ swz_lane_of<NCH, WIDE>(lrow));
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int ins = instr(w, i);
      off[i] = uint32_t((RPI * ins + lrow) * stride * 2) +
               (off_chunk ^ (16u * uint32_t(swz_instr_of<NCH, WIDE>(ins))));
    }
  }
  // Instruction i of this wave for the tile at LDS byte address lds_tile
  // (wave-uniform), source row 0 at src.  RAGGED: rows at or past `valid`
  // re-read row 0 (only the last chunk of a sequence can be ragged).
  template <bool RAGGED>
  __device__ __forceinline__ void issue(int i, uint32_t lds_tile, const uint16_t* src, int valid) const {
    const int ins = instr(w, i);
    uint32_t voff = off[i];
    if constexpr (RAGGED) {
      const uint32_t xo = 16u * uint32_t(swz_instr_of<NCH, WIDE>(ins));
      voff = (RPI * ins + lrow < valid) ? voff : (off_chunk ^ xo);
    }
    dma16(src, voff, lds_tile + uint32_t(ins) * 1024u);
  }
};

// WIDE_QK selects the 16-byte-fragment swizzle for the Q and K tiles.
template <int DK, int C, int BV, int NW, bool WIDE_QK = false>
struct ChunkDma {
  using TQ = DmaTile<C, DK, NW, WIDE_QK>;
  using TT = DmaTile<C, C, NW>;
  using TV = DmaTile<C, BV, NW>;
  static constexpr int PQ = TQ::PER_WAVE, PT = TT::PER_WAVE, PV = TV::PER_WAVE;
  static constexpr int COUNT = 2 * PQ + PT + PV;
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  TQ tq;
  TT tt;
  TV tv;
  int64_t qk_stride, v_stride;
  struct Src {
    const uint16_t *q, *k, *t, *v;
    int valid;
  };
  __device__ __forceinline__ void init(int64_t qk_stride_, int64_t v_stride_, int lane, int wave) {
    qk_stride = qk_stride_;
    v_stride = v_stride_;
    tq.init(qk_stride, lane, wave);
    tt.init(C, lane, wave);
    tv.init(v_stride, lane, wave);
  }
  template <bool RAGGED>
  __device__ __forceinline__ void issue(int j, uint32_t slot, const Src& src) const {
    if (j < PQ) tq.template issue<RAGGED>(j, slot + 2 * QOFF, src.q, src.valid);
    else if (j < 2 * PQ) tq.template issue<RAGGED>(j - PQ, slot + 2 * KOFF, src.k, src.valid);
    else if (j < 2 * PQ + PT) tt.template issue<false>(j - 2 * PQ, slot + 2 * TOFF, src.t, C);
    else tv.template issue<RAGGED>(j - 2 * PQ - PT, slot + 2 * VOFF, src.v, src.valid);
  }
  // Piece `part` of `parts` (an even split of the COUNT instructions) into
  // the ring slot at LDS byte address `slot`; src pointers are wave-uniform.
  __device__ __forceinline__ void issue_part(int part, int parts, uint32_t slot, const Src& src) const {
    if (src.valid == C) {
#pragma unroll
      for (int j = 0; j < COUNT; ++j)
        if (j >= part * COUNT / parts && j < (part + 1) * COUNT / parts) issue<false>(j, slot, src);
    } else {
#pragma unroll
      for (int j = 0; j < COUNT; ++j)
        if (j >= part * COUNT / parts && j < (part + 1) * COUNT / parts) issue<true>(j, slot, src);
    }
  }
};

template <int DK, int C, int BV>
struct V4Shape {
  static constexpr int NW = BV / 16, THREADS = NW * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;  // elements, a multiple of 512
  using Dma = ChunkDma<DK, C, BV, NW>;
  static constexpr int DMA_PER_WAVE = Dma::COUNT;
  static constexpr int STORES_PER_WAVE = NRT;  // one 8-byte O store per row tile
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that does not wait for outstanding memory operations; the
// caller waits for exactly the transfers it needs first.  The asm memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_nowait() { asm volatile("s_barrier" ::: "memory"); }

template <int DK, int C, int BV>
__global__ __launch_bounds__(4 * BV) void recurrence_v4_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ tws, const float* __restrict__ s0, uint16_t* __restrict__ o,
    float* __restrict__ sfin, int H, int64_t L, int NC, int DV, int NVB, int remap) {
  using S = V4Shape<DK, C, BV>;
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

inline bool v4_supported(int DK, int C, int BV) {
  return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64) && (BV == 16 || BV == 32 || BV == 64);
}

template <int DK, int C, int BV>
hipError_t recurrence_v4_launch_impl(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                     int B, int H, int64_t L, int DV, hipStream_t stream) {
  using S = V4Shape<DK, C, BV>;
  const int NC = int((L + C - 1) / C);
  const int BH = B * H;
  const int NVB = DV / BV;
  const int nwg = BH * NVB;
  if (nwg == 0) return hipSuccess;
  const int remap = (BH % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL((recurrence_v4_kernel<DK, C, BV>), dim3(unsigned(nwg)), dim3(S::THREADS), 0, stream, q,
                     k, v, tws, s0, o, sfin, H, L, NC, DV, NVB, remap);
  return hipGetLastError();
}

template <int DK, int C>
hipError_t recurrence_v4_bv(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* tws,
                            const float* s0, uint16_t* o, float* sfin, int B, int H, int64_t L, int DV,
                            int BV, hipStream_t s) {
  switch (BV) {
    case 16: return recurrence_v4_launch_impl<DK, C, 16>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
    case 32: return recurrence_v4_launch_impl<DK, C, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
    case 64: return recurrence_v4_launch_impl<DK, C, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, s);
  }
  return hipErrorInvalidValue;
}

inline hipError_t launch_recurrence_v4(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       hipStream_t s) {
  if (C == 32) {
    switch (DK) {
      case 32: return recurrence_v4_bv<32, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_v4_bv<64, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_v4_bv<128, 32>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return recurrence_v4_bv<32, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 64: return recurrence_v4_bv<64, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
      case 128: return recurrence_v4_bv<128, 64>(q, k, v, tws, s0, o, sfin, B, H, L, DV, BV, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
