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
//     three slots, issued two chunks ahead (at the end of the step that frees
//     the slot).  Each wave waits (s_waitcnt vmcnt) for its own transfers and
//     one s_barrier per chunk publishes the slot;
//   * LDS rows are unpadded (a DMA instruction fills 1 KiB contiguously) and
//     16-byte chunks are XOR-swizzled per row so that both the row-fragment
//     reads (16 rows x 8 B) and the transposing reads (4 rows x 32 B) of
//     ds_read_b64_tr_b16 are free of bank conflicts;
//   * K^T and the V tile come from ds_read_b64_tr_b16; P stays in registers.
#pragma once

#include "recurrence_v3.h"

namespace efla {

typedef __attribute__((address_space(3))) void lds_void_t;

// Physical 16-byte chunk for logical chunk `c` of row `r` in a row of NCH
// chunks (NCH = row bytes / 16).  Rows share the 64 LDS banks 256/(16 NCH) at
// a time; the swizzle spreads 16 consecutive rows over distinct chunk slots
// and keeps the two chunks of any 4 consecutive rows distinct.
template <int NCH>
__device__ __forceinline__ int swz_chunk(int r, int c) {
  if constexpr (NCH >= 16) return c ^ ((2 * r + (r >> 3)) & 15);
  else if constexpr (NCH == 8) return c ^ ((2 * (r >> 1) + (r >> 3)) & 7);
  else if constexpr (NCH == 4) return c ^ ((r >> 2) & 3);
  else return c;
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

// One direct global -> LDS transfer of 16 bytes per lane: lane L's bytes land
// at LDS byte address lds_addr + 16 L (lds_addr wave-uniform, held in M0).
// Issued through inline asm so the compiler's wait-count model, which cannot
// tell ring slots apart, does not add a drain of all transfers before every
// LDS read; the kernel waits for exactly the transfers it needs.  M0 is saved
// and restored around the transfer, and s_nop covers the M0-write hazard.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_addr)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)(p)));
}

// DMA of ROWS x ROWE bf16 (row t at src + t*stride) into a swizzled LDS tile.
// The tile is 1 KiB-aligned and a multiple of 1 KiB; wave w of NW issues
// instructions w, w + NW, ... and every wave issues exactly cdiv(ninstr, NW)
// of them (a wave past the end repeats its last one), so all waves issue the
// same count.  Rows at or past `valid` re-read row 0.
template <int ROWS, int ROWE, int NW>
struct DmaTile {
  static constexpr int BYTES = ROWS * ROWE * 2, NINSTR = BYTES / 1024, PER_WAVE = cdiv(NINSTR, NW);
  static_assert(BYTES % 1024 == 0, "DMA tiles are whole KiB");
  __device__ __forceinline__ static void issue(uint16_t* lds_tile, const uint16_t* src, int64_t stride,
                                               int valid, int w, int lane) {
    constexpr int NCH = ROWE / 8;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      int ins = w + i * NW;
      ins = ins < NINSTR ? ins : NINSTR - 1;
      const int p = ins * 512 + lane * 8;  // element offset this lane lands at
      const int r = p / ROWE, pc = (p % ROWE) >> 3;
      const int lc = swz_chunk<NCH>(r, pc);  // the swizzle is an involution
      const int rs = r < valid ? r : 0;
      dma16(src + rs * stride + lc * 8, __builtin_amdgcn_readfirstlane(lds_addr_of(lds_tile + ins * 512)));
    }
  }
};

template <int DK, int C, int BV>
struct V4Shape {
  static constexpr int NW = BV / 16, THREADS = NW * kWave;
  static constexpr int NRT = C / 16, NDT = DK / 16, NKU_D = DK / 32, NKU_C = C / 32;
  static constexpr int QOFF = 0, KOFF = C * DK, TOFF = 2 * C * DK, VOFF = 2 * C * DK + C * C;
  static constexpr int SLOT = 2 * C * DK + C * C + C * BV;  // elements, a multiple of 512
  static constexpr int OP = 24;  // padded pitch of a wave's output staging tile
  using DQ = DmaTile<C, DK, NW>;
  using DT = DmaTile<C, C, NW>;
  using DV = DmaTile<C, BV, NW>;
  static constexpr int DMA_PER_WAVE = 2 * DQ::PER_WAVE + DT::PER_WAVE + DV::PER_WAVE;
  static constexpr int STORES_PER_WAVE = NRT;  // one 16-byte O store per row tile
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
  constexpr int OP = S::OP;
  // Three separate arrays (not one indexed ring) so that alias analysis can
  // tell the slot being filled by DMA from the slot being read: the compiler
  // then leaves the in-flight transfers alone instead of waiting for them.
  __shared__ __align__(1024) uint16_t slot0[S::SLOT];
  __shared__ __align__(1024) uint16_t slot1[S::SLOT];
  __shared__ __align__(1024) uint16_t slot2[S::SLOT];
  __shared__ __align__(16) uint16_t Os[NW * 16 * OP];

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
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int col = v0 + 16 * w + li;
  uint16_t* Ow = Os + w * 16 * OP;

  const int64_t qk_stride = int64_t(H) * DK, v_stride = int64_t(H) * DV;
  auto chunk_valid = [&](int n) { return int(L - int64_t(n) * C < C ? L - int64_t(n) * C : C); };
  auto row_of = [&](int n) { return (b * L + int64_t(n) * C) * H + h; };
  // Issue the DMA of chunk n (clamped to the last chunk, so every wave always
  // issues the same number of transfers) into `slot`.
  auto issue_chunk = [&](uint16_t* slot, int n) {
    const int nn = n < NC ? n : NC - 1;
    const int64_t r0 = row_of(nn);
    const int valid = chunk_valid(nn);
    S::DQ::issue(slot + S::QOFF, q + r0 * DK, qk_stride, valid, w, lane);
    S::DQ::issue(slot + S::KOFF, k + r0 * DK, qk_stride, valid, w, lane);
    S::DT::issue(slot + S::TOFF, tws + (int64_t(bh) * NC + nn) * C * C, C, C, w, lane);
    S::DV::issue(slot + S::VOFF, v + r0 * DV + v0, v_stride, valid, w, lane);
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
    issue_chunk(slot0, 0);
    issue_chunk(slot1, 1);
  }

  constexpr int D = S::DMA_PER_WAVE, ST = S::STORES_PER_WAVE;
  // One chunk: `cur` holds chunk n; chunk n + 2 is sent to `fill`.
  auto chunk_step = [&](const uint16_t* __restrict__ cur, uint16_t* __restrict__ fill, int n) {
    // This wave's transfers for chunk n are done once at most the operations
    // issued after them are outstanding: for n >= 1 that is step n-1's output
    // stores and its transfers of chunk n+1; for n = 0, the transfers of chunk 1.
    if (n == 0) wait_vmcnt<D>();
    else wait_vmcnt<D + ST>();
    barrier_nowait();  // chunk n visible to all waves; `fill` no longer read

    const uint16_t* Qs = cur + S::QOFF;
    const uint16_t* Ks = cur + S::KOFF;
    const uint16_t* Ts = cur + S::TOFF;
    const uint16_t* Vs = cur + S::VOFF;
    const int valid = chunk_valid(n);
    const int64_t row0 = row_of(n);

    Frag<uint16_t> bS[NKU_D];
#pragma unroll
    for (int ku = 0; ku < NKU_D; ++ku) bS[ku] = acc_frag<uint16_t>(St[2 * ku], St[2 * ku + 1]);

    // K fragments of every row tile (rows are both Y's rows and P's s index)
    Frag<uint16_t> Kf[NRT][NKU_D];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) Kf[rt][ku] = sw_frag<DK>(Ks, 16 * rt + li, ku, g);

    f32x4 Y[NRT], Z[NRT], Pt[NRT][NRT];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      Frag<uint16_t> Qf[NKU_D];
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) Qf[ku] = sw_frag<DK>(Qs, 16 * rt + li, ku, g);
      Y[rt] = zero4();
      Z[rt] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU_D; ++ku) {
        mma(Y[rt], Kf[rt][ku], bS[ku]);
        mma(Z[rt], Qf[ku], bS[ku]);
      }
      // P tiles of this t-row tile: Pt[rt][c][qq] = P[16rt + li][16c + 4g + qq]
#pragma unroll
      for (int c = 0; c < NRT; ++c) {
        Pt[rt][c] = zero4();
        if (c <= rt) {
#pragma unroll
          for (int ku = 0; ku < NKU_D; ++ku) mma(Pt[rt][c], Kf[c][ku], Qf[ku]);
          if (c == rt) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
              if (4 * g + qq > li) Pt[rt][c][qq] = 0.0f;
          }
        }
      }
    }

    // D = V - Y  (V tile rows 16rt + 4g + e, column li, by transposing read)
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int j = lane & 15;
      const bf16x4 vv = lds_read_tr(Vs + swz_off<BV>(16 * rt + 4 * g + (j >> 2), 16 * w + 4 * (j & 3)));
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) Y[rt][qq] = static_cast<float>(vv[qq]) - Y[rt][qq];
    }

    // U' = T D
    Frag<uint16_t> Tf[NRT][NKU_C];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku <= 16 * rt + 15) Tf[rt][ku] = sw_frag<C>(Ts, 16 * rt + li, ku, g);
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

    // S += K^T U'  (K^T fragments by transposing reads, four tiles at a time)
#pragma unroll
    for (int d0 = 0; d0 < NDT; d0 += 4) {
      Frag<uint16_t> KTf[4][NKU_C];
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt)
          if (d0 + dd < NDT) KTf[dd][kt] = sw_frag_tr<DK>(Ks, 16 * (d0 + dd), kt, lane);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd)
#pragma unroll
        for (int kt = 0; kt < NKU_C; ++kt)
          if (d0 + dd < NDT) mma(St[d0 + dd], KTf[dd][kt], bU[kt]);
    }

    // O = Z + P U', staged through this wave's LDS tile into 16-byte row stores
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      f32x4 acc = Z[rt];
#pragma unroll
      for (int ku = 0; ku < NKU_C; ++ku)
        if (32 * ku <= 16 * rt + 15) {
          const f32x4 phi = (2 * ku + 1 <= rt) ? Pt[rt][(2 * ku + 1) % NRT] : zero4();
          mma(acc, acc_frag<uint16_t>(Pt[rt][2 * ku], phi), bU[ku]);
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
    // The transfers of chunk n + 2 go out after this step's last LDS read, so
    // the compiler has no LDS read behind them to hold back.
    issue_chunk(fill, n + 2);
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
