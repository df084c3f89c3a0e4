// ut_wave.h -- the per-chunk UT transform for bf16 inputs, one wavefront per
// chunk, with every operand in registers.
//
// For a chunk of C tokens with key rows K and coefficients a (Method step 3
// of the pages, computed here from beta and lambda = ||k||^2):
//     G = K K^T,   X = (I + diag(a) tril(G, -1))^{-1},   T = X diag(a)
// written row-major to workspace slots of C x C (zeros above the diagonal
// and in rows/columns of tokens past the sequence's end); common.h gives the
// slot of each chunk, for dense and for packed variable-length batches.
//
// Layout of the work inside one wavefront:
//   * K is loaded straight from global memory as 16-byte row fragments.  The
//     sum over the key dimension in K K^T does not depend on the order in
//     which the fragment slots visit the dims, so each lane takes 8
//     consecutive dims (one 16-byte load) per k-unit.
//   * G tiles come from bf16 matrix-core products: the diagonal 16x16 tiles
//     (for lambda and the diagonal solves) and the tiles above the diagonal,
//     which by symmetry are the transposes of the tiles below it.
//   * The diagonal 16x16 blocks of X are solved by forward substitution, one
//     lane per column, all blocks at once, through a small LDS copy of the
//     diagonal G blocks: each lane stores a row piece of its G tile as one
//     16-byte write (G is symmetric, so the tile's column piece is a row
//     piece), and the solve reads each row of G as 16-byte broadcasts.  A
//     wavefront's LDS instructions cost tens of cycles each whatever their
//     width, so the solve's reads were the transform's largest cost.
//   * The blocks below the diagonal follow block by block,
//         X_ij = -X_ii diag(a_i) sum_{j <= m < i} G_im X_mj,
//     on fp32 16x16x4 matrix-core products.  In the kk-th of the four
//     products that make up a 16-deep sum, lane group g supplies k = 4 g + kk:
//     then the B operand is element kk of an accumulator tile as it stands,
//     and the A operand is element kk of the accumulator tile of its
//     transpose, so every product reads its operands from registers.
//   * Every block below the diagonal is also formed transposed (the same two
//     operand tiles, swapped), so each lane holds four consecutive columns
//     of a row of T: T is staged through LDS as bf16 with one 8-byte write
//     per tile and stored with 16-byte row writes.
#pragma once

#include "common.h"

namespace efla {

template <int DK, int C>
struct UtWaveShape {
  static constexpr int NRT = C / 16, NKU = DK / 32;
  // diagonal G blocks, row-major 16 x 16 fp32; blocks 272 floats apart, so
  // the four blocks' rows fall on different banks (broadcast reads)
  static constexpr int GBLK = 272;
  // diagonal X blocks, column-major, columns of 16 (+4) floats
  static constexpr int XP = 20, XBLK = 16 * XP + 16;
  static constexpr int GX = (4 * GBLK + 4 * XBLK) * 4;  // bytes of the two
  static constexpr int TP = C + 8;                      // padded pitch of the bf16 T staging tile
  static constexpr int XST = 32 * (C + 4) * 4;          // a 32-row fp32 block of X (backward instance)
  static constexpr int SCRATCH = GX > C * TP * 2 ? (GX > XST ? GX : XST) : (C * TP * 2 > XST ? C * TP * 2 : XST);
  static constexpr int WAVES = 4;                       // chunks per workgroup
};

// acc += A B over a 16-deep sum with fp32 16x16x4 products: At holds the
// accumulator tile of A^T (element kk of lane (li, g) = A[li][4 g + kk]) and
// B the accumulator tile of B (element kk of lane (li, g) = B[4 g + kk][li]).
__device__ __forceinline__ void mma16_f32(f32x4& acc, const f32x4& At, const f32x4& B) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(At[kk], B[kk], acc, 0, 0, 0);
}

// Compiler-level ordering point for LDS traffic inside one wavefront (the
// hardware executes a wavefront's LDS operations in order).
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

// The instance for the backward pass (BWD) also writes, in fp32 per chunk
// slot: X (C x C, zeros above the diagonal), a (C) and P = tril(Q K^T) (C x C,
// the diagonal included; if PB16 rounded to bf16 and packed as [slots][C][C]
// bf16 from the start of the same buffer), with q the queries in the layout of
// k.  With PB16 and qtout it also writes the chunk's effective queries
//     Qe = Q - P T K   (bf16 [slots][C][d_k], rows of tokens past the end zero),
// the operand through which the output reads the chunk's start state
// (O = Qe S + P T V), so that the reverse pass over the chunks needs no P.
// t_plain: T with ordinary stores (a recurrence reads it next).
template <int DK, int C, bool BWD = false, bool PB16 = false>
__global__ __launch_bounds__(256) void ut_wave_kernel(const uint16_t* __restrict__ k,
                                                      const uint16_t* __restrict__ beta,
                                                      uint16_t* __restrict__ tws, int H, int64_t L, int NC,
                                                      int64_t nchunks, int rule, const int32_t* __restrict__ cu,
                                                      int N, int64_t nwg_ut, int32_t* __restrict__ order,
                                                      const uint16_t* __restrict__ q = nullptr,
                                                      float* __restrict__ xout = nullptr,
                                                      float* __restrict__ aout = nullptr,
                                                      float* __restrict__ pout = nullptr,
                                                      uint16_t* __restrict__ qtout = nullptr, int t_plain = 0) {
  using S = UtWaveShape<DK, C>;
  constexpr int NRT = S::NRT, NKU = S::NKU, GBLK = S::GBLK, XP = S::XP, XBLK = S::XBLK, TP = S::TP;
  constexpr int NKC = C / 32;  // k-units over the tokens of the chunk
  __shared__ __align__(16) unsigned char scratch_all[S::WAVES][S::SCRATCH];
  __shared__ float a_all[S::WAVES][64];

  if (order != nullptr && int64_t(blockIdx.x) >= nwg_ut) {  // packed batch: the workgroups after the chunks rank the sequences
    rank_sequences<C>(cu, N, L, int(blockIdx.x - nwg_ut), order, reinterpret_cast<int*>(scratch_all));
    return;
  }
  const int lane = threadIdx.x & 63, w = wave_id(), li = lane & 15, g = lane >> 4;
  const int64_t id = int64_t(blockIdx.x) * S::WAVES + w;  // workspace slot handled by this wavefront
  if (id >= nchunks) return;                              // no workgroup barriers below
  // slot id -> sequence and chunk (dense: id = (b H + h) NC + chunk)
  SeqSpan sp;
  int chunk;
  const int64_t h = cu == nullptr ? (id / NC) % H : id / NC;
  if (cu == nullptr) {
    chunk = int(id % NC);
    sp = seq_span<C>(nullptr, int(id / NC / H), h, H, L, NC);
  } else if (!slot_chunk<C>(cu, N, id % NC, h, H, L, NC, sp, chunk)) {
    return;  // a slot no chunk of the packed batch uses
  }
  const int64_t t0 = int64_t(chunk) * C;
  const int valid = int(sp.len - t0 < C ? sp.len - t0 : C);
  const int64_t row0 = (sp.bos + t0) * H + h;
  float* Gs = reinterpret_cast<float*>(scratch_all[w]);   // [4][GBLK] diagonal G blocks, row-major
  float* Xs = Gs + 4 * GBLK;                              // [4][XBLK] diagonal X blocks, column-major
  uint16_t* Ts = reinterpret_cast<uint16_t*>(scratch_all[w]);  // [C][TP] bf16 (after Gs/Xs are read)
  float* as = a_all[w];

  // ---- K row fragments and beta ------------------------------------------
  Frag<uint16_t> Kf[NRT][NKU];
#pragma unroll
  for (int rt = 0; rt < NRT; ++rt) {
    const int t = 16 * rt + li;
    const uint16_t* src = k + (row0 + int64_t(t) * H) * DK + 8 * g;
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) {
      if (t < valid) Kf[rt][ku].v = *reinterpret_cast<const bf16x8*>(src + 32 * ku);
      else Kf[rt][ku].v = bf16x8{};
    }
  }
  const float bt = (lane < valid) ? to_f32(beta[row0 + int64_t(lane) * H]) : 0.0f;


  // ---- G: diagonal tiles and the tiles above the diagonal ----------------
  // Gd[b][qq] = G[16b + 4g + qq][16b + li];  Gu[i][m][qq] = G[16m + 4g + qq][16i + li], m < i
  f32x4 Gd[NRT];
  f32x4 Gu[NRT][NRT];
#pragma unroll
  for (int bb = 0; bb < NRT; ++bb) {
    Gd[bb] = zero4();
#pragma unroll
    for (int ku = 0; ku < NKU; ++ku) mma(Gd[bb], Kf[bb][ku], Kf[bb][ku]);
  }
#pragma unroll
  for (int i = 1; i < NRT; ++i)
#pragma unroll
    for (int m = 0; m < i; ++m) {
      Gu[i][m] = zero4();
#pragma unroll
      for (int ku = 0; ku < NKU; ++ku) mma(Gu[i][m], Kf[m][ku], Kf[i][ku]);
    }

  // ---- lambda (the diagonal of G) and a ----------------------------------
  // Gd[bb][qq] = G[16bb + 4g + qq][16bb + li] = G[16bb + li][16bb + 4g + qq]:
  // row li, columns 4g .. 4g+3 of block bb, one 16-byte write
#pragma unroll
  for (int bb = 0; bb < NRT; ++bb) *reinterpret_cast<f32x4*>(Gs + bb * GBLK + li * 16 + 4 * g) = Gd[bb];
  wave_lds_order();
  if (lane < C) {
    const float lam = Gs[(lane >> 4) * GBLK + (lane & 15) * 17];
    as[lane] = (lane < valid) ? efla_alpha_rule(bt, lam, rule) : 0.0f;
  }
  wave_lds_order();

  // ---- diagonal blocks of X: forward substitution, lane = (block, column) --
  //   x_r = delta_rc - a_r * sum_{m < r} G_rm x_m
  // Row r of G is read as ceil(r / 4) 16-byte broadcasts (the lanes of one
  // block share each address); the sum runs as two partial sums.
  {
    const int bb = lane >> 4, c = lane & 15;
    if (bb < NRT) {
      const float* Gb = Gs + bb * GBLK;
      f32x4 ab[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) ab[j] = *reinterpret_cast<const f32x4*>(as + 16 * bb + 4 * j);
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
        for (int j = 0; 4 * j < r; ++j) {
          const f32x4 gr = *reinterpret_cast<const f32x4*>(Gb + r * 16 + 4 * j);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = 4 * j + e;
            if (m < r) {
              if (e & 1) s1 = fmaf(gr[e], x[m], s1);
              else s0 = fmaf(gr[e], x[m], s0);
            }
          }
        }
        x[r] = (r == c ? 1.0f : 0.0f) - ab[r / 4][r % 4] * (s0 + s1);
      }
      // column c of X_bb, four 16-byte writes
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(Xs + bb * XBLK + c * XP + 4 * j) = f32x4{x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]};
    }
  }
  wave_lds_order();
  // X[i][j][qq] = X[16i + 4g + qq][16j + li] (accumulator tiles), XT[i] the tile of X_ii^T
  f32x4 X[NRT][NRT], XT[NRT];
#pragma unroll
  for (int bb = 0; bb < NRT; ++bb) {
    X[bb][bb] = *reinterpret_cast<const f32x4*>(Xs + bb * XBLK + li * XP + 4 * g);
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) XT[bb][qq] = Xs[bb * XBLK + (4 * g + qq) * XP + li];
  }
  // coefficients a[16 i + 4 g + qq]
  f32x4 arow[NRT];
#pragma unroll
  for (int i = 0; i < NRT; ++i) arow[i] = *reinterpret_cast<const f32x4*>(as + 16 * i + 4 * g);
  wave_lds_order();

  // ---- blocks below the diagonal ----------------------------------------
  // XTo[i][j] is the tile of X_ij^T: with the operands of the last product
  // swapped it comes out of the same tiles, (X_ii D_i R)^T = R^T D_i X_ii^T.
  f32x4 XTo[NRT][NRT];
#pragma unroll
  for (int i = 0; i < NRT; ++i) XTo[i][i] = XT[i];
#pragma unroll
  for (int i = 1; i < NRT; ++i)
#pragma unroll
    for (int j = 0; j < i; ++j) {
      f32x4 R = zero4();
#pragma unroll
      for (int m = j; m < i; ++m) mma16_f32(R, Gu[i][m], X[m][j]);  // Gu[i][m] is the tile of G_im^T
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) R[qq] *= arow[i][qq];
      f32x4 Y = zero4(), YT = zero4();
      mma16_f32(Y, XT[i], R);
      mma16_f32(YT, R, XT[i]);
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        X[i][j][qq] = -Y[qq];
        XTo[i][j][qq] = -YT[qq];
      }
    }

  if constexpr (BWD) {  // X (the diagonal blocks as solved, zeros above) and a
    // X in blocks of 32 rows staged through the scratch as fp32 [32][C + 4],
    // then stored with 16-byte row writes
    constexpr int XP = C + 4;
    static_assert(32 * XP * 4 <= S::SCRATCH, "a 32-row block of X fits the scratch");
    float* Xst = reinterpret_cast<float*>(scratch_all[w]);
    float* xdst = xout + id * int64_t(C) * C;
#pragma unroll
    for (int hb = 0; hb < C / 32; ++hb) {
#pragma unroll
      for (int i = 2 * hb; i < 2 * hb + 2; ++i)
#pragma unroll
        for (int j = 0; j < NRT; ++j)
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const int r = 16 * i + 4 * g + qq, c = 16 * j + li;
            Xst[(r - 32 * hb) * XP + c] = (j < i || (j == i && c <= r)) ? X[i][j][qq] : 0.0f;
          }
      wave_lds_order();
#pragma unroll
      for (int idx = lane; idx < 32 * (C / 4); idx += 64) {
        const int r = idx / (C / 4), c0 = (idx % (C / 4)) * 4;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(Xst + r * XP + c0),
                                    reinterpret_cast<u32x4*>(xdst + (32 * hb + r) * C + c0));
      }
      wave_lds_order();  // the next block, then T's staging, reuse the scratch
    }
    if (lane < C) aout[id * int64_t(C) + lane] = as[lane];
  }

  // ---- T = X diag(a): stage as bf16 rows, then 16-byte row stores --------
  // lane (li, g) holds T[16 i + li][16 j + 4 g .. 4 g + 3] = X_ij^T[4 g + qq][li] a[16 j + 4 g + qq]
#pragma unroll
  for (int i = 0; i < NRT; ++i)
#pragma unroll
    for (int j = 0; j < NRT; ++j) {
      bf16x4 tv;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const bool on = j < i || (j == i && 4 * g + qq <= li);
        tv[qq] = static_cast<__bf16>(on ? XTo[i][j < i ? j : i][qq] * arow[j][qq] : 0.0f);
      }
      *reinterpret_cast<bf16x4*>(Ts + (16 * i + li) * TP + 16 * j + 4 * g) = tv;
    }
  wave_lds_order();
  uint16_t* out = tws + id * int64_t(C) * C;
  constexpr int VPR = C / 8;  // 16-byte vectors per row
#pragma unroll
  for (int idx = lane; idx < C * VPR; idx += 64) {
    const int r = idx / VPR, c0 = (idx % VPR) * 8;
    const u32x4 val = *reinterpret_cast<const u32x4*>(Ts + r * TP + c0);
    // nontemporal in the backward instance (the backward's passes ran faster
    // so, as with its other workspace stores); the forward's recurrence reads
    // T right after this kernel and ran ~8 us slower when T was written so
    // (t_plain: the backward instance run ahead of that recurrence)
    if (BWD && !t_plain) __builtin_nontemporal_store(val, reinterpret_cast<u32x4*>(out + r * C + c0));
    else *reinterpret_cast<u32x4*>(out + r * C + c0) = val;
  }

  // ---- backward instance: P = tril(Q K^T) and Qe = Q - P T K -------------
  // Q is read only here (the part above needs only K, whose fragments Kf are
  // held through the solve: with accumulators in ordinary VGPRs that still
  // leaves two wavefronts per SIMD).
  //
  // Qe: every operand comes from registers (the products are laid out so
  // that accumulator tiles are the next product's fragments, as above):
  //   (P T)^T = T^T P^T: tiles (j, rt), j <= rt; T^T's fragment (j, ku) is
  //     X[2 ku + e/4][j] scaled by a[16 j + li] (T = X diag(a)), P^T's is
  //     read back from P's staging tile;
  //   K in accumulator layout, token rows x key columns, by products of the
  //     K row fragments with a selection fragment (exact: one nonzero term);
  //   (P T K)^T = K^T (P T)^T: for key block D, accumulator rows 4 g + qq are
  //     key dims 32 (D / 2) + 8 g + 4 (D % 2) + qq, so the two blocks of a
  //     32-dim unit are, element for element, a Q row fragment (8 consecutive
  //     dims per lane): Qe leaves as 16-byte row pieces.
  if constexpr (BWD) {
    Frag<uint16_t> Kr[NRT][NKU], Qr[NRT][NKU];
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) {
      const int t = 16 * rt + li;
#pragma unroll
      for (int ku = 0; ku < NKU; ++ku) {
        Kr[rt][ku].v = Kf[rt][ku].v;
        Qr[rt][ku].v = bf16x8{};
        if (t < valid) Qr[rt][ku].v = *reinterpret_cast<const bf16x8*>(q + (row0 + int64_t(t) * H) * DK + 32 * ku + 8 * g);
      }
    }
    wave_lds_order();  // T's staging tile has been read: the scratch takes P
    // P = tril(Q K^T), diagonal included, in the same per-lane order of the
    // key dims for Q and K
    float* pdst = pout + id * int64_t(C) * C;                                    // fp32 P
    uint16_t* pdst16 = reinterpret_cast<uint16_t*>(pout) + id * int64_t(C) * C;  // bf16 P (PB16)
#pragma unroll
    for (int r = 0; r < NRT; ++r)
#pragma unroll
      for (int c = 0; c < NRT; ++c) {
        f32x4 acc = zero4();
        if (c <= r) {
#pragma unroll
          for (int ku = 0; ku < NKU; ++ku) mma(acc, Qr[r][ku], Kr[c][ku]);
        }
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          const int ii = 16 * r + 4 * g + qq, jj = 16 * c + li;
          const float pv = jj <= ii ? acc[qq] : 0.0f;
          if constexpr (PB16) Ts[ii * TP + jj] = from_f32<uint16_t>(pv);  // staged, stored as rows below
          else pdst[ii * C + jj] = pv;
        }
      }
    if constexpr (PB16) {  // bf16 P: 16-byte row stores from the staging tile
      wave_lds_order();
#pragma unroll
      for (int idx = lane; idx < C * (C / 8); idx += 64) {
        const int r = idx / (C / 8), c0 = (idx % (C / 8)) * 8;
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(Ts + r * TP + c0),
                                    reinterpret_cast<u32x4*>(pdst16 + r * C + c0));
      }
    }
    if (PB16 && qtout != nullptr) {
      // P^T as B operand fragments (k = token l, column = row 16 rt + li of P;
      // element e of lane group g is P[16 rt + li][32 ku + 16 (e / 4) + 4 g + e % 4]),
      // ku <= rt / 2 (P is lower triangular)
      Frag<uint16_t> PtB[NRT][NKC];
#pragma unroll
      for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
        for (int ku = 0; ku < NKC; ++ku)
          if (2 * ku <= rt) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(Ts + (16 * rt + li) * TP + 32 * ku + 4 * g);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(Ts + (16 * rt + li) * TP + 32 * ku + 16 + 4 * g);
            PtB[rt][ku].v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
      float acol[NRT];
#pragma unroll
      for (int j = 0; j < NRT; ++j) acol[j] = as[16 * j + li];
      f32x4 PTt[NRT][NRT];  // [j][rt]: (P T)^T[16 j + 4 g + qq][16 rt + li]
#pragma unroll
      for (int j = 0; j < NRT; ++j)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          PTt[j][rt] = zero4();
          if (j > rt) continue;
#pragma unroll
          for (int ku = j / 2; ku <= rt / 2; ++ku) {
            f32x4 lo = zero4(), hi = zero4();
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
              if (j <= 2 * ku) lo[qq] = X[2 * ku][j][qq] * acol[j];
              if (j <= 2 * ku + 1) hi[qq] = X[2 * ku + 1][j][qq] * acol[j];
            }
            mma(PTt[j][rt], acc_frag<uint16_t>(lo, hi), PtB[rt][ku]);
          }
        }
      Frag<uint16_t> PTB[NKC][NRT];  // (P T)^T as B operand: k = token, column = row 16 rt + li of P T
#pragma unroll
      for (int ku = 0; ku < NKC; ++ku)
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
          if (2 * ku <= rt) PTB[ku][rt] = acc_frag<uint16_t>(PTt[2 * ku][rt], PTt[2 * ku + 1][rt]);
      uint16_t* qdst = qtout + id * int64_t(C) * DK;
#pragma unroll
      for (int ku2 = 0; ku2 < NKU; ++ku2) {
        f32x4 Cq[2][NRT];  // [h][rt]: (P T K)[16 rt + li][32 ku2 + 8 g + 4 h + qq]
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          // selection: slot (g, e) of the k-unit is key dim 32 ku2 + 8 g + e in Kr;
          // column li picks dim 32 ku2 + 8 (li / 4) + 4 hh + li % 4
          Frag<uint16_t> sel;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            sel.v[e] = static_cast<__bf16>((g == (li >> 2) && e == 4 * hh + (li & 3)) ? 1.0f : 0.0f);
          f32x4 ZK[NRT];  // K[16 tb + 4 g + qq][that dim of column li]
#pragma unroll
          for (int tb = 0; tb < NRT; ++tb) {
            ZK[tb] = zero4();
            mma(ZK[tb], Kr[tb][ku2], sel);
          }
#pragma unroll
          for (int rt = 0; rt < NRT; ++rt) {
            Cq[hh][rt] = zero4();
#pragma unroll
            for (int ku = 0; 2 * ku <= rt; ++ku)
              mma(Cq[hh][rt], acc_frag<uint16_t>(ZK[2 * ku], ZK[2 * ku + 1]), PTB[ku][rt]);
          }
        }
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt) {
          const int t = 16 * rt + li;
          const bf16x8 qv = Qr[rt][ku2].v;
          bf16x8 o;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = static_cast<__bf16>(static_cast<float>(qv[e]) - Cq[e / 4][rt][e % 4]);
          __builtin_nontemporal_store(o, reinterpret_cast<bf16x8*>(qdst + t * DK + 32 * ku2 + 8 * g));
        }
      }
    }
  }
}

inline bool ut_wave_supported(int DK, int C) { return (DK == 32 || DK == 64 || DK == 128) && (C == 32 || C == 64); }

// Dense batches: B sequences of L tokens.  Packed batches (cu != nullptr):
// N sequences with offsets cu in a batch of L tokens (B is ignored).
template <int DK, int C>
hipError_t ut_wave_launch_impl(const uint16_t* k, const uint16_t* beta, uint16_t* tws, int B, int H, int64_t L,
                               int rule, const int32_t* cu, int N, int32_t* order, hipStream_t stream) {
  static_assert(64 * UtWaveShape<DK, C>::WAVES == kThreads && UtWaveShape<DK, C>::WAVES * UtWaveShape<DK, C>::SCRATCH >=
                    int(kRankSeqs * sizeof(int)), "ranking workgroups reuse the kernel's shape and LDS");
  const int NC = cu == nullptr ? int((L + C - 1) / C) : int(L / C) + N;
  const int64_t nchunks = int64_t(cu == nullptr ? B : 1) * H * NC;
  if (cu == nullptr) order = nullptr;
  const int64_t nwg = (nchunks + UtWaveShape<DK, C>::WAVES - 1) / UtWaveShape<DK, C>::WAVES;
  const int64_t nrank = order != nullptr ? (N + kRankSeqs - 1) / kRankSeqs : 0;
  if (nwg + nrank == 0) return hipSuccess;
  hipLaunchKernelGGL((ut_wave_kernel<DK, C>), dim3(unsigned(nwg + nrank)), dim3(64 * UtWaveShape<DK, C>::WAVES), 0,
                     stream, k, beta, tws, H, L, NC, nchunks, rule, cu, N, nwg, order);
  return hipGetLastError();
}

inline hipError_t launch_ut_wave(const uint16_t* k, const uint16_t* beta, uint16_t* tws, int B, int H, int64_t L,
                                 int DK, int C, int rule, const int32_t* cu, int N, int32_t* order, hipStream_t s) {
  if (C == 32) {
    switch (DK) {
      case 32: return ut_wave_launch_impl<32, 32>(k, beta, tws, B, H, L, rule, cu, N, order, s);
      case 64: return ut_wave_launch_impl<64, 32>(k, beta, tws, B, H, L, rule, cu, N, order, s);
      case 128: return ut_wave_launch_impl<128, 32>(k, beta, tws, B, H, L, rule, cu, N, order, s);
    }
  } else if (C == 64) {
    switch (DK) {
      case 32: return ut_wave_launch_impl<32, 64>(k, beta, tws, B, H, L, rule, cu, N, order, s);
      case 64: return ut_wave_launch_impl<64, 64>(k, beta, tws, B, H, L, rule, cu, N, order, s);
      case 128: return ut_wave_launch_impl<128, 64>(k, beta, tws, B, H, L, rule, cu, N, order, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace efla
