// launchers.h -- host-side launch functions of the EFLA kernels, one set per
// element type (float, or bf16 carried as uint16_t).  Each returns the HIP
// error of its launch; argument validation happens in the C ABI layer.
// Chunked launchers take a dense batch (B sequences of L tokens, cu ==
// nullptr) or a packed variable-length batch (N sequences with device
// offsets cu[0..N] into L tokens; B is then ignored), see SeqSpan.
#pragma once

#include "common.h"

namespace efla {

template <typename T>
hipError_t launch_coeff(const T* k, const T* beta, float* lam, float* alpha, int64_t n, int DK, int rule,
                        hipStream_t s);

template <typename T>
hipError_t launch_step(const T* q, const T* k, const T* v, const T* beta, float* state, T* o,
                       int64_t units, int DK, int DV, int rule, hipStream_t s);

// Packed batches: with order != nullptr the launch also writes the schedule
// of the N sequences (rank -> sequence, longest first, see rank_sequences)
// for the recurrence launch that follows.
template <typename T>
hipError_t launch_ut_transform(const T* k, const T* beta, T* tws, int B, int H, int64_t L, int DK,
                               int C, int rule, const int32_t* cu, int N, hipStream_t stream,
                               int32_t* order = nullptr);

// order (packed batches only, nullable): the schedule of sequences, rank ->
// sequence, written by the UT-transform launch; workgroups of rank 0 start first.
template <typename T>
hipError_t launch_recurrence(const T* q, const T* k, const T* v, const T* tws, const float* s0,
                             T* o, float* sfin, int B, int H, int64_t L, int DK, int DV, int C,
                             int BV, const int32_t* cu, int N, hipStream_t stream, int trans = 0,
                             const int32_t* order = nullptr);

// bf16 recurrence with one wavefront per 16-column state tile and a DMA-fed
// LDS ring (recurrence_tile.h); d_k in {32, 64, 128}, chunk in {32, 64},
// value blocks of 16, 32 or 64 columns.  Dense batches only.
bool recurrence_tile_supported(int DK, int C, int BV);
hipError_t launch_recurrence_tile_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                       const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                       int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                       hipStream_t s);

// bf16 recurrence with one role per wavefront: chain wavefronts, output, P
// and DMA (recurrence_roles.h); same d_k and chunk, value blocks of 16 or 32.
// With states given, the backward pass's instance runs instead: it writes the
// state at the start of every chunk (bf16, per chunk slot) and no output.
// o == NULL: final states only.  trans: the chunk-transition instance (V = 0,
// identity initial state, final states only; pass v = k and DV = DK).
bool recurrence_roles_supported(int DK, int C, int BV);
hipError_t launch_recurrence_roles_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                        int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                        const int32_t* cu, int N, hipStream_t s, uint16_t* states = nullptr,
                                        bool trans = false, const int32_t* order = nullptr);

// bf16 recurrence with each chunk's work spread over nine wavefronts
// (recurrence_split.h): d_k in {64, 128}, chunk 64, value blocks of 32;
// forward instance only (output and final state), dense or packed batches;
// statesT (dense batches, BV 32): also every chunk's start state as the bf16
// operand values, [slots][DV][DK] as the backward's state-only pass writes them.
bool recurrence_split_supported(int DK, int C, int BV);
hipError_t launch_recurrence_split_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                        const uint16_t* tws, const float* s0, uint16_t* o, float* sfin,
                                        int B, int H, int64_t L, int DK, int DV, int C, int BV,
                                        const int32_t* cu, int N, const int32_t* order, hipStream_t s,
                                        uint16_t* statesT = nullptr);

// bf16 state-only pass of the segment scan (recurrence_states.h): every
// sequence's N (state from zero, true values) into nout [N*H, DK, DV] and M
// (state from the identity, V = 0) into mout [N*H, DK, DK], fp32, in one
// pass; d_k in {64, 128}, d_v a multiple of 32, chunk 64.
bool recurrence_states_supported(int DK, int DV, int C);
hipError_t launch_recurrence_states_bf16(const uint16_t* k, const uint16_t* v, const uint16_t* tws, float* nout,
                                         float* mout, int B, int H, int64_t L, int DK, int DV, int C,
                                         const int32_t* cu, int N, hipStream_t s);
// The same pass as the backward's chunk-state run over a dense batch: the
// recurrence from s0 (NULL: zeros), writing the bf16 state at the start of
// every chunk transposed, statesT [B*H*NC][DV][DK]; same shapes.
hipError_t launch_chunk_states_t_bf16(const uint16_t* k, const uint16_t* v, const uint16_t* tws, const float* s0,
                                      uint16_t* statesT, int B, int H, int64_t L, int DK, int DV, int C,
                                      hipStream_t s);
// bf16 reverse pass of the backward (recurrence_reverse.h): dS at the end of
// every chunk, transposed, dstatesT [B*H*NC][DV][DK], and ds0 (fp32
// [B*H][DK][DV]) from dsf (same layout, NULL: zero), given the effective
// queries qe [B*H*NC][C][DK] of the backward UT instance; d_k 64 or 128,
// chunk 64, d_v a multiple of 32.
bool reverse_states_supported(int DK, int DV, int C);
hipError_t launch_reverse_states_bf16(const uint16_t* k, const uint16_t* qe, const uint16_t* tws,
                                      const uint16_t* dout, const float* dsf, float* ds0, uint16_t* dstatesT, int B,
                                      int H, int64_t L, int DK, int DV, int C, hipStream_t s);

// bf16 UT transform with one wavefront per chunk (ut_wave.h); d_k in
// {32, 64, 128}, chunk in {32, 64}.
bool ut_wave_bf16_supported(int DK, int C);
hipError_t launch_ut_wave_bf16(const uint16_t* k, const uint16_t* beta, uint16_t* tws, int B, int H, int64_t L,
                               int DK, int C, int rule, const int32_t* cu, int N, hipStream_t s,
                               int32_t* order = nullptr);
// The per-chunk backward kernel in two-workgroup form (bwd_chunk_tr.h): states
// and dstates transposed ([B*H*NC][DV][DK]); d_k 64 or 128, chunk 64, d_v a
// multiple of 32.  Arguments as the chunk kernels of bwd.hip.
bool bwd_chunk_tr_bf16_supported(int DK, int DV, int C);
hipError_t launch_bwd_chunk_tr_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* beta,
                                    const uint16_t* dout, const uint16_t* tws, const float* xws, const float* aws,
                                    const uint16_t* pws, const uint16_t* statesT, const uint16_t* dstatesT,
                                    uint16_t* dq, uint16_t* dk, uint16_t* dv, uint16_t* dbeta, int B, int H, int64_t L,
                                    int DK, int DV, int C, int rule, hipStream_t s);
// Its backward instance over a dense batch: T, X (fp32), a (fp32) and P
// (bf16, packed at the start of pws) of every chunk slot, and with qe the
// chunk's Q - P T K (bf16 [slots][C][DK]); same shapes.  t_plain: T with
// ordinary stores, for a forward recurrence that reads it next.
hipError_t launch_ut_wave_bwd_bf16(const uint16_t* k, const uint16_t* beta, const uint16_t* q, uint16_t* tws,
                                   float* xws, float* aws, float* pws, uint16_t* qe, int B, int H, int64_t L, int DK,
                                   int C, int rule, hipStream_t s, bool t_plain = false);

// Backward pass of the chunked forward (bwd.hip, bwd_kernels.h): dense
// batches, any supported d_k / d_v / chunk; ws holds bwd_layout(...).total bytes.
// saved: the forward pass stored the chunk start states in ws (region s,
// transposed); used where the bf16 matrix-core kernels run, else recomputed.
struct BwdLayout {
  size_t t, x, p, a, s, ds, qe, total;  // byte offsets of the workspace regions, and the size
};
BwdLayout bwd_layout(int B, int H, int64_t L, int DK, int DV, int C, size_t esz);
template <typename T>
hipError_t launch_chunk_bwd(const T* q, const T* k, const T* v, const T* beta, const float* s0, const T* dout,
                            const float* dsf, T* dq, T* dk, T* dv, T* dbeta, float* ds0, int B, int H, int64_t L,
                            int DK, int DV, int C, int rule, void* ws, hipStream_t s, bool saved = false);
// bf16 shapes whose training forward stores the chunk start states (the split
// recurrence with value blocks of 32, and the bf16 backward kernels)
bool train_saves_states(int DK, int DV, int C);

// Segment scan (seg.hip): offsets of the packed view of B sequences of L
// tokens cut into G segments of Ls tokens, and the combine along each sequence.
hipError_t launch_seg_offsets(int32_t* cu, int B, int G, int64_t L, int64_t Ls, hipStream_t s);
hipError_t launch_seg_combine(const float* M, const float* N, const float* s0, float* sin, float* sfin, int B, int H,
                              int G, int DK, int DV, hipStream_t s);

}  // namespace efla
