// api.hip -- the C ABI of libefla (declared in include/efla.h): argument
// validation, workspace sizing, choice of kernel instance, launches on the
// caller's stream.  Nothing here allocates device memory or synchronizes.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "efla.h"
#include "launchers.h"

namespace {

bool valid_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool valid_chunk(int c) { return c == 16 || c == 32 || c == 64; }
bool valid_dtype(efla_dtype dt) { return dt == EFLA_F32 || dt == EFLA_BF16; }
bool valid_rule(efla_rule r) { return r == EFLA_RULE_EXACT || r == EFLA_RULE_EULER; }
size_t elem_bytes(efla_dtype dt) { return dt == EFLA_BF16 ? 2 : 4; }
constexpr int64_t kMaxGrid = (int64_t(1) << 31) - 1;

efla_status from_hip(hipError_t e) { return e == hipSuccess ? EFLA_OK : EFLA_ERR_HIP; }

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Packed batches of at most this many sequences run longest first (the
// ordering kernel compares every pair of sequences).
constexpr int kMaxOrderedSeqs = 4096;

// The kernels move q, k, v, T and states with 16-byte vector accesses.
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by the chunked entry points (pointer checks are separate).
efla_status check_chunk_shape(int B, int H, int64_t L, int d_k, int d_v, int chunk, efla_dtype dt) {
  if (B < 1 || H < 1 || L < 0 || !valid_dtype(dt)) return EFLA_ERR_INVALID_ARG;
  if (!valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
  const int64_t bh = int64_t(B) * H;
  const int64_t nc = (L + chunk - 1) / chunk;
  if (bh * (d_v / 16) > kMaxGrid || bh * nc > kMaxGrid || nc > kMaxGrid) return EFLA_ERR_UNSUPPORTED;
  return EFLA_OK;
}

// Width of the value block one recurrence workgroup owns.  Wider blocks share
// each chunk's K/Q/T staging and P = tril(Q K^T) over more value columns.
// EFLA_VALUE_BLOCK (16, 32 or 64) overrides the choice for tuning; fp32 always
// uses 16.
int choose_value_block(efla_dtype dt, int d_v) {
  if (dt == EFLA_F32) return 16;
  if (const char* env = getenv("EFLA_VALUE_BLOCK")) {
    const int bv = atoi(env);
    if ((bv == 16 || bv == 32 || bv == 64) && bv <= d_v) return bv;
  }
  // Every 16 value columns of a (b, h) form one sequential chain whatever the
  // block width, so a wider block costs no parallelism; 32 columns (two chain
  // wavefronts) is the width the one-role-per-wavefront kernel is built for.
  return d_v >= 32 ? 32 : 16;
}

// Which recurrence kernel runs for given sizes.  bf16: the nine-wavefront
// split kernel (recurrence_split.h) where it applies, else one role per
// wavefront (recurrence_roles.h), else the generic kernel; fp32 always takes
// the generic kernel.  EFLA_RECURRENCE_IMPL=roles|tile|generic selects the
// role kernel, the one-wavefront-per-tile kernel (recurrence_tile.h) or the
// generic one for comparisons (falling through where the choice does not apply).
enum class Rec { kGeneric, kTile, kRoles, kSplit };
struct RecChoice {
  Rec kind;
  int bv;
};
RecChoice choose_recurrence(efla_dtype dt, int d_k, int d_v, int chunk) {
  const int bv = choose_value_block(dt, d_v);
  if (dt != EFLA_BF16) return {Rec::kGeneric, bv};
  const char* impl = getenv("EFLA_RECURRENCE_IMPL");
  const bool generic = impl && strcmp(impl, "generic") == 0, tile = impl && strcmp(impl, "tile") == 0;
  if (generic) return {Rec::kGeneric, bv};
  const bool roles = impl && strcmp(impl, "roles") == 0;
  if (!tile && !roles && efla::recurrence_split_supported(d_k, chunk, bv)) return {Rec::kSplit, bv};
  if (!tile && efla::recurrence_roles_supported(d_k, chunk, bv)) return {Rec::kRoles, bv};
  if (efla::recurrence_tile_supported(d_k, chunk, bv)) return {Rec::kTile, bv};
  return {Rec::kGeneric, bv};
}

// Stage 1 launch (arguments already validated).  Dense batch: cu == nullptr;
// packed batch: N sequences at device offsets cu into L tokens.
efla_status launch_ut(const void* k, const void* beta, int B, int H, int64_t L, int d_k, int chunk,
                      efla_dtype dtype, efla_rule rule, void* workspace, const int32_t* cu, int N,
                      hipStream_t s, int32_t* order = nullptr) {
  // bf16: one wavefront per chunk (ut_wave.h) where it applies, else one
  // workgroup per chunk; EFLA_UT_IMPL=workgroup pins the latter for comparisons.
  const char* impl = getenv("EFLA_UT_IMPL");
  const bool want_wg = impl && strcmp(impl, "workgroup") == 0;
  if (dtype == EFLA_BF16 && !want_wg && efla::ut_wave_bf16_supported(d_k, chunk))
    return from_hip(efla::launch_ut_wave_bf16(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(beta),
                                              static_cast<uint16_t*>(workspace), B, H, L, d_k, chunk,
                                              int(rule), cu, N, s, order));
  if (dtype == EFLA_BF16)
    return from_hip(efla::launch_ut_transform<uint16_t>(static_cast<const uint16_t*>(k),
                                                        static_cast<const uint16_t*>(beta),
                                                        static_cast<uint16_t*>(workspace), B, H, L, d_k,
                                                        chunk, int(rule), cu, N, s, order));
  return from_hip(efla::launch_ut_transform<float>(static_cast<const float*>(k),
                                                   static_cast<const float*>(beta),
                                                   static_cast<float*>(workspace), B, H, L, d_k, chunk,
                                                   int(rule), cu, N, s, order));
}

// Stage 2 launch (arguments already validated).  The one-wavefront-per-tile
// kernel takes dense batches only; packed batches use the role kernel there.
// trans: the chunk-transition run of the segment scan (V = 0, identity start,
// d_k value columns, final states only; v and d_v are ignored).
efla_status launch_rec(const void* q, const void* k, const void* v, const float* s0, void* o, float* s_final,
                       int B, int H, int64_t L, int d_k, int d_v, int chunk, efla_dtype dtype,
                       const void* workspace, const int32_t* cu, int N, hipStream_t s, bool trans = false,
                       const int32_t* order = nullptr) {
  if (trans) {
    v = k;
    d_v = d_k;
    o = nullptr;
    s0 = nullptr;
  }
  RecChoice rc = choose_recurrence(dtype, d_k, d_v, chunk);
  // the split kernel has the forward instance only; the tile kernel takes
  // dense forward passes only
  if ((rc.kind == Rec::kTile && cu != nullptr) || ((rc.kind == Rec::kTile || rc.kind == Rec::kSplit) &&
                                                   (trans || o == nullptr)))
    rc.kind = efla::recurrence_roles_supported(d_k, chunk, rc.bv) ? Rec::kRoles : Rec::kGeneric;
  if (dtype == EFLA_BF16) {
    const auto* qb = static_cast<const uint16_t*>(q);
    const auto* kb = static_cast<const uint16_t*>(k);
    const auto* vb = static_cast<const uint16_t*>(v);
    const auto* tb = static_cast<const uint16_t*>(workspace);
    auto* ob = static_cast<uint16_t*>(o);
    switch (rc.kind) {
      case Rec::kSplit:
        return from_hip(efla::launch_recurrence_split_bf16(qb, kb, vb, tb, s0, ob, s_final, B, H, L, d_k, d_v,
                                                           chunk, rc.bv, cu, N, order, s));
      case Rec::kRoles:
        return from_hip(efla::launch_recurrence_roles_bf16(qb, kb, vb, tb, s0, ob, s_final, B, H, L, d_k, d_v,
                                                           chunk, rc.bv, cu, N, s, nullptr, trans, order));
      case Rec::kTile:
        return from_hip(efla::launch_recurrence_tile_bf16(qb, kb, vb, tb, s0, ob, s_final, B, H, L, d_k, d_v,
                                                          chunk, rc.bv, s));
      case Rec::kGeneric:
        break;
    }
    return from_hip(efla::launch_recurrence<uint16_t>(qb, kb, vb, tb, s0, ob, s_final, B, H, L, d_k, d_v,
                                                      chunk, rc.bv, cu, N, s, int(trans), order));
  }
  return from_hip(efla::launch_recurrence<float>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(workspace), s0, static_cast<float*>(o), s_final, B, H, L, d_k, d_v, chunk,
      rc.bv, cu, N, s, int(trans), order));
}

// Fixed scratch of efla_chunk_fwd_noalloc: the per-chunk T matrices of one
// call.  Each GPU the library runs on holds its own copy from the time the
// code object is loaded there until the process ends.  In host code the name
// is only a stand-in; the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[EFLA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
efla_status scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EFLA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return EFLA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EFLA_OK;
}

}  // namespace

extern "C" {

const char* efla_status_string(efla_status s) {
  switch (s) {
    case EFLA_OK: return "EFLA_OK";
    case EFLA_ERR_INVALID_ARG: return "EFLA_ERR_INVALID_ARG: null pointer, negative size or bad enum";
    case EFLA_ERR_UNSUPPORTED: return "EFLA_ERR_UNSUPPORTED: d_k/d_v must be 16/32/64/128, chunk 16/32/64";
    case EFLA_ERR_WORKSPACE: return "EFLA_ERR_WORKSPACE: workspace missing or too small";
    case EFLA_ERR_HIP: return "EFLA_ERR_HIP: a HIP launch or runtime call failed";
    case EFLA_ERR_SCRATCH:
      return "EFLA_ERR_SCRATCH: the problem needs more than the library's fixed scratch (EFLA_NOALLOC_SCRATCH_BYTES)";
  }
  return "EFLA_ERR_UNKNOWN";
}

efla_status efla_coeff(const void* k, const void* beta, float* lambda, float* alpha, int64_t n_tok,
                       int d_k, efla_dtype dtype, void* stream) {
  return efla_coeff_rule(k, beta, lambda, alpha, n_tok, d_k, dtype, EFLA_RULE_EXACT, stream);
}

efla_status efla_coeff_rule(const void* k, const void* beta, float* lambda, float* alpha, int64_t n_tok,
                            int d_k, efla_dtype dtype, efla_rule rule, void* stream) {
  if (n_tok < 0 || !valid_dtype(dtype) || !valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  if (!valid_dim(d_k)) return EFLA_ERR_UNSUPPORTED;
  if (n_tok == 0) return EFLA_OK;
  if (k == nullptr || beta == nullptr || alpha == nullptr) return EFLA_ERR_INVALID_ARG;
  if ((n_tok + 255) / 256 > kMaxGrid) return EFLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == EFLA_BF16)
    return from_hip(efla::launch_coeff<uint16_t>(static_cast<const uint16_t*>(k),
                                                 static_cast<const uint16_t*>(beta), lambda, alpha,
                                                 n_tok, d_k, int(rule), s));
  return from_hip(efla::launch_coeff<float>(static_cast<const float*>(k), static_cast<const float*>(beta),
                                            lambda, alpha, n_tok, d_k, int(rule), s));
}

size_t efla_chunk_fwd_workspace_size(int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                     efla_dtype dtype) {
  if (check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype) != EFLA_OK) return 0;
  const int64_t nc = (L + chunk - 1) / chunk;
  return size_t(B) * size_t(H) * size_t(nc) * size_t(chunk) * size_t(chunk) * elem_bytes(dtype);
}

efla_status efla_chunk_ut_transform(const void* k, const void* beta, int B, int H, int64_t L, int d_k,
                                    int chunk, efla_dtype dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return efla_chunk_ut_transform_rule(k, beta, B, H, L, d_k, chunk, dtype, EFLA_RULE_EXACT, workspace,
                                      workspace_bytes, stream);
}

efla_status efla_chunk_ut_transform_rule(const void* k, const void* beta, int B, int H, int64_t L, int d_k,
                                         int chunk, efla_dtype dtype, efla_rule rule, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (!valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  const efla_status st = check_chunk_shape(B, H, L, d_k, 16, chunk, dtype);
  if (st != EFLA_OK) return st;
  if (L == 0) return EFLA_OK;
  if (k == nullptr || beta == nullptr || !aligned16(k)) return EFLA_ERR_INVALID_ARG;
  const size_t need = efla_chunk_fwd_workspace_size(B, H, L, d_k, 16, chunk, dtype);
  if (workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return EFLA_ERR_INVALID_ARG;
  return launch_ut(k, beta, B, H, L, d_k, chunk, dtype, rule, workspace, nullptr, 0,
                   static_cast<hipStream_t>(stream));
}

efla_status efla_chunk_recurrence(const void* q, const void* k, const void* v, const float* s0, void* o,
                                  float* s_final, int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                  efla_dtype dtype, const void* workspace, size_t workspace_bytes,
                                  void* stream) {
  const efla_status st = check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype);
  if (st != EFLA_OK) return st;
  if (L > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return EFLA_ERR_INVALID_ARG;
    const size_t need = efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype);
    if (workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return EFLA_ERR_INVALID_ARG;
  }
  if (L == 0 && s_final == nullptr) return EFLA_OK;
  return launch_rec(q, k, v, s0, o, s_final, B, H, L, d_k, d_v, chunk, dtype, workspace, nullptr, 0,
                    static_cast<hipStream_t>(stream));
}

const char* efla_chunk_recurrence_kernel(int d_k, int d_v, int chunk, efla_dtype dtype) {
  if (!valid_dtype(dtype) || !valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return "unsupported";
  switch (choose_recurrence(dtype, d_k, d_v, chunk).kind) {
    case Rec::kSplit: return "recurrence_split_kernel";
    case Rec::kRoles: return "recurrence_roles_kernel";
    case Rec::kTile: return "recurrence_tile_kernel";
    case Rec::kGeneric: break;
  }
  return "recurrence_kernel";
}

efla_status efla_chunk_fwd(const void* q, const void* k, const void* v, const void* beta, const float* s0,
                           void* o, float* s_final, int B, int H, int64_t L, int d_k, int d_v, int chunk,
                           efla_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return efla_chunk_fwd_rule(q, k, v, beta, s0, o, s_final, B, H, L, d_k, d_v, chunk, dtype, EFLA_RULE_EXACT,
                             workspace, workspace_bytes, stream);
}

efla_status efla_chunk_fwd_rule(const void* q, const void* k, const void* v, const void* beta,
                                const float* s0, void* o, float* s_final, int B, int H, int64_t L, int d_k,
                                int d_v, int chunk, efla_dtype dtype, efla_rule rule, void* workspace,
                                size_t workspace_bytes, void* stream) {
  if (!valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  const efla_status st = check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype);
  if (st != EFLA_OK) return st;
  if (L > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || o == nullptr)
      return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return EFLA_ERR_INVALID_ARG;
    const size_t need = efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype);
    if (workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
    const efla_status s1 = efla_chunk_ut_transform_rule(k, beta, B, H, L, d_k, chunk, dtype, rule, workspace,
                                                        workspace_bytes, stream);
    if (s1 != EFLA_OK) return s1;
  }
  return efla_chunk_recurrence(q, k, v, s0, o, s_final, B, H, L, d_k, d_v, chunk, dtype, workspace,
                               workspace_bytes, stream);
}

efla_status efla_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* beta,
                                   const float* s0, void* o, float* s_final, int B, int H, int64_t L, int d_k,
                                   int d_v, int chunk, efla_dtype dtype, efla_rule rule, void* stream) {
  if (!valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  const efla_status st = check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype);
  if (st != EFLA_OK) return st;
  const size_t need = efla_chunk_fwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype);
  if (need > EFLA_NOALLOC_SCRATCH_BYTES) return EFLA_ERR_SCRATCH;  // before any HIP call
  if (L > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || o == nullptr)
      return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return EFLA_ERR_INVALID_ARG;
  } else if (s_final == nullptr) {
    return EFLA_OK;
  }
  void* ws = nullptr;
  const efla_status sp = scratch_on_current_device(&ws);
  if (sp != EFLA_OK) return sp;
  // the same two launches as efla_chunk_fwd_rule, with the scratch as workspace
  return efla_chunk_fwd_rule(q, k, v, beta, s0, o, s_final, B, H, L, d_k, d_v, chunk, dtype, rule, ws,
                             EFLA_NOALLOC_SCRATCH_BYTES, stream);
}

efla_status efla_step(const void* q, const void* k, const void* v, const void* beta, float* state, void* o,
                      int N, int H, int d_k, int d_v, efla_dtype dtype, void* stream) {
  return efla_step_rule(q, k, v, beta, state, o, N, H, d_k, d_v, dtype, EFLA_RULE_EXACT, stream);
}

efla_status efla_step_rule(const void* q, const void* k, const void* v, const void* beta, float* state,
                           void* o, int N, int H, int d_k, int d_v, efla_dtype dtype, efla_rule rule,
                           void* stream) {
  if (N < 0 || H < 0 || !valid_dtype(dtype) || !valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  if (!valid_dim(d_k) || !valid_dim(d_v)) return EFLA_ERR_UNSUPPORTED;
  const int64_t units = int64_t(N) * H;
  if (units == 0) return EFLA_OK;
  if (units > kMaxGrid) return EFLA_ERR_UNSUPPORTED;
  if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || state == nullptr || o == nullptr)
    return EFLA_ERR_INVALID_ARG;
  if (!aligned16(state)) return EFLA_ERR_INVALID_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == EFLA_BF16)
    return from_hip(efla::launch_step<uint16_t>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
        static_cast<const uint16_t*>(beta), state, static_cast<uint16_t*>(o), units, d_k, d_v, int(rule), s));
  return from_hip(efla::launch_step<float>(static_cast<const float*>(q), static_cast<const float*>(k),
                                           static_cast<const float*>(v), static_cast<const float*>(beta),
                                           state, static_cast<float*>(o), units, d_k, d_v, int(rule), s));
}

}  // extern "C"

size_t efla_chunk_fwd_varlen_workspace_size(int N, int H, int64_t T, int d_k, int d_v, int chunk,
                                            efla_dtype dtype) {
  if (N < 1 || H < 1 || T < 0 || T > INT32_MAX || !valid_dtype(dtype)) return 0;
  if (!valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return 0;
  const int64_t slots = T / chunk + N;  // chunk slots per head
  if (int64_t(H) * slots > kMaxGrid) return 0;
  // T slots, then the schedule (int32 per sequence)
  return al256(size_t(H) * size_t(slots) * size_t(chunk) * size_t(chunk) * elem_bytes(dtype)) +
         al256(size_t(N) * 4);
}

efla_status efla_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* beta,
                                  const int32_t* cu_seqlens, int N, const float* s0, void* o, float* s_final,
                                  int H, int64_t T, int d_k, int d_v, int chunk, efla_dtype dtype,
                                  efla_rule rule, void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 0 || H < 1 || T < 0 || !valid_dtype(dtype) || !valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  if (!valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return EFLA_ERR_UNSUPPORTED;
  if (T > INT32_MAX) return EFLA_ERR_UNSUPPORTED;  // offsets are int32
  if (N == 0) return EFLA_OK;
  if (cu_seqlens == nullptr) return EFLA_ERR_INVALID_ARG;
  const int64_t slots = T / chunk + N;
  if (int64_t(N) * H * (d_v / 16) > kMaxGrid || int64_t(H) * slots > kMaxGrid) return EFLA_ERR_UNSUPPORTED;
  if (T > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || o == nullptr)
      return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return EFLA_ERR_INVALID_ARG;
    const size_t need = efla_chunk_fwd_varlen_workspace_size(N, H, T, d_k, d_v, chunk, dtype);
    if (workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return EFLA_ERR_INVALID_ARG;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* order = nullptr;
  if (T > 0) {
    if (N <= kMaxOrderedSeqs)  // the UT launch also ranks the sequences, longest first
      order = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) +
                                         al256(size_t(H) * size_t(slots) * size_t(chunk) * size_t(chunk) *
                                               elem_bytes(dtype)));
    const efla_status s1 = launch_ut(k, beta, 1, H, T, d_k, chunk, dtype, rule, workspace, cu_seqlens, N, s,
                                     order);
    if (s1 != EFLA_OK) return s1;
  } else if (s_final == nullptr) {
    return EFLA_OK;
  }
  return launch_rec(q, k, v, s0, o, s_final, 1, H, T, d_k, d_v, chunk, dtype, workspace, cu_seqlens, N, s, false,
                    order);
}

size_t efla_chunk_bwd_workspace_size(int B, int H, int64_t L, int d_k, int d_v, int chunk, efla_dtype dtype) {
  if (check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype) != EFLA_OK) return 0;
  if (L == 0) return 0;
  return efla::bwd_layout(B, H, L, d_k, d_v, chunk, elem_bytes(dtype)).total;
}

namespace {
efla_status chunk_bwd(const void* q, const void* k, const void* v, const void* beta, const float* s0,
                      const void* d_o, const float* ds_final, void* dq, void* dk, void* dv, void* dbeta, float* ds0,
                      int B, int H, int64_t L, int d_k, int d_v, int chunk, efla_dtype dtype, efla_rule rule,
                      void* workspace, size_t workspace_bytes, void* stream, bool saved) {
  if (!valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  const efla_status st = check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype);
  if (st != EFLA_OK) return st;
  if (L > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || d_o == nullptr || dq == nullptr ||
        dk == nullptr || dv == nullptr || dbeta == nullptr)
      return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(d_o)) return EFLA_ERR_INVALID_ARG;
    const size_t need = efla_chunk_bwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype);
    if (workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return EFLA_ERR_INVALID_ARG;
  } else if (ds0 == nullptr) {
    return EFLA_OK;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == EFLA_BF16) {
    using U = uint16_t;
    return from_hip(efla::launch_chunk_bwd<U>(
        static_cast<const U*>(q), static_cast<const U*>(k), static_cast<const U*>(v), static_cast<const U*>(beta),
        s0, static_cast<const U*>(d_o), ds_final, static_cast<U*>(dq), static_cast<U*>(dk), static_cast<U*>(dv),
        static_cast<U*>(dbeta), ds0, B, H, L, d_k, d_v, chunk, int(rule), workspace, s, saved));
  }
  return from_hip(efla::launch_chunk_bwd<float>(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(beta), s0, static_cast<const float*>(d_o), ds_final, static_cast<float*>(dq),
      static_cast<float*>(dk), static_cast<float*>(dv), static_cast<float*>(dbeta), ds0, B, H, L, d_k, d_v, chunk,
      int(rule), workspace, s));
}
}  // namespace

efla_status efla_chunk_bwd(const void* q, const void* k, const void* v, const void* beta, const float* s0,
                           const void* d_o, const float* ds_final, void* dq, void* dk, void* dv, void* dbeta,
                           float* ds0, int B, int H, int64_t L, int d_k, int d_v, int chunk, efla_dtype dtype,
                           efla_rule rule, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd(q, k, v, beta, s0, d_o, ds_final, dq, dk, dv, dbeta, ds0, B, H, L, d_k, d_v, chunk, dtype, rule,
                   workspace, workspace_bytes, stream, false);
}

int efla_chunk_train_saves_states(int d_k, int d_v, int chunk, efla_dtype dtype) {
  if (dtype != EFLA_BF16 || !valid_dim(d_k) || !valid_dim(d_v) || !valid_chunk(chunk)) return 0;
  return efla::train_saves_states(d_k, d_v, chunk) ? 1 : 0;
}

efla_status efla_chunk_fwd_train(const void* q, const void* k, const void* v, const void* beta, const float* s0,
                                 void* o, float* s_final, int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                 efla_dtype dtype, efla_rule rule, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  if (!valid_rule(rule)) return EFLA_ERR_INVALID_ARG;
  const efla_status st = check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype);
  if (st != EFLA_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (L > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || o == nullptr)
      return EFLA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return EFLA_ERR_INVALID_ARG;
    const size_t need = efla_chunk_bwd_workspace_size(B, H, L, d_k, d_v, chunk, dtype);
    if (workspace == nullptr || workspace_bytes < need) return EFLA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return EFLA_ERR_INVALID_ARG;
    if (efla_chunk_train_saves_states(d_k, d_v, chunk, dtype)) {
      // the backward's UT instance (T, and X, a, bf16 P and Qe for the
      // backward), then the recurrence storing the chunk start states, all
      // in the backward workspace's regions
      unsigned char* ws = static_cast<unsigned char*>(workspace);
      const efla::BwdLayout lay = efla::bwd_layout(B, H, L, d_k, d_v, chunk, 2);
      const auto* kb = static_cast<const uint16_t*>(k);
      auto* tws = reinterpret_cast<uint16_t*>(ws + lay.t);
      if (hipError_t e = efla::launch_ut_wave_bwd_bf16(
              kb, static_cast<const uint16_t*>(beta), static_cast<const uint16_t*>(q), tws,
              reinterpret_cast<float*>(ws + lay.x), reinterpret_cast<float*>(ws + lay.a),
              reinterpret_cast<float*>(ws + lay.p), reinterpret_cast<uint16_t*>(ws + lay.qe), B, H, L, d_k, chunk,
              int(rule), s, true);
          e != hipSuccess)
        return from_hip(e);
      return from_hip(efla::launch_recurrence_split_bf16(
          static_cast<const uint16_t*>(q), kb, static_cast<const uint16_t*>(v), tws, s0, static_cast<uint16_t*>(o),
          s_final, B, H, L, d_k, d_v, chunk, 32, nullptr, 0, nullptr, s, reinterpret_cast<uint16_t*>(ws + lay.s)));
    }
    // T at the workspace's start, where efla_chunk_fwd keeps it too
    const efla_status s1 = launch_ut(k, beta, B, H, L, d_k, chunk, dtype, rule, workspace, nullptr, 0, s);
    if (s1 != EFLA_OK) return s1;
  } else if (s_final == nullptr) {
    return EFLA_OK;
  }
  return launch_rec(q, k, v, s0, o, s_final, B, H, L, d_k, d_v, chunk, dtype, workspace, nullptr, 0, s);
}

efla_status efla_chunk_bwd_train(const void* q, const void* k, const void* v, const void* beta, const float* s0,
                                 const void* d_o, const float* ds_final, void* dq, void* dk, void* dv, void* dbeta,
                                 float* ds0, int B, int H, int64_t L, int d_k, int d_v, int chunk, efla_dtype dtype,
                                 efla_rule rule, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_bwd(q, k, v, beta, s0, d_o, ds_final, dq, dk, dv, dbeta, ds0, B, H, L, d_k, d_v, chunk, dtype, rule,
                   workspace, workspace_bytes, stream, efla_chunk_train_saves_states(d_k, d_v, chunk, dtype) != 0);
}

namespace {
// Layout of the segment scan's workspace (byte offsets, 256-aligned regions).
struct SegLayout {
  int G;        // segments per sequence actually used
  int64_t Ls;   // tokens per segment (a multiple of the chunk)
  size_t t, cu, m, n, sin, total;
};
// The state-only pass (N and M together) of the segment scan; EFLA_SEG_STATES=0
// selects the two separate passes of the general recurrence instead.
bool seg_states_fused(efla_dtype dtype, int d_k, int d_v, int chunk) {
  const char* env = getenv("EFLA_SEG_STATES");
  if (env != nullptr && env[0] == '0') return false;
  return dtype == EFLA_BF16 && efla::recurrence_states_supported(d_k, d_v, chunk);
}
SegLayout seg_layout(int B, int H, int64_t L, int d_k, int d_v, int chunk, int segments, efla_dtype dt) {
  SegLayout w{};
  const int64_t nc = (L + chunk - 1) / chunk;
  const int64_t per = (nc + segments - 1) / segments;  // chunks per segment
  w.Ls = per * chunk;
  w.G = int((L + w.Ls - 1) / w.Ls);
  const int64_t U = int64_t(B) * w.G;
  const int64_t slots = int64_t(H) * ((int64_t(B) * L) / chunk + U);
  w.t = 0;
  w.cu = al256(size_t(slots) * chunk * chunk * elem_bytes(dt));
  w.m = w.cu + al256(size_t(U + 1) * 4);
  w.n = w.m + al256(size_t(U) * H * d_k * d_k * 4);
  w.sin = w.n + al256(size_t(U) * H * d_k * d_v * 4);
  w.total = w.sin + al256(size_t(U) * H * d_k * d_v * 4);
  return w;
}
}  // namespace

size_t efla_chunk_fwd_segmented_workspace_size(int B, int H, int64_t L, int d_k, int d_v, int chunk, int segments,
                                               efla_dtype dtype) {
  if (segments < 1 || check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype) != EFLA_OK || L == 0) return 0;
  if (int64_t(B) * L > INT32_MAX) return 0;
  return seg_layout(B, H, L, d_k, d_v, chunk, segments, dtype).total;
}

efla_status efla_chunk_fwd_segmented(const void* q, const void* k, const void* v, const void* beta,
                                     const float* s0, void* o, float* s_final, int B, int H, int64_t L, int d_k,
                                     int d_v, int chunk, int segments, efla_dtype dtype, efla_rule rule,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_rule(rule) || segments < 1) return EFLA_ERR_INVALID_ARG;
  const efla_status st = check_chunk_shape(B, H, L, d_k, d_v, chunk, dtype);
  if (st != EFLA_OK) return st;
  if (int64_t(B) * L > INT32_MAX) return EFLA_ERR_UNSUPPORTED;  // offsets of the packed view are int32
  if (L == 0) return efla_chunk_fwd_rule(q, k, v, beta, s0, o, s_final, B, H, L, d_k, d_v, chunk, dtype, rule,
                                         nullptr, 0, stream);
  if (q == nullptr || k == nullptr || v == nullptr || beta == nullptr || o == nullptr) return EFLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return EFLA_ERR_INVALID_ARG;
  const SegLayout lay = seg_layout(B, H, L, d_k, d_v, chunk, segments, dtype);
  if (workspace == nullptr || workspace_bytes < lay.total) return EFLA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return EFLA_ERR_INVALID_ARG;
  const int64_t U = int64_t(B) * lay.G, T = int64_t(B) * L;
  if (U * H * (d_k / 16 > d_v / 16 ? d_k / 16 : d_v / 16) > kMaxGrid) return EFLA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto* ws = static_cast<unsigned char*>(workspace);
  void* tws = ws + lay.t;
  auto* cu = reinterpret_cast<int32_t*>(ws + lay.cu);
  auto* M = reinterpret_cast<float*>(ws + lay.m);
  auto* Nf = reinterpret_cast<float*>(ws + lay.n);
  auto* Sin = reinterpret_cast<float*>(ws + lay.sin);
  const int Ui = int(U);
  efla_status e = from_hip(efla::launch_seg_offsets(cu, B, lay.G, L, lay.Ls, s));
  // T of every chunk of every segment (the packed view of the batch)
  if (e == EFLA_OK) e = launch_ut(k, beta, 1, H, T, d_k, chunk, dtype, rule, tws, cu, Ui, s);
  // every segment from zero (N_g) and every segment's transition (M_g): in
  // one state-only pass where the kernel exists, else one pass each
  if (e == EFLA_OK && seg_states_fused(dtype, d_k, d_v, chunk)) {
    e = from_hip(efla::launch_recurrence_states_bf16(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                                     static_cast<const uint16_t*>(tws), Nf, M, 1, H, T, d_k, d_v,
                                                     chunk, cu, Ui, s));
  } else {
    if (e == EFLA_OK) e = launch_rec(q, k, v, nullptr, nullptr, Nf, 1, H, T, d_k, d_v, chunk, dtype, tws, cu, Ui, s);
    if (e == EFLA_OK)
      e = launch_rec(q, k, v, nullptr, nullptr, M, 1, H, T, d_k, d_v, chunk, dtype, tws, cu, Ui, s, true);
  }
  // incoming states along each sequence, and the final state
  if (e == EFLA_OK) e = from_hip(efla::launch_seg_combine(M, Nf, s0, Sin, s_final, B, H, lay.G, d_k, d_v, s));
  // every segment again from its incoming state, with output
  if (e == EFLA_OK) e = launch_rec(q, k, v, Sin, o, nullptr, 1, H, T, d_k, d_v, chunk, dtype, tws, cu, Ui, s);
  return e;
}
