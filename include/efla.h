/*
 * efla.h -- C ABI of the MI355X (gfx950) Exact Flow Linear Attention library.
 *
 * The method ("Exact Flow Linear Attention: Exact Solution from Continuous-Time
 * Dynamics", gist.science summary pages, Method steps 2-3): per (batch, head)
 * sequence, with lambda_t = ||k_t||^2 and
 *     alpha_t = (1 - exp(-beta_t * lambda_t)) / lambda_t,
 * the associative state S (d_k x d_v) evolves as
 *     S_t = (I - alpha_t k_t k_t^T) S_{t-1} + alpha_t k_t v_t^T
 * and the output is read out after each update as o_t = S_t^T q_t.
 * The pages note that the update keeps the rank-1 structure of the delta rule,
 * so the WY/UT chunkwise-parallel scheme applies (Method step 3); the chunked
 * entry points below compute exactly that recurrence, chunk by chunk.
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and keeps no mutable global state; calls on different
 *     streams with disjoint outputs may run concurrently.  The one exception
 *     is efla_chunk_fwd_noalloc, whose fixed scratch array (one per GPU) is
 *     shared by all its calls on that GPU.
 *   - Layouts are dense row-major:
 *         q, k   [B, L, H, d_k]       v, o   [B, L, H, d_v]       beta [B, L, H]
 *         state  [B, H, d_k, d_v]  (float32; S[i][j], i = key dim, j = value dim)
 *     Decode uses the same layouts with L = 1 folded away: q, k [N, H, d_k],
 *     v, o [N, H, d_v], beta [N, H], state [N, H, d_k, d_v].
 *   - dtype selects the element type of q, k, v, beta and o (float32 or
 *     bfloat16).  States are always float32; arithmetic is float32 (bf16 inputs
 *     feed bf16 matrix-core products with float32 accumulation).
 *   - Supported sizes: d_k, d_v in {16, 32, 64, 128}; chunk in {16, 32, 64};
 *     any L >= 0 (a ragged last chunk is handled); B, H >= 1 with B*H < 2^31.
 *   - stream is a hipStream_t passed as void* (NULL = default stream).  Calls are
 *     asynchronous: EFLA_OK means the work was enqueued.
 *   - q, k, v, o (chunked), the workspace and decode states must be 16-byte aligned (torch
 *     allocations are); a misaligned pointer is EFLA_ERR_INVALID_ARG.
 *   - Errors: arguments are validated before anything is launched; on a
 *     validation error nothing is written.  A failed launch returns
 *     EFLA_ERR_HIP; outputs are then undefined.  NaN/Inf inputs are not checked
 *     and propagate.
 */
#ifndef EFLA_H
#define EFLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum efla_status {
    EFLA_OK = 0,
    EFLA_ERR_INVALID_ARG = 1, /* null pointer, negative size, bad enum       */
    EFLA_ERR_UNSUPPORTED = 2, /* d_k / d_v / chunk outside the supported set  */
    EFLA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
    EFLA_ERR_HIP = 4,         /* a HIP launch or runtime call failed          */
    EFLA_ERR_SCRATCH = 5      /* efla_chunk_fwd_noalloc: problem exceeds the  */
                              /* library's fixed scratch                      */
} efla_status;

typedef enum efla_dtype {
    EFLA_F32 = 0,  /* float32 q, k, v, beta, o */
    EFLA_BF16 = 1  /* bfloat16 q, k, v, beta, o */
} efla_dtype;

/*
 * The update rule.  EFLA_RULE_EXACT is the exact flow of Method step 3
 * (alpha_t = (1 - exp(-beta_t lambda_t)) / lambda_t); every entry point without
 * a rule argument uses it.  EFLA_RULE_EULER is one explicit Euler step of
 * length beta_t of the same ODE, which the pages identify with the delta rule
 * of DeltaNet (Problem statement; Key Contributions 1): alpha_t = beta_t, so
 *     S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T.
 * Both rules share the chunked algebra and every kernel except where alpha is
 * formed; the _rule entry points below exist to run and time the two side by
 * side (Experimental Results: EFLA's training throughput matches DeltaNet's).
 */
typedef enum efla_rule {
    EFLA_RULE_EXACT = 0,
    EFLA_RULE_EULER = 1
} efla_rule;

/* Human-readable name of a status code (static string, never NULL). */
const char *efla_status_string(efla_status s);

/*
 * Base name of the GPU kernel that efla_chunk_recurrence (and the second
 * stage of efla_chunk_fwd) launches for these sizes, as a profiler lists it
 * (e.g. "recurrence_roles_kernel"); "unsupported" for sizes outside the
 * supported set.  Static string, never NULL; launches nothing.  For profiling
 * and roofline accounting only.
 */
const char *efla_chunk_recurrence_kernel(int d_k, int d_v, int chunk, efla_dtype dtype);

/*
 * efla_coeff -- the coefficient of Method step 3 for n_tok key rows.
 *   k      [n_tok, d_k] (dtype), beta [n_tok] (dtype)
 *   lambda [n_tok] float32 out, may be NULL: lambda_t = ||k_t||^2
 *   alpha  [n_tok] float32 out: alpha_t = (1 - exp(-beta_t lambda_t)) / lambda_t,
 *          evaluated as beta_t * (-expm1(-x)/x), x = beta_t * lambda_t, which is
 *          beta_t when x == 0 (lambda -> 0 limit) and 1/lambda_t when x == +inf.
 * n_tok may be 0 (nothing is launched).
 */
efla_status efla_coeff(const void *k, const void *beta, float *lambda, float *alpha,
                       int64_t n_tok, int d_k, efla_dtype dtype, void *stream);
/* efla_coeff under a given rule (EFLA_RULE_EULER: alpha = beta; lambda as above).
 * An invalid rule is EFLA_ERR_INVALID_ARG. */
efla_status efla_coeff_rule(const void *k, const void *beta, float *lambda, float *alpha,
                            int64_t n_tok, int d_k, efla_dtype dtype, efla_rule rule,
                            void *stream);

/*
 * Bytes of device workspace efla_chunk_fwd needs (0 if L == 0).  The workspace
 * holds, per (b, h, chunk), the chunk's UT-transform matrix
 * T = (I + tril(diag(alpha) K K^T, -1))^{-1} diag(alpha)  (chunk x chunk, dtype).
 * Returns 0 for unsupported arguments.
 */
size_t efla_chunk_fwd_workspace_size(int B, int H, int64_t L, int d_k, int d_v,
                                     int chunk, efla_dtype dtype);

/*
 * efla_chunk_fwd -- chunkwise-parallel EFLA forward pass (Method step 3 and the
 * WY/UT chunked scheme it refers to).  For every (b, h):
 *     S = s0[b, h] (or zeros if s0 == NULL)
 *     for t = 0 .. L-1:  S = (I - alpha_t k_t k_t^T) S + alpha_t k_t v_t^T;
 *                        o[b, t, h] = S^T q_t
 *     s_final[b, h] = S     (skipped if s_final == NULL; may alias s0)
 * computed chunk by chunk: per chunk of C tokens with start state S,
 *     T  = (I + tril(diag(alpha) K K^T, -1))^{-1} diag(alpha)
 *     U' = T (V - K S);   O = Q S + tril(Q K^T) U';   S <- S + K^T U'.
 * q, k, v, beta, o in dtype; s0, s_final float32.  workspace must hold
 * efla_chunk_fwd_workspace_size(...) bytes, 16-byte aligned.  o must not
 * alias any input.
 */
efla_status efla_chunk_fwd(const void *q, const void *k, const void *v, const void *beta,
                           const float *s0, void *o, float *s_final,
                           int B, int H, int64_t L, int d_k, int d_v, int chunk,
                           efla_dtype dtype, void *workspace, size_t workspace_bytes,
                           void *stream);
/* efla_chunk_fwd under a given rule (alpha per efla_rule); same workspace. */
efla_status efla_chunk_fwd_rule(const void *q, const void *k, const void *v, const void *beta,
                                const float *s0, void *o, float *s_final,
                                int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                efla_dtype dtype, efla_rule rule, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * efla_chunk_fwd_noalloc -- efla_chunk_fwd_rule with no workspace argument,
 * for callers that cannot allocate device memory around the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It calls no hipMalloc, hipFree or other allocating routine.  The per-chunk T
 * matrices go to a fixed device array of EFLA_NOALLOC_SCRATCH_BYTES (64 MiB)
 * inside the library, one copy per GPU, which each GPU holds from the time
 * the library's code is loaded on it until the process ends; the first call
 * on a device looks up that copy's address (with the device current) and
 * keeps it.  Sizes whose efla_chunk_fwd_workspace_size(...) exceeds the array
 * return EFLA_ERR_SCRATCH before anything is launched (B*H*ceil(L/chunk)
 * chunks of chunk x chunk elements: 8192 chunks of 64 x 64 in bf16, e.g. the
 * B=4, H=16, L=4096 layer twice over).  Every call on one GPU uses the same
 * array and leaves its contents behind: calls that overlap in time on one GPU
 * (on different streams, or from different threads) race and give undefined
 * results -- serialize them.  Nothing in the array needs to start at zero:
 * each call writes every scratch byte it reads.  Other arguments, errors and
 * results as for efla_chunk_fwd_rule.
 */
#define EFLA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
efla_status efla_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *beta,
                                   const float *s0, void *o, float *s_final,
                                   int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                   efla_dtype dtype, efla_rule rule, void *stream);

/*
 * The two stages of efla_chunk_fwd, exposed so that each can be checked and
 * timed on its own.  Calling efla_chunk_ut_transform then efla_chunk_recurrence
 * on the same stream with the same workspace is exactly efla_chunk_fwd.
 *
 * efla_chunk_ut_transform -- per (b, h, chunk): alpha from k and beta (as
 * efla_coeff), then the chunk's T (definition above) written to the workspace
 * as [B, H, ceil(L/chunk), chunk, chunk] row-major in dtype; entries above the
 * diagonal and rows/columns of tokens past L are zero.
 */
efla_status efla_chunk_ut_transform(const void *k, const void *beta, int B, int H, int64_t L,
                                    int d_k, int chunk, efla_dtype dtype, void *workspace,
                                    size_t workspace_bytes, void *stream);
/* efla_chunk_ut_transform under a given rule (the recurrence stage has none). */
efla_status efla_chunk_ut_transform_rule(const void *k, const void *beta, int B, int H, int64_t L,
                                         int d_k, int chunk, efla_dtype dtype, efla_rule rule,
                                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * efla_chunk_recurrence -- the sequential pass over chunks of every (b, h):
 * U' = T (V - K S), O = Q S + tril(Q K^T) U', S <- S + K^T U', reading T from
 * a workspace filled by efla_chunk_ut_transform with the same sizes.
 */
efla_status efla_chunk_recurrence(const void *q, const void *k, const void *v,
                                  const float *s0, void *o, float *s_final,
                                  int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                  efla_dtype dtype, const void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * efla_chunk_bwd -- gradients through efla_chunk_fwd (same q, k, v, beta, s0,
 * sizes and rule).  The pages give the forward recurrence only (Method step
 * 3); the backward pass is its reverse-mode derivative.  For a scalar loss with
 *     d_o      [B, L, H, d_v] (dtype)     = dLoss / do
 *     ds_final [B, H, d_k, d_v] float32   = dLoss / dS_L  (NULL: zero)
 * it writes dq, dk [B, L, H, d_k], dv [B, L, H, d_v], dbeta [B, L, H] (dtype)
 * and ds0 [B, H, d_k, d_v] float32 = dLoss / ds0 (NULL: not written).  dbeta
 * and dk include the paths through alpha(beta, lambda) and lambda = ||k||^2.
 * float32 inputs: float32 arithmetic throughout.  bf16 inputs (d_k, chunk
 * and d_v multiples of 32): products on bf16 matrix cores with float32
 * accumulation, each intermediate operand (P, the states, dS, the per-chunk
 * products) rounded to bf16 once, the UT-transform part and the coefficient
 * gradients in float32 (other bf16 shapes: float32 arithmetic on the widened
 * values); gradients are rounded to dtype on output.  The
 * workspace (size below) holds per chunk the UT-transform quantities, the
 * states the pass recomputes and their gradients (bf16: also the chunk's
 * Q - P T K, with P = tril(Q K^T) and T the UT transform, through which the
 * reverse pass over the chunks reads d_o); it is scratch and may be reused
 * once the call has completed on the stream.
 * q, k, v, d_o and the workspace must be 16-byte aligned.
 */
size_t efla_chunk_bwd_workspace_size(int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                     efla_dtype dtype);
efla_status efla_chunk_bwd(const void *q, const void *k, const void *v, const void *beta,
                           const float *s0, const void *d_o, const float *ds_final, void *dq,
                           void *dk, void *dv, void *dbeta, float *ds0, int B, int H, int64_t L,
                           int d_k, int d_v, int chunk, efla_dtype dtype, efla_rule rule,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training pair: a forward pass that keeps in the workspace what the backward
 * pass would otherwise recompute, and that backward pass.  Same operation,
 * arguments, layouts and results as efla_chunk_fwd_rule and efla_chunk_bwd
 * (Method step 3 and its reverse-mode derivative); the workspace is the one
 * of efla_chunk_bwd_workspace_size(...) (caller-owned, 16-byte aligned), and
 * must pass unchanged from efla_chunk_fwd_train to efla_chunk_bwd_train with
 * the same q, k, v, beta, s0, sizes, dtype and rule, on the same stream (or
 * ordered after it).  Where efla_chunk_train_saves_states(...) is 1 (bf16,
 * d_k 64 or 128, d_v a multiple of 32, chunk 64), the forward pass stores
 * there every chunk's UT-transform quantities (T, X, a, P and Q - P T K, as
 * the backward pass forms them) and its start state (as the bf16 values the
 * forward products use), and the backward pass reads them instead of running
 * the UT transform and the forward recurrence a second time; elsewhere the
 * pair behaves as efla_chunk_fwd_rule followed by efla_chunk_bwd.  o and
 * s_final are bitwise those of efla_chunk_fwd_rule.
 * Errors as for those two calls; a workspace written by anything else in
 * between gives wrong gradients, not an error.
 */
int efla_chunk_train_saves_states(int d_k, int d_v, int chunk, efla_dtype dtype);
efla_status efla_chunk_fwd_train(const void *q, const void *k, const void *v, const void *beta,
                                 const float *s0, void *o, float *s_final, int B, int H, int64_t L,
                                 int d_k, int d_v, int chunk, efla_dtype dtype, efla_rule rule,
                                 void *workspace, size_t workspace_bytes, void *stream);
efla_status efla_chunk_bwd_train(const void *q, const void *k, const void *v, const void *beta,
                                 const float *s0, const void *d_o, const float *ds_final, void *dq,
                                 void *dk, void *dv, void *dbeta, float *ds0, int B, int H, int64_t L,
                                 int d_k, int d_v, int chunk, efla_dtype dtype, efla_rule rule,
                                 void *workspace, size_t workspace_bytes, void *stream);

/*
 * Variable-length batches.  N sequences of different lengths packed along one
 * token axis, as a training or serving batch without padding holds them:
 *     q, k [T, H, d_k]   v, o [T, H, d_v]   beta [T, H]   (dtype)
 *     cu_seqlens [N + 1] int32, DEVICE memory: sequence i is tokens
 *         cu_seqlens[i] .. cu_seqlens[i+1] - 1 (nondecreasing, cu_seqlens[0] >= 0,
 *         cu_seqlens[N] <= T; lengths may be 0 or ragged)
 *     s0, s_final [N, H, d_k, d_v] float32 (each nullable, as in efla_chunk_fwd)
 * Every sequence runs the recurrence of efla_chunk_fwd on its own, from its own
 * initial state (Method step 3 per sequence).  Tokens outside every sequence
 * are not written.  The offsets are read on the device, so the library cannot
 * check them: offsets that break the rules above give unspecified numbers,
 * though every access stays inside the T tokens and the workspace (offsets
 * are clamped into [0, T]).  T < 2^31.
 *
 * efla_chunk_fwd_varlen_workspace_size -- bytes of workspace for these sizes:
 * H * (floor(T / chunk) + N) chunk slots of chunk x chunk (dtype), rounded up
 * to 256 bytes, then N int32 (the schedule below), rounded up to 256 bytes;
 * 0 for unsupported or invalid arguments (N < 1 included).
 *
 * Schedule: with N <= 4096, the UT-transform launch also ranks the
 * sequences by chunk count, longest first (ties by index), and the recurrence
 * hands them to its workgroups in that order, so the longest chains start
 * first.  The order
 * only changes which workgroup runs a sequence, never its arithmetic: results
 * are the same bits either way.
 */
size_t efla_chunk_fwd_varlen_workspace_size(int N, int H, int64_t T, int d_k, int d_v, int chunk,
                                            efla_dtype dtype);
/* efla_chunk_fwd_varlen -- the chunked forward pass over a packed batch (see
 * above), under a given rule.  N == 0 launches nothing; T == 0 only copies s0
 * (or zeros) into s_final.  Workspace, alignment and error rules as for
 * efla_chunk_fwd. */
efla_status efla_chunk_fwd_varlen(const void *q, const void *k, const void *v, const void *beta,
                                  const int32_t *cu_seqlens, int N, const float *s0, void *o,
                                  float *s_final, int H, int64_t T, int d_k, int d_v, int chunk,
                                  efla_dtype dtype, efla_rule rule, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * efla_chunk_fwd_segmented -- efla_chunk_fwd for batches of few, long
 * sequences: each sequence is cut into `segments` runs of whole chunks that
 * proceed in parallel.  The update is affine in the state (Method step 3), so
 * a run maps its incoming state S to M S + N, with M the product of the
 * chunks' (I - K^T T K) and N the state the run reaches from zero.  The call
 * computes every run's N and M (two passes over the segments in parallel),
 * chains the incoming states along each sequence, then reruns every segment
 * from its incoming state with output: three passes of the work over
 * `segments` times as many workgroups, a gain where B * H * d_v / 32 is well
 * below the GPU's 256 compute units.  Results equal efla_chunk_fwd's up to
 * rounding.  Arguments as for efla_chunk_fwd_rule, plus segments >= 1 (more
 * than the sequence's chunks is clamped); B * L < 2^31.
 */
size_t efla_chunk_fwd_segmented_workspace_size(int B, int H, int64_t L, int d_k, int d_v, int chunk,
                                               int segments, efla_dtype dtype);
efla_status efla_chunk_fwd_segmented(const void *q, const void *k, const void *v, const void *beta,
                                     const float *s0, void *o, float *s_final, int B, int H, int64_t L,
                                     int d_k, int d_v, int chunk, int segments, efla_dtype dtype,
                                     efla_rule rule, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * efla_step -- one decode step: a single token per (n, h) applied in place
 * (Method step 3):
 *     state[n, h] = (I - alpha k k^T) state[n, h] + alpha k v^T
 *     o[n, h]     = state[n, h]^T q        (post-update readout)
 * q, k [N, H, d_k], v, o [N, H, d_v], beta [N, H] in dtype; state [N, H, d_k, d_v]
 * float32, read and written once.  N*H may be 0.
 */
efla_status efla_step(const void *q, const void *k, const void *v, const void *beta,
                      float *state, void *o, int N, int H, int d_k, int d_v,
                      efla_dtype dtype, void *stream);
/* efla_step under a given rule. */
efla_status efla_step_rule(const void *q, const void *k, const void *v, const void *beta,
                           float *state, void *o, int N, int H, int d_k, int d_v,
                           efla_dtype dtype, efla_rule rule, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* EFLA_H */
