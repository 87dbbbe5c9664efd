/*
 * efla.h - C ABI of the Exact Flow Linear Attention (EFLA) library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (Exact Flow Linear Attention summary page, sections 3.1-3.3;
 * the pages print no equation, this is the plain reading of what they state):
 * for every sequence and head, with a d_k x d_v state S starting at zero,
 *
 *   lambda_t = k_t . k_t                                  (key energy, section 3.4)
 *   alpha_t  = (1 - exp(-beta_t lambda_t)) / lambda_t      (alpha_t = beta_t if lambda_t = 0)
 *   S_t      = S_{t-1} + alpha_t k_t (v_t - S_{t-1}^T k_t)^T   (exact ZOH flow of
 *              dS/dtau = -k k^T S + k v^T over tau in [0, beta_t]; sections 3.1, 3.2)
 *   o_t      = scale * S_t^T q_t                           (read after the update)
 *
 * computed chunkwise (64 tokens) with the UT transform of section 3.3:
 *   T = (I + strictly_lower(diag(alpha) K K^T))^{-1} diag(alpha),  W = T K,  U = T V,
 *   U~ = U - W S,  O = scale (Q S + tril(Q K^T) U~),  S <- S + K^T U~.
 *
 * Conventions for every entry point:
 *  - Tensors are dense, contiguous, head-first: q, k [B,H,T,dk]; v, o, do [B,H,T,dv];
 *    beta [B,H,T]. They hold elements of the problem dtype (fp32 or bf16).
 *    Accumulation is always fp32.
 *  - Every data pointer is a DEVICE pointer, 16-byte aligned, owned by the caller.
 *    The library never allocates or frees device memory and never synchronises;
 *    it enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *  - All arguments are validated on the host before anything is enqueued. On an
 *    error nothing is launched and no output is written. A failed launch returns
 *    EFLA_ERR_HIP (outputs are then unspecified). No C++ exception crosses the ABI.
 *  - Packed batches: when `cu_seqlens` (device int32 [n_seqs+1]) is set, B must be 1,
 *    the T axis holds n_seqs sequences back to back, and the state restarts at every
 *    offset. Its contents must satisfy 0 = cu[0] <= cu[1] <= ... <= cu[n_seqs] = T;
 *    that is the caller's contract and is not checked (it lives on the device).
 *  - Supported: chunk = 64; dk, dv in {64, 128}; bf16 with any of those, fp32 with
 *    dk = dv = 64. Other sizes return EFLA_ERR_UNSUPPORTED.
 *  - Calls on different streams that share a workspace or saved buffer race.
 */
#ifndef EFLA_H
#define EFLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EFLA_ABI_VERSION 10

/* Size of the static device workspace of efla_fwd_noalloc (per GPU): 64 MiB. */
#define EFLA_NOALLOC_WS_BYTES (64ull << 20)

typedef enum {
  EFLA_OK = 0,
  EFLA_ERR_NULL = 1,        /* a required pointer is NULL */
  EFLA_ERR_SHAPE = 2,       /* inconsistent sizes (negative, B != 1 with cu_seqlens, ...) */
  EFLA_ERR_DTYPE = 3,       /* dtype is not EFLA_F32 / EFLA_BF16 */
  EFLA_ERR_UNSUPPORTED = 4, /* valid but not implemented (chunk != 64, head size, ...) */
  EFLA_ERR_WORKSPACE = 5,   /* workspace or saved buffer smaller than required */
  EFLA_ERR_HIP = 6,         /* a HIP launch failed */
  EFLA_ERR_ALIGN = 7        /* a data pointer is not 16-byte aligned */
} efla_status;

typedef enum { EFLA_F32 = 0, EFLA_BF16 = 1 } efla_dtype;

/* Step rule. EFLA_EXACT: alpha_t = (1 - exp(-beta_t lambda_t)) / lambda_t, the exact flow
 * (summary page, section 3.2). EFLA_EULER: alpha_t = beta_t, the delta rule, which is the
 * explicit Euler step of the same dynamics (summary page, section 2; DeltaNet page); it runs
 * through the same kernels and exists for comparisons. */
typedef enum { EFLA_EXACT = 0, EFLA_EULER = 1 } efla_mode;

typedef struct {
  int32_t B, H, T, dk, dv;      /* q,k: [B,H,T,dk]; v,o: [B,H,T,dv]; beta: [B,H,T] */
  int32_t dtype;                /* efla_dtype of q, k, v, beta, o, do and every gradient */
  int32_t chunk;                /* must be 64 */
  float scale;                  /* multiplies the read-out: o_t = scale * S_t^T q_t */
  const int32_t* cu_seqlens;    /* device pointer or NULL (see packed batches above) */
  int32_t n_seqs;               /* number of packed sequences when cu_seqlens is set */
  int32_t mode;                 /* efla_mode; other values return EFLA_ERR_UNSUPPORTED */
  int32_t segments;             /* state scans of long sequences (forward and backward),
                                   dense batches only (packed batches always use 1): 0 = chosen
                                   by the library, 1 = one sequential chain of chunks per
                                   sequence, n >= 2 = split each sequence into at most n
                                   segments scanned in parallel (segment-parallel scan, see
                                   efla_fwd and efla_bwd_state); < 0 = EFLA_ERR_SHAPE */
} efla_problem;

/* Byte offsets of the tensors inside the buffer that efla_fwd saves for efla_bwd.
 *   w      : fp32 problems: W = T K per chunk, [B,H,T,dk], fp32; bf16 problems: empty (the
 *            scans form U~ = X (diag(b) V - diag(alpha~) K S) and W^T dU~ = K^T diag(alpha~)
 *            X^T dU~ from X and coef instead)
 *   ut     : U~ = U - W S per chunk, [B,H,T,dv], problem dtype
 *   states : state entering each chunk, [n_chunk_slots][H][dk][dv], problem dtype;
 *            slot = b * ceil(T/64) + c (dense batch) or chunk_start[s] + c (packed),
 *            where chunk_start[s] = sum over earlier sequences of ceil(len/64)
 *   table  : chunk_start, int32 [n_seqs+1] (packed batches only, else unused)
 *   m      : tril(Q K^T) of each chunk, [n_chunk_slots][H][64][64], problem dtype (zero above
 *            the diagonal and in rows past the end of a sequence)
 *   x      : X = (I + strictly_lower(diag(alpha) K K^T))^{-1} of each chunk (so that
 *            T = X diag(alpha)), [n_chunk_slots][H][64][64], problem dtype
 *   coef   : bf16 problems only (empty for fp32): the per-token column scales of the chunk
 *            factors, fp32 [2][n_chunk_slots][H][64]: alpha~ = alpha (gated: alpha e^{c}),
 *            then b, the gated input coefficient (written by the gated forward only), so that
 *            W = X diag(alpha~) K and U = X diag(b) V (ungated b = alpha)
 *   cum    : gated forward only: running sums of the log-decays inside each chunk,
 *            fp32 [n_chunk_slots][H][64] (then w, m and x hold the decayed factors of
 *            efla_fwd_gated)
 *   segp   : segment-parallel plans only (empty otherwise): each segment's transition, the
 *            product of (I - K^T W) over its chunks (gated: with the decays), fp32
 *            [B * G][H][dk][dk]; the backward chains the state gradients with its transpose
 *   total  : size of the whole buffer = efla_saved_bytes()                               */
typedef struct {
  size_t w, ut, states, table, m, x, coef, cum, segp, total;
  int64_t n_chunk_slots;
} efla_saved_layout;

/* Library ABI version (EFLA_ABI_VERSION of the build). */
int efla_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* efla_status_str(efla_status s);

/* Validate a problem without launching anything. */
efla_status efla_check_problem(const efla_problem* p);

/* Device workspace that efla_fwd (for_backward = 0) or efla_bwd (for_backward = 1)
 * needs, in bytes; 0 if the problem is invalid. (Sizing queries of this library; no passage of
 * the pages defines them.) For efla_bwd the figure assumes
 * saved == NULL (recompute); with a saved buffer less is used, never more. */
size_t efla_workspace_bytes(const efla_problem* p, int for_backward);

/* Size of the forward->backward buffer (chunk factors and chunk states); 0 if invalid. */
size_t efla_saved_bytes(const efla_problem* p);

/* Offsets inside that buffer (see efla_saved_layout). */
efla_status efla_get_saved_layout(const efla_problem* p, efla_saved_layout* out);

/* Per-token coefficients of the exact flow (section 3.2: beta_t replaced by alpha_t;
 * section 3.4: lambda_t = ||k_t||^2 in the denominator). Reads k [B,H,T,dk] and
 * beta [B,H,T]; writes fp32 [B,H,T] arrays:
 *   lam = ||k||^2, alpha, dalpha_dbeta = exp(-beta lam), dalpha_dlam = beta^2 phi'(beta lam)
 * with phi(x) = (1 - e^-x)/x. `alpha` is required, the other outputs may be NULL.
 * cu_seqlens is ignored (the coefficients are per token). */
efla_status efla_prep(const efla_problem* p, const void* k, const void* beta, float* lam,
                      float* alpha, float* dalpha_dbeta, float* dalpha_dlam, void* stream);

/* UT transform of every chunk (section 3.3): W = T K, U = T V with
 * T = (I + strictly_lower(diag(alpha) K K^T))^{-1} diag(alpha), written in the problem
 * dtype as w [B,H,T,dk], u [B,H,T,dv]. Chunks start at every sequence start.
 * ws must hold efla_workspace_bytes(p, 0) bytes. */
efla_status efla_chunk_ut(const efla_problem* p, const void* k, const void* v, const void* beta,
                          void* w, void* u, void* ws, size_t ws_bytes, void* stream);

/* Forward: o [B,H,T,dv] (problem dtype). `saved` (NULL, or efla_saved_bytes(p) bytes)
 * receives U~, the chunk states, M, X and W (fp32) or the column scales (bf16) for efla_bwd.
 * ws: efla_workspace_bytes(p, 0).
 * Segment-parallel scan (summary page, section 3.3: from chunk to chunk the state follows an
 * affine map, S <- (I - K^T W) S + K^T U, so the maps of consecutive chunks compose): when
 * the plan splits sequences into G > 1 segments, every segment's composed transition P and
 * zero-start state R are formed in parallel (one launch), a short sequential pass chains them
 * (S_in of segment j+1 = P_j S_in_j + R_j, fp32), and the output scan runs over all segments
 * at once from those states. Same results up to rounding; the workspace grows by
 * 4 B G H dk (2 dv + dk) bytes, and a saved buffer keeps the P_j for the backward.
 * The library's choice (segments = 0) splits only when B * H * dv / 32 < 128 and a
 * sequence has at least 32 chunks, aiming at about 256 scan workgroups (one per compute unit)
 * and at least 16 chunks per segment. */
efla_status efla_fwd(const efla_problem* p, const void* q, const void* k, const void* v,
                     const void* beta, void* o, void* saved, size_t saved_bytes, void* ws,
                     size_t ws_bytes, void* stream);

/* Forward with recurrent state I/O. States are fp32 [n_state][H][dk][dv] with n_state = B
 * (dense) or n_seqs (packed), one per sequence: h0 (NULL = zero) is the state entering each
 * sequence, ht (NULL = not written) receives the state after its last token, so a long stream
 * can be processed in pieces (summary page, section 3.3: the chunk-level recurrence carries the
 * state from chunk to chunk). efla_fwd(...) is efla_fwd_state(..., NULL, o, NULL, ...). */
efla_status efla_fwd_state(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const float* h0, void* o, float* ht, void* saved,
                           size_t saved_bytes, void* ws, size_t ws_bytes, void* stream);

/* Forward for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. Same results as efla_fwd_state(p, q, k, v,
 * beta, h0, o, ht, NULL, 0, ws, ...) with no saved buffer, but it takes no workspace: it uses a
 * static device array of EFLA_NOALLOC_WS_BYTES inside the library, one per GPU, which each GPU
 * holds until the process ends. Problems whose efla_workspace_bytes(p, 0) exceeds that size
 * return EFLA_ERR_WORKSPACE before anything is enqueued (64 MiB holds, for example, 16 heads of
 * 16,384 bf16 tokens at d_k = d_v = 128, with the library's segment plan). It allocates nothing,
 * ever. Every call on a GPU uses that GPU's array and leaves its contents behind: calls that
 * overlap on one GPU (different streams or host threads) race; calls on one stream are ordered.
 * No part of the array has to start at zero. On the first call on a device the array's address is looked up
 * (hipGetSymbolAddress); EFLA_ERR_HIP if that fails. */
efla_status efla_fwd_noalloc(const efla_problem* p, const void* q, const void* k, const void* v,
                             const void* beta, const float* h0, void* o, float* ht, void* stream);

/* Gated EFLA forward (summary page, section 3.4 names it; the appendix applies the exact flow
 * to Gated DeltaNet; the pages print no formula, this is the reading taken): a per-token
 * log-decay a_t (gate, [B,H,T], problem dtype; a_t <= 0 decays; a_t > 0, growth, is computed
 * by the same formulas, unclipped) adds -a_t / beta_t times the
 * identity to the dynamics matrix over the step interval, and the exact flow is
 *   S_t = e^{a_t} (I - alpha_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T,
 *   alpha_t = beta_t phi(beta_t lambda_t),  b_t = beta_t phi(beta_t lambda_t - a_t),
 * phi(x) = (1 - e^{-x}) / x (mode EFLA_EULER: alpha_t = b_t = beta_t, the gated delta rule).
 * a = 0 gives efla_fwd_state. Computed chunkwise with the running log-decay sums c of each
 * chunk: A_ts = alpha_t e^{c_t - c_s} k_t . k_s, W = X diag(alpha e^c) K, U = X diag(b) V,
 * O = scale (diag(e^c) Q S + (tril(Q K^T) * e^{c_t - c_s}) U~),
 * S <- e^{c_last} S + K^T diag(e^{c_last - c}) U~. h0 / ht as in efla_fwd_state; segments as in
 * efla_fwd. `saved` (NULL, or efla_saved_bytes(p) bytes) receives the decayed factors, U~,
 * the chunk states and the running log-decay sums for efla_bwd_gated. bf16 problems only
 * (EFLA_ERR_UNSUPPORTED otherwise). ws: efla_workspace_bytes(p, 0). */
efla_status efla_fwd_gated(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const void* gate, const float* h0, void* o,
                           float* ht, void* saved, size_t saved_bytes, void* ws, size_t ws_bytes,
                           void* stream);

/* Backward of sum(o * d_o): dq, dk [B,H,T,dk], dv [B,H,T,dv], dbeta [B,H,T], all in
 * the problem dtype (every output fully overwritten). The pages print no backward; this is
 * reverse-mode differentiation of the chunk form (summary page, section 3.3: chunk-level
 * recurrence and UT transform) and of the exact-flow step (section 3.2: alpha_t replaces beta_t,
 * so dbeta = dalpha e^{-beta lambda} and the key energy adds 2 k dalpha beta^2 phi'(beta lambda),
 * phi(x) = (1 - e^{-x}) / x). `saved` is the buffer a forward
 * call on the same inputs filled, or NULL to recompute it inside ws.
 * ws: efla_workspace_bytes(p, 1). */
efla_status efla_bwd(const efla_problem* p, const void* q, const void* k, const void* v,
                     const void* beta, const void* d_o, const void* saved, size_t saved_bytes,
                     void* dq, void* dk, void* dv, void* dbeta, void* ws, size_t ws_bytes,
                     void* stream);

/* Backward with recurrent state I/O: the gradient of sum(o * d_o) + <ht, dht> with respect to
 * q, k, v, beta and h0. With a segment plan (efla_problem.segments) the reverse state-gradient
 * scan is segment-parallel like the forward's: going backwards a chunk maps the gradient
 * affinely, G <- (I - W^T K) G + scale (Q - M W)^T dO; over a segment these maps compose to the
 * transpose of the forward's segment transition P_j (saved by the forward, or recomputed with
 * it), so only each segment's zero-start gradient R is formed, in parallel; the segments are
 * chained from the last to the first with P_j^T, and the full scan then runs over all segments
 * from their incoming gradients. With a saved buffer the workspace then needs 8 B G H dk dv more
 * bytes (never more than efla_workspace_bytes(p, 1)). The saved buffer must come from a forward
 * call with the same problem, segment plan included. h0 must be what the forward used (only read when saved == NULL; NULL =
 * zero); dht (NULL = zero) is the gradient arriving at the final states; dh0 (NULL = not
 * written) receives the gradient at the initial states. fp32 [n_state][H][dk][dv] each. */
efla_status efla_bwd_state(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const float* h0, const void* d_o, const float* dht,
                           const void* saved, size_t saved_bytes, void* dq, void* dk, void* dv,
                           void* dbeta, float* dh0, void* ws, size_t ws_bytes, void* stream);

/* Backward of gated EFLA: the gradient of sum(o * d_o) + <ht, dht> with respect to q, k, v,
 * beta, the log-decays (dgate [B,H,T], problem dtype) and h0, for the forward of
 * efla_fwd_gated. Reverse mode of the chunk form given there: per chunk, with c its running
 * log-decay sums, Gamma = e^c, r = e^{c_last - c}, D_ts = e^{c_t - c_s}, P = tril(Q K^T) * D and
 * G the gradient of the state leaving the chunk,
 *   dU~ = scale P^T dO + diag(r) K G,  G_in = e^{c_last} G + scale Q^T diag(Gamma) dO - W^T dU~;
 * every factor e^{c} also contributes to dc, and dgate_t = sum over s >= t in the chunk of dc_s
 * plus db_t db_t/da_t. `saved` is the buffer efla_fwd_gated filled on the same inputs, or NULL to
 * recompute it inside ws (then h0 must be the forward's). Other arguments as efla_bwd_state.
 * bf16 problems only. ws: efla_workspace_bytes(p, 1). */
efla_status efla_bwd_gated(const efla_problem* p, const void* q, const void* k, const void* v,
                           const void* beta, const void* gate, const float* h0, const void* d_o,
                           const float* dht, const void* saved, size_t saved_bytes, void* dq,
                           void* dk, void* dv, void* dbeta, void* dgate, float* dh0, void* ws,
                           size_t ws_bytes, void* stream);

/* Recurrent inference: the token recurrence itself (summary page, section 3.2), one token
 * after the other, for dense batches (cu_seqlens must be NULL). Reads q, k [B,H,T,dk],
 * v [B,H,T,dv], beta [B,H,T] (problem dtype) and state, fp32 [B][H][dk][dv] in place: on
 * entry the state before the first token, on return the state after the last one. Writes
 * o [B,H,T,dv]. Meant for short T (decoding one or a few tokens per call); the chunked
 * efla_fwd_state is the fast path for long T. Needs no workspace. */
efla_status efla_decode(const efla_problem* p, const void* q, const void* k, const void* v,
                        const void* beta, float* state, void* o, void* stream);

/* Recurrent inference of gated EFLA (the recurrence of efla_fwd_gated, token by token), with
 * gate [B,H,T] in the problem dtype; otherwise as efla_decode. */
efla_status efla_decode_gated(const efla_problem* p, const void* q, const void* k,
                              const void* v, const void* beta, const void* gate, float* state,
                              void* o, void* stream);

/* Kernel timing for profiling. While enabled, every kernel that efla_* enqueues is
 * bracketed by two HIP events recorded on the same stream. efla_profile_read waits for
 * those events and reports, per kernel name, the launch count and summed milliseconds
 * since the last reset; it returns the number of kernels written (at most max_kernels).
 * names receives max_kernels NUL-terminated strings of name_stride bytes each.
 * Not thread-safe; meant for benchmarks. */
efla_status efla_profile_enable(int on);
int efla_profile_read(char* names, int name_stride, int64_t* counts, double* total_ms,
                      int max_kernels);
void efla_profile_reset(void);

#ifdef __cplusplus
}
#endif

#endif /* EFLA_H */
