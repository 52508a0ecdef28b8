/*
 * rsm.h -- C ABI of librsm.so: the Routing State Model (RSM) mixer of Raven on one
 * AMD Instinct MI355X (gfx950).
 *
 * Per head the mixer keeps a slot memory H of M slots x Dv columns.  For every token
 * it scores the M slots with a sigmoid of the router logits z, keeps the top K scores
 * (ties go to the lower slot index), decays and writes only those slots, and reads the
 * memory with the query (Raven README page, "How Raven Works" listing):
 *
 *     s      = TopK(sigmoid(z))                      (zeros outside the top K)
 *     alpha  = exp(s * f)                            (1, i.e. untouched, outside the top K)
 *     H[i,:] = alpha_i * H[i,:] + (1 - alpha_i) * k_i * v     for the selected slots i
 *     o      = q . H = sum_i q_i * H[i,:]            (read after the update)
 *
 * Unselected slots keep their exact bits (Raven paper summary, section 4.1 and appendix
 * A.7).  The chunked forward evaluates the same recurrence chunk by chunk (appendix
 * A.5: T split into chunks of length C) with per-slot cumulative log-decay taken from
 * the chunk start.
 *
 * Conventions shared by every entry point
 *  - Tensors are dense, contiguous, row-major device buffers in the shapes given.
 *    q, k, z are [.., M]; v is [.., Dv]; f is one fp32 scalar per token and head and
 *    must be <= 0 (-inf allowed: full overwrite of the selected slots).
 *  - dtype selects the element type of q, k, z, v: RSM_F32 (float) or RSM_BF16
 *    (bfloat16 bits).  f, states and outputs are always fp32.
 *  - The caller owns every buffer.  The library keeps no global mutable state and
 *    allocates no device memory; calls are asynchronous on `stream` (a hipStream_t,
 *    NULL = the default stream) and return after enqueueing.
 *  - Errors: argument errors return a negative rsm_status before anything is enqueued;
 *    a failed launch returns RSM_ERR_HIP.  Data values are not validated: f > 0, NaN or
 *    infinite z/q/k/v give unspecified results.
 *  - Supported shapes: M in {16, 32, 64, 128, 256}; Dv in {16, 32, 64, 128, 256};
 *    1 <= K <= M; chunk C in {16, 32, 64}; B, T, Hh >= 0 (T need not be a multiple of C;
 *    an empty call enqueues nothing except copying H0, or zeros, into H_out).
 */
#ifndef RSM_H
#define RSM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { RSM_F32 = 0, RSM_BF16 = 1 } rsm_dtype;

typedef enum {
    RSM_OK = 0,
    RSM_ERR_NULL = -1,        /* a required pointer is NULL */
    RSM_ERR_SHAPE = -2,       /* a size is negative or outside the supported set */
    RSM_ERR_K = -3,           /* K outside [1, M] */
    RSM_ERR_DTYPE = -4,       /* dtype is not RSM_F32 / RSM_BF16 */
    RSM_ERR_UNSUPPORTED = -5, /* a combination the library was not built for */
    RSM_ERR_WORKSPACE = -6,   /* workspace NULL or smaller than the queried size */
    RSM_ERR_HIP = -7,         /* the HIP runtime reported an error at launch */
    RSM_ERR_ALIAS = -8,       /* an output overlaps an input it must not overlap */
    RSM_ERR_TOO_LARGE = -9    /* the call needs more scratch than rsm_noalloc_scratch_bytes() */
} rsm_status;

/* Human-readable text of a status code (static storage, never NULL). */
const char* rsm_status_string(int status);

/* Version of this ABI (major*10000 + minor*100 + patch). */
int rsm_abi_version(void);

/*
 * Router: sigmoid scores, top K per token-head row (RSM router, "How Raven Works":
 * TopK(sigmoid(r_proj(x))); the logits z are taken as given).
 *   z     [B,T,Hh,M]  dtype          router logits
 *   idx   [B,T,Hh,K]  int32  out     selected slots, ascending slot order
 *   score [B,T,Hh,K]  fp32   out     sigmoid(z) at those slots; may be NULL
 * Ranking is on z (equivalent to ranking the exact sigmoid, which is strictly
 * increasing); equal logits (-0 == +0) go to the lower slot index.
 */
int rsm_route_topk(const void* z, int dtype, int64_t B, int64_t T, int64_t Hh, int64_t M,
                   int64_t K, int32_t* idx, float* score, void* stream);

/*
 * Bytes of device workspace rsm_forward_chunked needs for these sizes (0 if T == 0).
 * The workspace holds the route of every token-head, padded to whole chunks (a selection
 * bit mask, 8 bytes per 64 slots, and the K decay factors of the selected slots, fp32),
 * and, when few heads make the forward cut each sequence into S segments, the fp32 end
 * state (M x Dv) and decay product (M) of every segment but the last, per head, plus room
 * for a copy of H0 that an in-place call (H_out == H0) reads instead of H0.  With
 * M = 256 it holds the router's output instead: K slot indices (int32) and K weights (fp32)
 * per token-head.
 * Returns 0 for unsupported arguments as well; the forward call then reports the error.
 */
size_t rsm_forward_workspace_bytes(int dtype, int64_t B, int64_t T, int64_t Hh, int64_t M,
                                   int64_t Dv, int64_t C, int64_t K);

/*
 * Chunked forward over a whole sequence (RSM update and read of "How Raven Works",
 * evaluated chunkwise as in the Raven paper's appendix A.5).
 *   q, k, z  [B,T,Hh,M]   dtype
 *   v        [B,T,Hh,Dv]  dtype
 *   f        [B,T,Hh]     fp32, <= 0 (-inf allowed)
 *   H0       [B,Hh,M,Dv]  fp32 initial state, or NULL for a zero state
 *   o        [B,T,Hh,Dv]  fp32 out (must not overlap any input)
 *   H_out    [B,Hh,M,Dv]  fp32 out final state, or NULL; may be the same buffer as H0
 *   idx_out  [B,T,Hh,K]   int32 out selected slots (ascending), or NULL
 *   workspace/workspace_bytes: device scratch of at least
 *            rsm_forward_workspace_bytes(dtype, B, T, Hh, M, Dv, C, K) bytes (owned by the
 *            caller, contents undefined on entry and on return)
 * Slots never selected in the sequence come back in H_out bit-identical to H0.
 * C only sets how the work is cut: results agree across C up to rounding.  With M = 128
 * the kernels run C = 64 as chunks of 32 (their tiles would not fit in the 160 KB of LDS of
 * a compute unit).
 * Chunks whose decay over the chunk falls below 2^-100 for some slot (f = -inf, or very
 * strong decay) are evaluated token by token instead of in factored form.
 * With M = 256 (the pages' default slot count) the chunk tiles do not fit in LDS and the
 * call evaluates the recurrence token by token instead (the recurrent form the README
 * names for generation): the router over all rows, then one workgroup per head and column
 * tile that keeps its part of H in registers; C is then only validated.  T < 2^31.
 */
int rsm_forward_chunked(const void* q, const void* k, const void* z, const void* v, int dtype,
                        const float* f, const float* H0, int64_t B, int64_t T, int64_t Hh,
                        int64_t M, int64_t Dv, int64_t K, int64_t C, float* o, float* H_out,
                        int32_t* idx_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent step for B x Hh heads (fused route + update + read; the README's
 * "fused recurrent kernels for generation").
 *   q, k, z  [B,Hh,M]     dtype
 *   v        [B,Hh,Dv]    dtype
 *   f        [B,Hh]       fp32, <= 0 (-inf allowed)
 *   H        [B,Hh,M,Dv]  fp32 state, updated in place: only the K selected rows of
 *                         each head are written, every other row keeps its bits
 *   o        [B,Hh,Dv]    fp32 out, read after the update
 *   idx_out  [B,Hh,K]     int32 out selected slots (ascending), or NULL
 */
int rsm_decode_step(const void* q, const void* k, const void* z, const void* v, int dtype,
                    const float* f, float* H, int64_t B, int64_t Hh, int64_t M, int64_t Dv,
                    int64_t K, float* o, int32_t* idx_out, void* stream);

/*
 * Router and decay variants, each named on the pages.  The *_ex entry points take one;
 * NULL, or a zero-initialised struct, is the default router of the entry points above
 * (and runs the same kernels).
 *  - score = RSM_SCORE_SOFTMAX: softmax over all M logits instead of the sigmoid (README
 *    configuration table, "top-k sigmoid/softmax", and its router_score option; paper
 *    summary section 6.2.1).  The softmax increases with each logit, so the same K slots
 *    are selected; slot i takes exp(z_i - max z) / sum_j exp(z_j - max z).
 *  - normalize = 1: the selected scores are divided by their sum, which then is one (paper
 *    summary section 4.1).  A zero sum leaves them unchanged.
 *  - f_per_slot = 1: f holds one decay rate per slot, shape [.., M] instead of [..] (the
 *    GLA decay option of the README configuration table, a diagonal gate; paper summary
 *    section 2.1): alpha_i = exp(s_i * f_i).  Ignored by rsm_route_topk_ex.
 *  - noise != NULL: fp32 device buffer shaped like z, added to the logits before selection
 *    and scoring as an fp32 sum (Gumbel exploration noise during training, paper summary
 *    section 6.2.2; the caller draws it).  It must not overlap an output.
 * A field outside {0, 1} (score outside the enum) returns RSM_ERR_UNSUPPORTED.
 */
typedef enum { RSM_SCORE_SIGMOID = 0, RSM_SCORE_SOFTMAX = 1 } rsm_score_kind;

typedef struct {
    int score;          /* rsm_score_kind */
    int normalize;      /* 0 or 1 */
    int f_per_slot;     /* 0: f [.., 1 per token-head]; 1: f [.., M] */
    const float* noise; /* NULL or fp32 [.., M], device memory, read only */
} rsm_router_opts;

/* rsm_route_topk with a router variant; score (nullable) receives the routing weight of
 * each selected slot after the softmax / renormalisation. */
int rsm_route_topk_ex(const void* z, int dtype, const rsm_router_opts* opts, int64_t B, int64_t T,
                      int64_t Hh, int64_t M, int64_t K, int32_t* idx, float* score, void* stream);

/* rsm_forward_chunked with a router / decay variant: f is [B,T,Hh] or, with f_per_slot,
 * [B,T,Hh,M]; noise, if given, is [B,T,Hh,M].  Same workspace size. */
int rsm_forward_chunked_ex(const void* q, const void* k, const void* z, const void* v, int dtype,
                           const float* f, const float* H0, int64_t B, int64_t T, int64_t Hh,
                           int64_t M, int64_t Dv, int64_t K, int64_t C, float* o, float* H_out,
                           int32_t* idx_out, void* workspace, size_t workspace_bytes,
                           const rsm_router_opts* opts, void* stream);

/* rsm_decode_step with a router / decay variant: f is [B,Hh] or, with f_per_slot,
 * [B,Hh,M]; noise, if given, is [B,Hh,M]. */
int rsm_decode_step_ex(const void* q, const void* k, const void* z, const void* v, int dtype,
                       const float* f, float* H, int64_t B, int64_t Hh, int64_t M, int64_t Dv,
                       int64_t K, float* o, int32_t* idx_out, const rsm_router_opts* opts,
                       void* stream);

/*
 * Backward pass for training (the pages' chunked kernels exist for training: README kernel
 * notes): the gradients of L = sum(dO * o) + sum(dH_T * H_out) for the default router, i.e.
 * the vector-Jacobian product of rsm_forward_chunked with upstream gradients dO and dH_T.
 *   q, k, z  [B,T,Hh,M]   dtype;  v [B,T,Hh,Dv] dtype;  f [B,T,Hh] fp32;  H0 [B,Hh,M,Dv] or NULL
 *   dO       [B,T,Hh,Dv]  fp32 upstream gradient of o
 *   dH_T     [B,Hh,M,Dv]  fp32 upstream gradient of the final state, or NULL (zero)
 *   dq, dk, dz [B,T,Hh,M] fp32 out;  dv [B,T,Hh,Dv] fp32 out;  df [B,T,Hh] fp32 out
 *   dH0      [B,Hh,M,Dv]  fp32 out, or NULL
 *   workspace: at least rsm_backward_workspace_bytes() bytes (contents undefined)
 * The top-K selection is piecewise constant in z: dz is nonzero only on the selected slots
 * (through the sigmoid).  A full overwrite (f = -inf) gives no df or dz on that token.
 * Outputs must not overlap any input or each other.  M in {16, 32, 64, 128, 256}, Dv in
 * {16, ..., 256}.  The kernels walk each head's sequence token by token, its state split
 * by slot groups (dq, dk, dz, df, dH0) or by column tiles (dv).
 */
size_t rsm_backward_workspace_bytes(int dtype, int64_t B, int64_t T, int64_t Hh, int64_t M,
                                    int64_t Dv, int64_t K);
int rsm_backward(const void* q, const void* k, const void* z, const void* v, int dtype,
                 const float* f, const float* H0, const float* dO, const float* dH_T, int64_t B,
                 int64_t T, int64_t Hh, int64_t M, int64_t Dv, int64_t K, float* dq, float* dk,
                 float* dz, float* dv, float* df, float* dH0, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * rsm_forward_chunked without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as rsm_forward_chunked, whose kernels it
 * runs; the workspace is a fixed array inside the library (rsm_noalloc_scratch_bytes(),
 * 64 MiB, one copy per device, held until the process ends).  A problem whose
 * rsm_forward_workspace_bytes() exceeds it returns RSM_ERR_TOO_LARGE before anything is
 * enqueued.  The call allocates nothing.  Calls that overlap on one device (several streams
 * or host threads) share that array and race: serialise them.
 */
size_t rsm_noalloc_scratch_bytes(void);
int rsm_forward_chunked_noalloc(const void* q, const void* k, const void* z, const void* v,
                                int dtype, const float* f, const float* H0, int64_t B, int64_t T,
                                int64_t Hh, int64_t M, int64_t Dv, int64_t K, int64_t C, float* o,
                                float* H_out, int32_t* idx_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RSM_H */
