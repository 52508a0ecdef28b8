/*
 * rsm_oracle.c -- plain, slow, float64 CPU reference of the Routing State Model (RSM)
 * mixer of Raven: sigmoid + top-k router, sparse gated slot update, read.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the package's smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code, header,
 * table or helper with the HIP library; the product path never calls it.
 *
 * What it computes, per (batch b, head h), token by token (Raven README page,
 * "How Raven Works": route_scores = TopK(sigmoid(r_proj(x))), decay = exp(route_scores*f),
 * H = H*decay + (1-decay)*k (x) v, o = q . H):
 *
 *   1. route: rank every slot by (z descending, slot index ascending); the K best are
 *      selected.  Ranking the logits z equals ranking the exact sigmoid scores because
 *      the sigmoid is strictly increasing; equal logits (as values, so -0 == +0) go to
 *      the lower slot index.  s_i = 1/(1+exp(-z_i)) for selected slots.
 *   2. update, selected slots only: alpha_i = exp(s_i * f_t), then
 *      H[i,:] = alpha_i*H[i,:] + (1-alpha_i)*k_i*v_t[:].  Unselected slots are not
 *      touched at all, so they keep their bits (Raven paper summary, section 4.1: slots
 *      with near-zero routing remain untouched; appendix A.7: unselected slots
 *      preserve their contents exactly).  A selected slot whose alpha is exactly 1
 *      (s_i*f_t == 0, e.g. a score that underflowed to 0) is frozen as well (section
 *      3.2: a slot with zero routing is frozen until selected again).  f_t = -inf gives
 *      alpha = 0 (full overwrite) for every selected slot with s_i > 0.
 *   3. read after the update (the order of the README's listing): o_t = sum_i q_i H[i,:]
 *      over all M slots, slot index ascending.
 *
 * Heads and d_v columns are independent (slot separability, paper summary section 3.1
 * and appendix A.2), so the work is split over (b, h, column block) with OpenMP; each
 * column block re-derives the routing, which is cheap and keeps every item standalone.
 *
 * Layouts (row-major, contiguous): q,k,z [B,T,Hh,M]; v [B,T,Hh,Dv]; f [B,T,Hh];
 * H0/H_out [B,Hh,M,Dv]; o [B,T,Hh,Dv]; idx [B,T,Hh,K] (ascending slot order).
 *
 * Router and decay variants (the *_ex entry points), each named on the pages:
 *  - score kind: sigmoid (default) or softmax over all M slots (README configuration
 *    table "top-k sigmoid/softmax" and the router_score option; paper summary section
 *    6.2.1).  The softmax is increasing in each logit, so the selection is the same top-K
 *    of the logits; the selected slots take softmax(z)_i = exp(z_i - max z) / sum_j
 *    exp(z_j - max z).
 *  - normalize: the selected scores divided by their sum, so they sum to one over the K
 *    selected slots (paper summary section 4.1).  A zero sum leaves them as they are.
 *  - per-slot decay: f [B,T,Hh,M], alpha_i = exp(s_i * f_i) (the GLA decay option of the
 *    README configuration table is a diagonal gate, paper summary section 2.1).
 *  - exploration noise: g [B,T,Hh,M] added to the logits before selection and scoring
 *    (paper summary section 6.2.2, Gumbel noise during training).  The caller draws g.
 *    The noisy logit is part of the input's definition: z and g are handed over as fp32
 *    tensors, and the logit the router ranks and scores is their fp32 sum fl32(z + g),
 *    the tensor a caller holding both in fp32 forms before routing.  The oracle builds
 *    that input exactly (one fp32 add) and works in float64 from there.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Selection flags by the rank-count definition of top-K with ties to the lower index. */
static void oracle_select(const double* z, long M, long K, unsigned char* sel) {
    for (long i = 0; i < M; ++i) {
        long rank = 0;
        for (long j = 0; j < M; ++j) {
            if (z[j] > z[i] || (j < i && z[j] == z[i])) rank++;
        }
        sel[i] = (unsigned char)(rank < K);
    }
}

static double oracle_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/* Router variant: score kind (0 sigmoid, 1 softmax) and whether the selected scores are
 * divided by their sum. */
typedef struct {
    int softmax;
    int normalize;
} oracle_router;

/* Logits of one row as the router ranks them: z, or the noisy-logit input fl32(z + g). */
static void oracle_logits(const double* z, const double* g, long M, double* zp) {
    for (long i = 0; i < M; ++i) zp[i] = g ? (double)((float)z[i] + (float)g[i]) : z[i];
}

/* Selection flags and the score of every selected slot (s[i] for sel[i]; 0 elsewhere). */
static void oracle_route_row(const double* zp, long M, long K, oracle_router r, unsigned char* sel,
                             double* s) {
    oracle_select(zp, M, K, sel);
    double zmax = zp[0], den = 0.0;
    if (r.softmax) {
        for (long i = 1; i < M; ++i) zmax = zp[i] > zmax ? zp[i] : zmax;
        for (long i = 0; i < M; ++i) den += exp(zp[i] - zmax);
    }
    double tot = 0.0;
    for (long i = 0; i < M; ++i) {
        s[i] = 0.0;
        if (!sel[i]) continue;
        s[i] = r.softmax ? exp(zp[i] - zmax) / den : oracle_sigmoid(zp[i]);
        tot += s[i];
    }
    if (r.normalize && tot > 0.0)
        for (long i = 0; i < M; ++i) s[i] /= tot;
}

/* One token on the columns [c0, c1) of one head's state H [M, Dv].  f holds one decay
 * rate (fstride 0) or one per slot (fstride 1); g is the noise row or NULL; w is scratch
 * of 2*M doubles. */
static void oracle_token(const double* q, const double* k, const double* z, const double* g,
                         const double* v, const double* f, long fstride, oracle_router r,
                         double* H, long M, long Dv, long K, long c0, long c1, double* o,
                         int32_t* idx, unsigned char* sel, double* w) {
    double* zp = w;
    double* sc = w + M;
    oracle_logits(z, g, M, zp);
    oracle_route_row(zp, M, K, r, sel, sc);
    long n = 0;
    for (long i = 0; i < M; ++i) {
        if (!sel[i]) continue;
        if (idx) idx[n] = (int32_t)i;
        n++;
        double s = sc[i];
        double alpha = (s == 0.0) ? 1.0 : exp(s * f[i * fstride]);
        if (alpha == 1.0) continue; /* frozen */
        double w = (1.0 - alpha) * k[i];
        double* row = H + i * Dv;
        for (long c = c0; c < c1; ++c) row[c] = alpha * row[c] + w * v[c];
    }
    for (long c = c0; c < c1; ++c) {
        double acc = 0.0;
        for (long i = 0; i < M; ++i) acc += q[i] * H[i * Dv + c];
        o[c] = acc;
    }
}

/* Router alone: idx [N,K] ascending slot order, score [N,K] (nullable) = the routing
 * weight of each selected slot.  noise [N,M] or NULL; softmax, normalize as above. */
int rsm_oracle_route_ex(const double* z, const double* noise, long N, long M, long K, int softmax,
                        int normalize, int32_t* idx, double* score) {
    if (!z || !idx || N < 0 || M < 1 || K < 1 || K > M) return -1;
    unsigned char* sel = (unsigned char*)malloc((size_t)M);
    double* w = (double*)malloc(sizeof(double) * (size_t)(2 * M));
    if (!sel || !w) { free(sel); free(w); return -2; }
    oracle_router rr = {softmax != 0, normalize != 0};
    for (long r = 0; r < N; ++r) {
        oracle_logits(z + r * M, noise ? noise + r * M : NULL, M, w);
        oracle_route_row(w, M, K, rr, sel, w + M);
        long n = 0;
        for (long i = 0; i < M; ++i) {
            if (!sel[i]) continue;
            idx[r * K + n] = (int32_t)i;
            if (score) score[r * K + n] = w[M + i];
            n++;
        }
    }
    free(sel);
    free(w);
    return 0;
}

int rsm_oracle_route_topk(const double* z, long N, long M, long K, int32_t* idx, double* score) {
    return rsm_oracle_route_ex(z, NULL, N, M, K, 0, 0, idx, score);
}

/* Whole-sequence recurrence.  H0 may be NULL (zero state).  H_out, idx_out may be NULL.
 * H_trace (nullable) receives the state after every token: [B,Hh,T,M,Dv].
 * noise [B,T,Hh,M] or NULL; f is [B,T,Hh] (f_per_slot 0) or [B,T,Hh,M] (f_per_slot 1). */
int rsm_oracle_forward_ex(const double* q, const double* k, const double* z, const double* noise,
                          const double* v, const double* f, int f_per_slot, const double* H0,
                          long B, long T, long Hh, long M, long Dv, long K, int softmax,
                          int normalize, double* o, double* H_out, int32_t* idx_out,
                          double* H_trace, int nthreads) {
    if (!q || !k || !z || !v || !f || !o) return -1;
    const oracle_router rr = {softmax != 0, normalize != 0};
    if (B < 1 || T < 0 || Hh < 1 || M < 1 || Dv < 1 || K < 1 || K > M) return -1;
    long ncb = 1;
    if (B * Hh < 64) ncb = Dv >= 8 ? 8 : Dv; /* split columns when heads are few */
    long items = B * Hh * ncb;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long it = 0; it < items; ++it) {
        long bh = it / ncb, cb = it % ncb;
        long b = bh / Hh, h = bh % Hh;
        long c0 = (Dv * cb) / ncb, c1 = (Dv * (cb + 1)) / ncb;
        double* H = (double*)malloc(sizeof(double) * (size_t)(M * Dv));
        unsigned char* sel = (unsigned char*)malloc((size_t)M);
        double* orow = (double*)malloc(sizeof(double) * (size_t)Dv);
        double* w = (double*)malloc(sizeof(double) * (size_t)(2 * M));
        if (!H || !sel || !orow || !w) {
            free(H); free(sel); free(orow); free(w);
            status = -2;
            continue;
        }
        for (long i = 0; i < M; ++i)
            for (long c = 0; c < Dv; ++c)
                H[i * Dv + c] = H0 ? H0[((b * Hh + h) * M + i) * Dv + c] : 0.0;
        for (long t = 0; t < T; ++t) {
            long row = (b * T + t) * Hh + h; /* token-head row index */
            int32_t* idx = (idx_out && cb == 0) ? idx_out + row * K : NULL;
            oracle_token(q + row * M, k + row * M, z + row * M, noise ? noise + row * M : NULL,
                         v + row * Dv, f_per_slot ? f + row * M : f + row, f_per_slot ? 1 : 0, rr,
                         H, M, Dv, K, c0, c1, orow, idx, sel, w);
            for (long c = c0; c < c1; ++c) o[row * Dv + c] = orow[c];
            if (H_trace) {
                double* dst = H_trace + (((b * Hh + h) * T + t) * M) * Dv;
                for (long i = 0; i < M; ++i)
                    for (long c = c0; c < c1; ++c) dst[i * Dv + c] = H[i * Dv + c];
            }
        }
        if (H_out)
            for (long i = 0; i < M; ++i)
                for (long c = c0; c < c1; ++c)
                    H_out[((b * Hh + h) * M + i) * Dv + c] = H[i * Dv + c];
        free(H); free(sel); free(orow); free(w);
    }
    return status;
}

int rsm_oracle_forward(const double* q, const double* k, const double* z, const double* v,
                       const double* f, const double* H0, long B, long T, long Hh, long M,
                       long Dv, long K, double* o, double* H_out, int32_t* idx_out,
                       double* H_trace, int nthreads) {
    return rsm_oracle_forward_ex(q, k, z, NULL, v, f, 0, H0, B, T, Hh, M, Dv, K, 0, 0, o, H_out,
                                 idx_out, H_trace, nthreads);
}

/* One decode step for every (b, h): q,k,z [B,Hh,M], v [B,Hh,Dv], f [B,Hh] (or [B,Hh,M]
 * with f_per_slot); noise [B,Hh,M] or NULL; H [B,Hh,M,Dv] updated in place; o [B,Hh,Dv];
 * idx_out [B,Hh,K] nullable. */
int rsm_oracle_decode_ex(const double* q, const double* k, const double* z, const double* noise,
                         const double* v, const double* f, int f_per_slot, double* H, long B,
                         long Hh, long M, long Dv, long K, int softmax, int normalize, double* o,
                         int32_t* idx_out, int nthreads) {
    if (!q || !k || !z || !v || !f || !H || !o) return -1;
    const oracle_router rr = {softmax != 0, normalize != 0};
    if (B < 1 || Hh < 1 || M < 1 || Dv < 1 || K < 1 || K > M) return -1;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (long bh = 0; bh < B * Hh; ++bh) {
        unsigned char* sel = (unsigned char*)malloc((size_t)M);
        double* w = (double*)malloc(sizeof(double) * (size_t)(2 * M));
        if (!sel || !w) { free(sel); free(w); status = -2; continue; }
        oracle_token(q + bh * M, k + bh * M, z + bh * M, noise ? noise + bh * M : NULL, v + bh * Dv,
                     f_per_slot ? f + bh * M : f + bh, f_per_slot ? 1 : 0, rr, H + bh * M * Dv, M,
                     Dv, K, 0, Dv, o + bh * Dv, idx_out ? idx_out + bh * K : NULL, sel, w);
        free(sel);
        free(w);
    }
    return status;
}

int rsm_oracle_decode_step(const double* q, const double* k, const double* z, const double* v,
                           const double* f, double* H, long B, long Hh, long M, long Dv, long K,
                           double* o, int32_t* idx_out, int nthreads) {
    return rsm_oracle_decode_ex(q, k, z, NULL, v, f, 0, H, B, Hh, M, Dv, K, 0, 0, o, idx_out,
                                nthreads);
}

/* Gradients of the default-router recurrence (sigmoid scores, one decay rate per token-head)
 * for the loss L = sum(dO . o) + sum(dH_T . H_T), i.e. the vector-Jacobian product with the
 * upstream gradients dO [B,T,Hh,Dv] and dHT [B,Hh,M,Dv] (NULL = 0).  Outputs (all written):
 * dq, dk, dz [B,T,Hh,M], dv [B,T,Hh,Dv], df [B,T,Hh], dH0 [B,Hh,M,Dv].
 *
 * Per (b, h) the forward runs first and keeps every state H_t (the state after token t,
 * H_{-1} = H0).  The backward then walks t = T-1 .. 0 carrying G = dL/dH_t, written out from
 * the chain rule on the update of the README listing, H_t[i,:] = a_i H_{t-1}[i,:] +
 * (1 - a_i) k_i v_t for the selected slots (a_i = exp(s_i f_t), s_i = sigmoid(z_i)), and the
 * read o_t = q_t . H_t:
 *   G        += q_t (x) dO_t                       (the read of token t)
 *   dq_t[i]   = sum_c dO_t[c] H_t[i,c]
 *   for every selected slot i with s_i > 0:
 *     dk_t[i]   = (1 - a_i) sum_c G[i,c] v_t[c]
 *     dv_t[c]  += (1 - a_i) k_i G[i,c]
 *     da        = sum_c G[i,c] (H_{t-1}[i,c] - k_i v_t[c])
 *     dg        = a_i da                          (a = exp(g), g = s_i f_t)
 *     df_t     += dg s_i,   dz_t[i] = dg f_t s_i (1 - s_i)
 *     G[i,:]   *= a_i                             (what flows to H_{t-1})
 *   dH0 = G after token 0.
 * The top-K selection is piecewise constant in z, so an unselected slot gets dz = 0 and passes
 * G through unchanged.  A selected slot whose score is 0 (sigmoid underflow) is frozen: no
 * gradient.  With a = 0 (f = -inf, or exp underflow) a does not move with s or f, so dg = 0
 * (no df or dz contribution) while dk, dv and the cut of G still apply. */
int rsm_oracle_backward(const double* q, const double* k, const double* z, const double* v,
                        const double* f, const double* H0, const double* dO, const double* dHT,
                        long B, long T, long Hh, long M, long Dv, long K, double* dq, double* dk,
                        double* dz, double* dv, double* df, double* dH0, int nthreads) {
    if (!q || !k || !z || !v || !f || !dO || !dq || !dk || !dz || !dv || !df || !dH0) return -1;
    if (B < 1 || T < 0 || Hh < 1 || M < 1 || Dv < 1 || K < 1 || K > M) return -1;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
#endif
    for (long bh = 0; bh < B * Hh; ++bh) {
        long b = bh / Hh, h = bh % Hh;
        double* Hs = (double*)malloc(sizeof(double) * (size_t)((T + 1) * M * Dv)); /* H_{t-1}, t = 0..T */
        double* sc = (double*)malloc(sizeof(double) * (size_t)(T * M));            /* s, 0 if unselected */
        double* G = (double*)malloc(sizeof(double) * (size_t)(M * Dv));
        unsigned char* sel = (unsigned char*)malloc((size_t)M);
        double* w = (double*)malloc(sizeof(double) * (size_t)(2 * M));
        double* orow = (double*)malloc(sizeof(double) * (size_t)Dv);
        if (!Hs || !sc || !G || !sel || !w || !orow) {
            free(Hs); free(sc); free(G); free(sel); free(w); free(orow);
            status = -2;
            continue;
        }
        /* forward, keeping every state: Hs + (t+1)*M*Dv holds H_t */
        for (long i = 0; i < M * Dv; ++i) Hs[i] = H0 ? H0[bh * M * Dv + i] : 0.0;
        const oracle_router rr = {0, 0};
        for (long t = 0; t < T; ++t) {
            long row = (b * T + t) * Hh + h;
            double* Hn = Hs + (t + 1) * M * Dv;
            memcpy(Hn, Hs + t * M * Dv, sizeof(double) * (size_t)(M * Dv));
            oracle_token(q + row * M, k + row * M, z + row * M, NULL, v + row * Dv, f + row, 0, rr, Hn, M,
                         Dv, K, 0, Dv, orow, NULL, sel, w);
            for (long i = 0; i < M; ++i) sc[t * M + i] = sel[i] ? w[M + i] : 0.0;
        }
        /* backward */
        for (long i = 0; i < M * Dv; ++i) G[i] = dHT ? dHT[bh * M * Dv + i] : 0.0;
        for (long t = T - 1; t >= 0; --t) {
            long row = (b * T + t) * Hh + h;
            const double* qt = q + row * M;
            const double* kt = k + row * M;
            const double* vt = v + row * Dv;
            const double* dOt = dO + row * Dv;
            const double* Ht = Hs + (t + 1) * M * Dv;
            const double* Hp = Hs + t * M * Dv;
            for (long i = 0; i < M; ++i)
                for (long c = 0; c < Dv; ++c) G[i * Dv + c] += qt[i] * dOt[c];
            for (long i = 0; i < M; ++i) {
                double acc = 0.0;
                for (long c = 0; c < Dv; ++c) acc += dOt[c] * Ht[i * Dv + c];
                dq[row * M + i] = acc;
            }
            for (long c = 0; c < Dv; ++c) dv[row * Dv + c] = 0.0;
            double dft = 0.0;
            for (long i = 0; i < M; ++i) {
                double s = sc[t * M + i];
                dk[row * M + i] = 0.0;
                dz[row * M + i] = 0.0;
                if (s == 0.0) continue; /* unselected, or frozen */
                double a = exp(s * f[row]);
                double u = 0.0, da = 0.0;
                for (long c = 0; c < Dv; ++c) {
                    u += G[i * Dv + c] * vt[c];
                    da += G[i * Dv + c] * (Hp[i * Dv + c] - kt[i] * vt[c]);
                }
                dk[row * M + i] = (1.0 - a) * u;
                for (long c = 0; c < Dv; ++c) dv[row * Dv + c] += (1.0 - a) * kt[i] * G[i * Dv + c];
                if (a > 0.0) {
                    double dg = a * da;
                    dft += dg * s;
                    dz[row * M + i] = dg * f[row] * s * (1.0 - s);
                }
                for (long c = 0; c < Dv; ++c) G[i * Dv + c] *= a;
            }
            df[row] = dft;
        }
        for (long i = 0; i < M * Dv; ++i) dH0[bh * M * Dv + i] = G[i];
        free(Hs); free(sc); free(G); free(sel); free(w); free(orow);
    }
    return status;
}

int rsm_oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
