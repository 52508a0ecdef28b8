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

/* One token on the columns [c0, c1) of one head's state H [M, Dv]. */
static void oracle_token(const double* q, const double* k, const double* z, const double* v,
                         double f, double* H, long M, long Dv, long K, long c0, long c1,
                         double* o, int32_t* idx, unsigned char* sel) {
    oracle_select(z, M, K, sel);
    long n = 0;
    for (long i = 0; i < M; ++i) {
        if (!sel[i]) continue;
        if (idx) idx[n] = (int32_t)i;
        n++;
        double s = oracle_sigmoid(z[i]);
        double alpha = (s == 0.0) ? 1.0 : exp(s * f);
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

/* Router alone: idx [N,K] ascending slot order, score [N,K] = sigmoid(z) (nullable). */
int rsm_oracle_route_topk(const double* z, long N, long M, long K, int32_t* idx, double* score) {
    if (!z || !idx || N < 0 || M < 1 || K < 1 || K > M) return -1;
    unsigned char* sel = (unsigned char*)malloc((size_t)M);
    if (!sel) return -2;
    for (long r = 0; r < N; ++r) {
        const double* zr = z + r * M;
        oracle_select(zr, M, K, sel);
        long n = 0;
        for (long i = 0; i < M; ++i) {
            if (!sel[i]) continue;
            idx[r * K + n] = (int32_t)i;
            if (score) score[r * K + n] = oracle_sigmoid(zr[i]);
            n++;
        }
    }
    free(sel);
    return 0;
}

/* Whole-sequence recurrence.  H0 may be NULL (zero state).  H_out, idx_out may be NULL.
 * H_trace (nullable) receives the state after every token: [B,Hh,T,M,Dv]. */
int rsm_oracle_forward(const double* q, const double* k, const double* z, const double* v,
                       const double* f, const double* H0, long B, long T, long Hh, long M,
                       long Dv, long K, double* o, double* H_out, int32_t* idx_out,
                       double* H_trace, int nthreads) {
    if (!q || !k || !z || !v || !f || !o) return -1;
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
        if (!H || !sel || !orow) {
            free(H); free(sel); free(orow);
            status = -2;
            continue;
        }
        for (long i = 0; i < M; ++i)
            for (long c = 0; c < Dv; ++c)
                H[i * Dv + c] = H0 ? H0[((b * Hh + h) * M + i) * Dv + c] : 0.0;
        for (long t = 0; t < T; ++t) {
            long row = (b * T + t) * Hh + h; /* token-head row index */
            int32_t* idx = (idx_out && cb == 0) ? idx_out + row * K : NULL;
            oracle_token(q + row * M, k + row * M, z + row * M, v + row * Dv, f[row], H, M, Dv,
                         K, c0, c1, orow, idx, sel);
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
        free(H); free(sel); free(orow);
    }
    return status;
}

/* One decode step for every (b, h): q,k,z [B,Hh,M], v [B,Hh,Dv], f [B,Hh];
 * H [B,Hh,M,Dv] updated in place; o [B,Hh,Dv]; idx_out [B,Hh,K] nullable. */
int rsm_oracle_decode_step(const double* q, const double* k, const double* z, const double* v,
                           const double* f, double* H, long B, long Hh, long M, long Dv, long K,
                           double* o, int32_t* idx_out, int nthreads) {
    if (!q || !k || !z || !v || !f || !H || !o) return -1;
    if (B < 1 || Hh < 1 || M < 1 || Dv < 1 || K < 1 || K > M) return -1;
    int status = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
    for (long bh = 0; bh < B * Hh; ++bh) {
        unsigned char* sel = (unsigned char*)malloc((size_t)M);
        if (!sel) { status = -2; continue; }
        oracle_token(q + bh * M, k + bh * M, z + bh * M, v + bh * Dv, f[bh], H + bh * M * Dv,
                     M, Dv, K, 0, Dv, o + bh * Dv, idx_out ? idx_out + bh * K : NULL, sel);
        free(sel);
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
