// rsm_recurrent.hip -- whole-sequence forward in the recurrent form, for slot counts whose
// chunk tiles do not fit in LDS (M = 256, the pages' default layer shape).
//
// Raven README page, "How Raven Works": per token the top-K slots by router score are
// decayed by alpha = exp(s*f) and written with (1-alpha)*k_i*v, then o = q . H is read
// after the write; the README pairs chunked kernels for training with fused recurrent
// kernels for generation -- both compute the same sequence of states.
//
// Two launches on the caller's stream:
//  1. the router over every token-head row at once (route_topk_launch: idx in ascending
//     slot order and the routing weight s of each selected slot), into the workspace or
//     idx_out;
//  2. recurrent_scan_kernel: one 256-thread workgroup per (head, column tile) holds its tile
//     of H [M, DTC] in registers for the whole sequence and applies the tokens in order.
//     Each token's q, k (one slot per thread), v columns, route and f are loaded ahead into
//     a register ring of two sets of PD tokens (one set in flight while the other is
//     applied); the selected slots are marked in LDS with the token index (no clearing
//     between tokens), the thread of each slot forms its alpha and write weight, and every
//     thread then updates its rows from one 16-byte LDS read per row; three barriers per
//     token, which wait for LDS only, so the ring's loads stay in flight across them.
#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

// state columns per workgroup: the whole row unless M * DV is large (as in the decode step)
template <int M, int DV>
constexpr int rec_cols() { return DV < 16384 / M ? DV : 16384 / M; }

// Inputs as loaded (raw bf16 bits or fp32), converted to fp32 only when used: a conversion
// next to the load would make the wave wait for it there and defeat the prefetch.
__device__ __forceinline__ float raw_to_f(float x) { return x; }
__device__ __forceinline__ float raw_to_f(bf16_t x) { return bf16_to_float(x.bits); }
template <typename T> struct Raw4;  // four consecutive inputs
template <> struct Raw4<float> {
    float4 x;
    __device__ __forceinline__ void load(const float* p) { x = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ float4 get() const { return x; }
};
template <> struct Raw4<bf16_t> {
    uint2 x;
    __device__ __forceinline__ void load(const bf16_t* p) { x = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float4 get() const {
        return make_float4(__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xFFFF0000u),
                           __uint_as_float(x.y << 16), __uint_as_float(x.y & 0xFFFF0000u));
    }
};

// KR: route entries per router lane (K <= 64 * KR); FSLOT: f holds one rate per slot.
// The ring's loads are free of branches (token index clamped to the sequence, every wave
// loading the route entries), so the compiler can count them across the token loop and
// wait only for the entry it is about to use.
template <typename T, int M, int DV, int KR, bool FSLOT>
__global__ __launch_bounds__(256) void recurrent_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ f,
    const float* __restrict__ H0, long T_len, int Hh, int K, const int32_t* __restrict__ ridx,
    const float* __restrict__ rsc, float* __restrict__ o, float* __restrict__ H_out) {
    static_assert(M == 256, "one slot per thread of the workgroup");
    constexpr int DTC = rec_cols<M, DV>(), NTL = DV / DTC;
    constexpr int TPR = DTC / 4;              // threads per state row, one float4 each
    constexpr int RPP = 256 / TPR;            // rows covered per pass of the workgroup
    constexpr int RPT = (M + RPP - 1) / RPP;  // rows held per thread
    constexpr int PD = 4;                     // tokens per ring set
    __shared__ float s_s[M];
    __shared__ int s_sel[M];
    __shared__ float4 s_coef[M];  // per slot: alpha, (1 - alpha) * k, q, update flag
    __shared__ float4 s_red[RPP][TPR];

    const long bh = blockIdx.x / NTL;
    const int tile = int(blockIdx.x % NTL), c0 = tile * DTC;
    const int tid = threadIdx.x;
    const int cg = tid % TPR, rg = tid / TPR;
    const long b = bh / Hh;
    const int h = int(bh % Hh);
    const long row0 = b * T_len * Hh + h;  // token-head row of token 0; token t is row0 + t * Hh
    const long hoff = bh * long(M) * DV + c0;

    float4 hv[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = rg + j * RPP;
        hv[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (row < M && H0) hv[j] = *reinterpret_cast<const float4*>(H0 + hoff + long(row) * DV + 4 * cg);
    }
    s_sel[tid] = -1;

    const int lane = tid % kWave;
    // register ring of 2 * PD tokens in two sets (entries 0..PD-1 and PD..2PD-1): while one
    // set's tokens are applied, the other set's loads for the next PD tokens are in flight
    T pq[2 * PD], pk[2 * PD];
    float pf[2 * PD], ps[2 * PD][KR];
    Raw4<T> pv[2 * PD];
    int pi[2 * PD][KR];
    auto fetch = [&](int u, long t) {
        const long r = row0 + (t < T_len ? t : T_len - 1) * Hh;  // past the end: reload the last token
        pq[u] = q[r * M + tid];
        pk[u] = k[r * M + tid];
        if constexpr (FSLOT) {
            pf[u] = f[r * M + tid];
        } else {
            // a uniform address would become a scalar-cache load, which the barriers' LDS
            // wait (lgkmcnt) would then wait for: keep the index in vector registers
            long fi = r;
            __asm__("" : "+v"(fi));
            pf[u] = f[fi];
        }
        pv[u].load(v + r * DV + c0 + 4 * cg);
#pragma unroll
        for (int rr = 0; rr < KR; ++rr) {
            const int n = rr * kWave + lane;
            const long e = r * K + (n < K ? n : K - 1);
            pi[u][rr] = ridx[e];
            ps[u][rr] = rsc[e];
        }
    };
    // token t from ring entry u: mark the selected slots, let each slot's thread form its
    // coefficients, update the rows held, reduce o_t.  Three barriers; every read of the
    // previous token's LDS values ended at one of its barriers before it is overwritten.
    auto apply = [&](int u, long t) {
        const long r = row0 + t * Hh;
        const int stamp = int(t);
        if (tid < kWave) {
#pragma unroll
            for (int rr = 0; rr < KR; ++rr) {
                const int slot = pi[u][rr];
                if (rr * kWave + lane < K && unsigned(slot) < unsigned(M)) {
                    s_s[slot] = ps[u][rr];
                    s_sel[slot] = stamp;
                }
            }
        }
        wg_barrier();
        {  // slot tid: alpha = exp(s f) if selected (1 when s f = 0), weight (1 - alpha) k
            float a = 1.0f, wk = 0.0f;
            if (s_sel[tid] == stamp) {
                const float sc = s_s[tid];
                if (sc > 0.0f) a = __expf(sc * pf[u]);
                if (a != 1.0f) wk = (1.0f - a) * raw_to_f(pk[u]);
            }
            s_coef[tid] = make_float4(a, wk, raw_to_f(pq[u]), a != 1.0f ? 1.0f : 0.0f);
        }
        const float4 vv = pv[u].get();
        wg_barrier();

        float4 cf[RPT];
#pragma unroll
        for (int j = 0; j < RPT; ++j) cf[j] = s_coef[rg + j * RPP];
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const float a = cf[j].x, wk = cf[j].y, qi = cf[j].z;
            const bool upd = cf[j].w != 0.0f;  // rows not written keep their bits
            float4 hh = hv[j];
            hh.x = upd ? fmaf(a, hh.x, wk * vv.x) : hh.x;
            hh.y = upd ? fmaf(a, hh.y, wk * vv.y) : hh.y;
            hh.z = upd ? fmaf(a, hh.z, wk * vv.z) : hh.z;
            hh.w = upd ? fmaf(a, hh.w, wk * vv.w) : hh.w;
            hv[j] = hh;
            acc.x = fmaf(qi, hh.x, acc.x);
            acc.y = fmaf(qi, hh.y, acc.y);
            acc.z = fmaf(qi, hh.z, acc.z);
            acc.w = fmaf(qi, hh.w, acc.w);
        }
        s_red[rg][cg] = acc;
        wg_barrier();
        if (rg == 0) {
            float4 sum = s_red[0][cg];
            for (int g = 1; g < RPP; ++g) {
                const float4 p = s_red[g][cg];
                sum.x += p.x;
                sum.y += p.y;
                sum.z += p.z;
                sum.w += p.w;
            }
            *reinterpret_cast<float4*>(o + r * DV + c0 + 4 * cg) = sum;
        }
    };

#pragma unroll
    for (int u = 0; u < PD; ++u) fetch(u, u);
    __syncthreads();  // s_sel initialised before the first token marks it

    for (long t0 = 0; t0 < T_len; t0 += 2 * PD) {
#pragma unroll
        for (int u = 0; u < PD; ++u) fetch(PD + u, t0 + PD + u);
#pragma unroll
        for (int u = 0; u < PD; ++u)
            if (t0 + u < T_len) apply(u, t0 + u);  // uniform over the workgroup
        if (t0 + PD >= T_len) break;
#pragma unroll
        for (int u = 0; u < PD; ++u) fetch(u, t0 + 2 * PD + u);
#pragma unroll
        for (int u = 0; u < PD; ++u)
            if (t0 + PD + u < T_len) apply(PD + u, t0 + PD + u);
    }
    if (H_out) {
#pragma unroll
        for (int j = 0; j < RPT; ++j) {
            const int row = rg + j * RPP;
            if (row < M) *reinterpret_cast<float4*>(H_out + hoff + long(row) * DV + 4 * cg) = hv[j];
        }
    }
}

static size_t align256r(size_t x) { return (x + 255) / 256 * 256; }

size_t forward_recurrent_workspace(long B, long T, long Hh, int K) {
    const size_t n = size_t(B) * size_t(T) * size_t(Hh) * size_t(K) * 4;
    return n == 0 ? 0 : 2 * align256r(n);
}

template <typename T, int M, int DV>
static int launch_scan_dv(const T* q, const T* k, const T* v, const float* f, const float* H0, long n_heads, long T_len,
                          int Hh, int K, int f_per_slot, const int32_t* ridx, const float* rsc, float* o, float* H_out,
                          hipStream_t s) {
    const dim3 grid(unsigned(n_heads * (DV / rec_cols<M, DV>()))), block(256);
#define RSM_REC(KR, FS)                                                                                           \
    hipLaunchKernelGGL((recurrent_scan_kernel<T, M, DV, KR, FS>), grid, block, 0, s, q, k, v, f, H0, T_len, Hh, K, \
                       ridx, rsc, o, H_out)
    if (K <= kWave) {
        if (f_per_slot) RSM_REC(1, true);
        else RSM_REC(1, false);
    } else {
        if (f_per_slot) RSM_REC(4, true);
        else RSM_REC(4, false);
    }
#undef RSM_REC
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

template <typename T>
static int launch_scan(const void* q, const void* k, const void* v, const float* f, const float* H0, long n_heads,
                       long T_len, int Hh, int M, int Dv, int K, int f_per_slot, const int32_t* ridx, const float* rsc,
                       float* o, float* H_out, hipStream_t s) {
    const T *qq = static_cast<const T*>(q), *kk = static_cast<const T*>(k), *vv = static_cast<const T*>(v);
    if (M != 256) return RSM_ERR_UNSUPPORTED;
    switch (Dv) {
        case 16: return launch_scan_dv<T, 256, 16>(qq, kk, vv, f, H0, n_heads, T_len, Hh, K, f_per_slot, ridx, rsc, o, H_out, s);
        case 32: return launch_scan_dv<T, 256, 32>(qq, kk, vv, f, H0, n_heads, T_len, Hh, K, f_per_slot, ridx, rsc, o, H_out, s);
        case 64: return launch_scan_dv<T, 256, 64>(qq, kk, vv, f, H0, n_heads, T_len, Hh, K, f_per_slot, ridx, rsc, o, H_out, s);
        case 128: return launch_scan_dv<T, 256, 128>(qq, kk, vv, f, H0, n_heads, T_len, Hh, K, f_per_slot, ridx, rsc, o, H_out, s);
        case 256: return launch_scan_dv<T, 256, 256>(qq, kk, vv, f, H0, n_heads, T_len, Hh, K, f_per_slot, ridx, rsc, o, H_out, s);
    }
    return RSM_ERR_UNSUPPORTED;
}

int forward_recurrent_launch(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                             const float* H0, long B, long T, long Hh, int M, int Dv, int K, float* o, float* H_out,
                             int32_t* idx_out, void* workspace, const RouterOpts& op, hipStream_t stream) {
    const long rows = B * T * Hh;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    int32_t* ridx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws);
    float* rsc = reinterpret_cast<float*>(ws + align256r(size_t(rows) * size_t(K) * 4));
    int st = route_topk_launch(z, dtype, rows, M, K, ridx, rsc, op, stream);
    if (st != RSM_OK) return st;
    if (dtype == RSM_F32)
        return launch_scan<float>(q, k, v, f, H0, B * Hh, T, int(Hh), M, Dv, K, op.f_per_slot, ridx, rsc, o, H_out,
                                  stream);
    return launch_scan<bf16_t>(q, k, v, f, H0, B * Hh, T, int(Hh), M, Dv, K, op.f_per_slot, ridx, rsc, o, H_out,
                               stream);
}

}  // namespace rsm
