// rsm_backward.hip -- gradients of the RSM recurrence (default router) for training: the
// vector-Jacobian product with upstream gradients dO (of the outputs) and dH_T (of the final
// state).  The pages' chunked kernels exist for training (Raven README, kernel notes); this
// is the backward pass of the same recurrence.
//
// For the update H_t[i,:] = a_ti H_{t-1}[i,:] + (1 - a_ti) k_ti v_t (selected slots,
// a = exp(s f_t), s = sigmoid(z)) and the read o_t = q_t . H_t, with G_t = dL/dH_t:
//     G_t   = q_t (x) dO_t + diag(a_{t+1}) G_{t+1},          G_{T-1} = dH_T + q_{T-1} (x) dO_{T-1}
//     dq_t  = H_t dO_t                     (per slot: row i of H_t against dO_t)
//     u_t   = G_t v_t,   dk_t = (1 - a_t) o u_t,   dv_t = G_t^T ((1 - a_t) o k_t)
//     dH0   = diag(a_0) G_0
// and the decay gradient dg = a da (g = s f) through the row identity
//     D_t = G_t[i,:] . H_t[i,:] = q_ti dq_ti + D_{t+1} - k_{t+1,i} dk_{t+1,i},  D_{T-1} = q dq + dH_T[i,:] . H_{T-1}[i,:]
//     dg_ti = D_ti - k_ti u_ti   (selected slots with a > 0; 0 when a = 0)
// (a H_{t-1} = H_t - (1 - a) k v on a selected row), so no pass needs H and G at once:
//     dz_ti = dg_ti f_t s_ti (1 - s_ti),   df_t = sum_i dg_ti s_ti.
// The top-K selection is piecewise constant in z: unselected slots get dz = 0.
//
// Passes (each walks the whole sequence of a head in order; the state stays in registers):
//  1. route: the router kernel's indices and scores, scattered into dense per-slot alpha and s
//     (alpha = 1, s = 0 off the top K) in the workspace.
//  2. rows forward (one workgroup per head and group of 16 slots; a thread holds Dv/16
//     columns of one slot row of H): dq_t, then D's start value dH_T . H_{T-1} per slot.
//  3. rows backward (same layout, rows of G): u, dk, dg (-> dz and dg s per slot), dH0.
//  4. columns backward (one workgroup per head and tile of 16 columns; a thread holds M/16
//     slots of one column of G): dv_t.
// Each pass keeps the loads of the next eight tokens in flight (register ring) and sums
// across the 16 lanes of a row with DPP row rotations.
//  5. df_t = sum over slots of dg s.
// Rows and columns of the state are independent in the recurrence, so the passes split a
// head's state by slot groups (dq, u are row dot products) or by column tiles (dv sums the
// slots of a column) without any exchange between workgroups.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p, long i) {
    return Elem<T>::load(p, i);
}

// sum over the 16 lanes of a row by DPP row rotations (every lane gets the sum)
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_sum(float x) {
    x = dpp_add<0x128>(x);  // row_ror:8
    x = dpp_add<0x124>(x);  // row_ror:4
    x = dpp_add<0x122>(x);  // row_ror:2
    return dpp_add<0x121>(x);  // row_ror:1
}

template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
    [&]<int... J>(std::integer_sequence<int, J...>) { (f(std::integral_constant<int, J>{}), ...); }
    (std::make_integer_sequence<int, N>{});
}

// dense alpha and s of the selected slots (alpha = 1, s = 0 elsewhere): 256 / M rows per block,
// thread = (row, slot); each thread scans its row's K selected slots
__global__ __launch_bounds__(256) void dense_route_kernel(const int32_t* __restrict__ idx,
                                                          const float* __restrict__ score, const float* __restrict__ f,
                                                          long rows, int M, int K, float* __restrict__ a_d,
                                                          float* __restrict__ s_d) {
    const int rpb = 256 / M;
    const long r = long(blockIdx.x) * rpb + threadIdx.x / M;
    const int i = threadIdx.x % M;
    if (r >= rows) return;
    float a = 1.0f, sv = 0.0f;
    const float ft = f[r];
    for (int n = 0; n < K; ++n) {
        if (idx[r * K + n] == i) {
            sv = score[r * K + n];
            a = sv > 0.0f ? __expf(sv * ft) : 1.0f;  // as the forward router forms it
        }
    }
    a_d[r * M + i] = a;
    s_d[r * M + i] = sv;
}

constexpr int kPF = 8;  // tokens of loads in flight ahead of the one being applied

// Pass 2: rows forward.  Block = (head, group of 16 slots), 256 threads: slot 16*g + tid/16,
// columns (tid%16)*CG .. +CG.
template <typename T, int CG>
__global__ __launch_bounds__(256) void bwd_rows_fwd_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                           const float* __restrict__ H0, const float* __restrict__ dO,
                                                           const float* __restrict__ dHT,
                                                           const float* __restrict__ a_d, long T_len, int Hh,
                                                           int M, float* __restrict__ dq, float* __restrict__ Fst) {
    constexpr int Dv = 16 * CG;
    const int ng = M / 16;
    const long bh = blockIdx.x / ng;
    const int i = (blockIdx.x % ng) * 16 + threadIdx.x / 16, cg = threadIdx.x % 16;
    const long b = bh / Hh, h = bh % Hh;
    const long r0 = b * T_len * Hh + h;  // row of token t: r0 + t * Hh
    float H[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) H[c] = H0 ? H0[(bh * M + i) * Dv + cg * CG + c] : 0.0f;
    float pa[kPF], pk[kPF], pv[kPF][CG], pd[kPF][CG];
    auto load = [&](int j, long t) __attribute__((always_inline)) {
        const long row = r0 + (t < T_len ? t : T_len - 1) * Hh;  // past the end: a valid row, unused
        pa[j] = a_d[row * M + i];
        pk[j] = ld(k, row * M + i);
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            pv[j][c] = ld(v, row * Dv + cg * CG + c);
            pd[j][c] = dO[row * Dv + cg * CG + c];
        }
    };
#pragma unroll
    for (int j = 0; j < kPF; ++j) load(j, j);
    for (long t0 = 0; t0 < T_len; t0 += kPF) {
        unroll<kPF>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const long t = t0 + j;
            if (t < T_len) {
                const float a = pa[j], kw = (1.0f - a) * pk[j];
                float p = 0.0f;
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    // unselected rows (a == 1) keep their bits
                    H[c] = a != 1.0f ? fmaf(a, H[c], kw * pv[j][c]) : H[c];
                    p = fmaf(pd[j][c], H[c], p);
                }
                p = row16_sum(p);
                if (cg == 0) dq[(r0 + t * Hh) * M + i] = p;
            }
            load(j, t + kPF);
        });
    }
    float F = 0.0f;
    if (dHT) {
#pragma unroll
        for (int c = 0; c < CG; ++c) F = fmaf(dHT[(bh * M + i) * Dv + cg * CG + c], H[c], F);
    }
    F = row16_sum(F);
    if (cg == 0) Fst[bh * M + i] = F;
}

// Pass 3: rows backward (layout of pass 2) -> dk, dz, dg s, dH0.
template <typename T, int CG>
__global__ __launch_bounds__(256) void bwd_rows_rev_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const float* __restrict__ f,
                                                           const float* __restrict__ dO, const float* __restrict__ dHT,
                                                           const float* __restrict__ a_d, const float* __restrict__ s_d,
                                                           const float* __restrict__ dq, const float* __restrict__ Fst,
                                                           long T_len, int Hh, int M, float* __restrict__ dk,
                                                           float* __restrict__ dz, float* __restrict__ dgs,
                                                           float* __restrict__ dH0) {
    constexpr int Dv = 16 * CG;
    const int ng = M / 16;
    const long bh = blockIdx.x / ng;
    const int i = (blockIdx.x % ng) * 16 + threadIdx.x / 16, cg = threadIdx.x % 16;
    const long b = bh / Hh, h = bh % Hh;
    const long r0 = b * T_len * Hh + h;
    float G[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) G[c] = dHT ? dHT[(bh * M + i) * Dv + cg * CG + c] : 0.0f;
    float R = Fst[bh * M + i];  // D_{t+1} - k_{t+1} dk_{t+1}, started at dH_T . H_{T-1}
    float pq[kPF], pk[kPF], pa[kPF], ps[kPF], pdq[kPF], pf[kPF], pv[kPF][CG], pd[kPF][CG];
    auto load = [&](int j, long t) __attribute__((always_inline)) {
        const long row = r0 + (t >= 0 ? t : 0) * Hh;
        pq[j] = ld(q, row * M + i);
        pk[j] = ld(k, row * M + i);
        pa[j] = a_d[row * M + i];
        ps[j] = s_d[row * M + i];
        pdq[j] = dq[row * M + i];
        pf[j] = f[row];
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            pv[j][c] = ld(v, row * Dv + cg * CG + c);
            pd[j][c] = dO[row * Dv + cg * CG + c];
        }
    };
#pragma unroll
    for (int j = 0; j < kPF; ++j) load(j, T_len - 1 - j);
    for (long t0 = T_len - 1; t0 >= 0; t0 -= kPF) {
        unroll<kPF>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const long t = t0 - j;
            if (t >= 0) {
                const long row = r0 + t * Hh;
                const float qi = pq[j], ki = pk[j], a = pa[j], s = ps[j];
                float u = 0.0f;
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    G[c] = fmaf(qi, pd[j][c], G[c]);
                    u = fmaf(G[c], pv[j][c], u);
                }
                u = row16_sum(u);
                const float D = fmaf(qi, pdq[j], R);
                const bool sel = s > 0.0f;
                const float dki = sel ? (1.0f - a) * u : 0.0f;
                // a = 0 (f = -inf) does not move with s or f: no decay-rate or logit gradient there
                const bool live = sel && a > 0.0f;
                const float dg = live ? D - ki * u : 0.0f;
                R = D - ki * dki;
                if (cg == 0) {
                    dk[row * M + i] = dki;
                    dz[row * M + i] = live ? dg * pf[j] * s * (1.0f - s) : 0.0f;
                    dgs[row * M + i] = dg * s;
                }
#pragma unroll
                for (int c = 0; c < CG; ++c) G[c] = a != 1.0f ? a * G[c] : G[c];
            }
            load(j, t - kPF);
        });
    }
    if (dH0) {
#pragma unroll
        for (int c = 0; c < CG; ++c) dH0[(bh * M + i) * Dv + cg * CG + c] = G[c];
    }
}

// Pass 4: columns backward.  Block = (head, tile of CT columns), 16*CT threads: column
// CT*tile + tid/16, slots (tid%16)*SPT .. +SPT.
template <typename T, int SPT, int CT>
__global__ __launch_bounds__(256) void bwd_cols_rev_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const float* __restrict__ dO, const float* __restrict__ dHT,
                                                           const float* __restrict__ a_d, long T_len, int Hh, int Dv,
                                                           float* __restrict__ dv) {
    constexpr int M = 16 * SPT;
    const int nt = Dv / CT;
    const long bh = blockIdx.x / nt;
    const int c = (blockIdx.x % nt) * CT + threadIdx.x / 16, sg = threadIdx.x % 16;
    const long b = bh / Hh, h = bh % Hh;
    const long r0 = b * T_len * Hh + h;
    float G[SPT];
#pragma unroll
    for (int j = 0; j < SPT; ++j) G[j] = dHT ? dHT[(bh * M + sg * SPT + j) * Dv + c] : 0.0f;
    float pdo[kPF], pq[kPF][SPT], pw[kPF][SPT], pa[kPF][SPT];
    auto load = [&](int j, long t) __attribute__((always_inline)) {
        const long row = r0 + (t >= 0 ? t : 0) * Hh;
        pdo[j] = dO[row * Dv + c];
#pragma unroll
        for (int x = 0; x < SPT; ++x) {
            const int i = sg * SPT + x;
            pq[j][x] = ld(q, row * M + i);
            pa[j][x] = a_d[row * M + i];
            pw[j][x] = (1.0f - pa[j][x]) * ld(k, row * M + i);
        }
    };
#pragma unroll
    for (int j = 0; j < kPF; ++j) load(j, T_len - 1 - j);
    for (long t0 = T_len - 1; t0 >= 0; t0 -= kPF) {
        unroll<kPF>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const long t = t0 - j;
            if (t >= 0) {
                float p = 0.0f;
#pragma unroll
                for (int x = 0; x < SPT; ++x) {
                    G[x] = fmaf(pq[j][x], pdo[j], G[x]);
                    p = fmaf(pw[j][x], G[x], p);
                    G[x] = pa[j][x] != 1.0f ? pa[j][x] * G[x] : G[x];
                }
                p = row16_sum(p);
                if (sg == 0) dv[(r0 + t * Hh) * Dv + c] = p;
            }
            load(j, t - kPF);
        });
    }
}

__global__ void df_kernel(const float* __restrict__ dgs, long rows, int M, float* __restrict__ df) {
    const long r = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    float acc = 0.0f;
    for (int i = 0; i < M; ++i) acc += dgs[r * M + i];
    df[r] = acc;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__global__ void zero_kernel(float* __restrict__ x, long n) {
    const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) x[i] = 0.0f;
}

}  // namespace

size_t backward_workspace(long B, long T, long Hh, int M, int K) {
    const size_t rows = size_t(B) * size_t(T) * size_t(Hh);
    return align256(rows * K * 4) * 2 + align256(rows * M * 4) * 3 + align256(size_t(B) * size_t(Hh) * M * 4);
}

int backward_launch(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                    const float* H0, const float* dO, const float* dHT, long B, long T, long Hh, int M, int Dv, int K,
                    float* dq, float* dk, float* dz, float* dv, float* df, float* dH0, void* workspace,
                    hipStream_t s) {
    const long rows = B * T * Hh, BH = B * Hh;
    if (BH == 0) return RSM_OK;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    size_t off = 0;
    auto take = [&](size_t n) {
        unsigned char* p = ws + off;
        off += align256(n);
        return p;
    };
    int32_t* idx = reinterpret_cast<int32_t*>(take(size_t(rows) * K * 4));
    float* sc = reinterpret_cast<float*>(take(size_t(rows) * K * 4));
    float* a_d = reinterpret_cast<float*>(take(size_t(rows) * M * 4));
    float* s_d = reinterpret_cast<float*>(take(size_t(rows) * M * 4));
    float* dgs = reinterpret_cast<float*>(take(size_t(rows) * M * 4));
    float* Fst = reinterpret_cast<float*>(take(size_t(BH) * M * 4));
    if (T == 0) {  // dH0 = dH_T (or zero)
        if (dH0) {
            if (dHT) {
                if (hipMemcpyAsync(dH0, dHT, size_t(BH) * M * Dv * 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
                    return RSM_ERR_HIP;
            } else {
                hipLaunchKernelGGL(zero_kernel, dim3(unsigned((BH * M * Dv + 255) / 256)), dim3(256), 0, s, dH0,
                                   BH * M * Dv);
            }
        }
        return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
    }
    const RouterOpts op{0, 0, 0, nullptr};
    int st = route_topk_launch(z, dtype, rows, M, K, idx, sc, op, s);
    if (st != RSM_OK) return st;
    const long rpb = 256 / M;
    hipLaunchKernelGGL(dense_route_kernel, dim3(unsigned((rows + rpb - 1) / rpb)), dim3(256), 0, s, idx, sc, f, rows,
                       M, K, a_d, s_d);
    const bool bf = dtype == RSM_BF16;
    const unsigned gr = unsigned(BH * (M / 16)), gc = unsigned(BH * (Dv / 16));
#define RSM_ROWS(CGV)                                                                                                 \
    if (bf) {                                                                                                         \
        hipLaunchKernelGGL((bwd_rows_fwd_kernel<bf16_t, CGV>), dim3(gr), dim3(256), 0, s,                             \
                           static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), H0, dO, dHT, a_d, T,        \
                           int(Hh), M, dq, Fst);                                                                      \
        hipLaunchKernelGGL((bwd_rows_rev_kernel<bf16_t, CGV>), dim3(gr), dim3(256), 0, s,                             \
                           static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),                              \
                           static_cast<const bf16_t*>(v), f, dO, dHT, a_d, s_d, dq, Fst, T, int(Hh), M, dk, dz,      \
                           dgs, dH0);                                                                                 \
    } else {                                                                                                          \
        hipLaunchKernelGGL((bwd_rows_fwd_kernel<float, CGV>), dim3(gr), dim3(256), 0, s,                              \
                           static_cast<const float*>(k), static_cast<const float*>(v), H0, dO, dHT, a_d, T, int(Hh), \
                           M, dq, Fst);                                                                               \
        hipLaunchKernelGGL((bwd_rows_rev_kernel<float, CGV>), dim3(gr), dim3(256), 0, s, static_cast<const float*>(q), \
                           static_cast<const float*>(k), static_cast<const float*>(v), f, dO, dHT, a_d, s_d, dq, Fst, \
                           T, int(Hh), M, dk, dz, dgs, dH0);                                                          \
    }
    switch (Dv) {
        case 16: RSM_ROWS(1) break;
        case 32: RSM_ROWS(2) break;
        case 64: RSM_ROWS(4) break;
        case 128: RSM_ROWS(8) break;
        case 256: RSM_ROWS(16) break;
        default: return RSM_ERR_UNSUPPORTED;
    }
#undef RSM_ROWS
#define RSM_COLS(SPTV)                                                                                                \
    if (bf)                                                                                                           \
        hipLaunchKernelGGL((bwd_cols_rev_kernel<bf16_t, SPTV, 16>), dim3(gc), dim3(256), 0, s,                        \
                           static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), dO, dHT, a_d, T, int(Hh),    \
                           Dv, dv);                                                                                   \
    else                                                                                                              \
        hipLaunchKernelGGL((bwd_cols_rev_kernel<float, SPTV, 16>), dim3(gc), dim3(256), 0, s,                         \
                           static_cast<const float*>(q), static_cast<const float*>(k), dO, dHT, a_d, T, int(Hh), Dv, \
                           dv);
    switch (M) {
        case 16: RSM_COLS(1) break;
        case 32: RSM_COLS(2) break;
        case 64: RSM_COLS(4) break;
        case 128: RSM_COLS(8) break;
        case 256: RSM_COLS(16) break;
        default: return RSM_ERR_UNSUPPORTED;
    }
#undef RSM_COLS
    hipLaunchKernelGGL(df_kernel, dim3(unsigned((rows + 255) / 256)), dim3(256), 0, s, dgs, rows, M, df);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

}  // namespace rsm
