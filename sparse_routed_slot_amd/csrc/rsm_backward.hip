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
// Passes (each walks a sequence segment of a head in order; the state stays in registers):
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
//
// Sequence segments.  Both recurrences are linear in their state, so a head's tokens are cut
// into S segments walked in parallel.  Forward: a first pass runs every segment but the last
// from a zero state (its end state dH_s and the product E_s of its alphas), the segment fold
// turns them into start states, H_start(s+1) = diag(E_s) H_start(s) + dH_s.  Backward, with
// C_s = diag(alpha_{a_s}) G_{a_s} the gradient a segment [a_s, b_s) passes to the one before
// it (C_S = dH_T): a pass runs every segment but the first from zero (its local carry) and
// C_s = local_s + diag(E_s) C_{s+1} is folded from the end.  The row identity starts a
// segment from R = C_{s+1} . H_start(s+1) per slot, the state after its last token.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "rsm_device.h"
#include "rsm_launch.h"
#include "rsm_scan_args.h"

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
// thread = (row, slot).  The block's rows' idx and scores are staged in LDS (one coalesced
// read), then each thread scans its row's K entries there.
__global__ __launch_bounds__(256) void dense_route_kernel(const int32_t* __restrict__ idx,
                                                          const float* __restrict__ score, const float* __restrict__ f,
                                                          long rows, int M, int K, float* __restrict__ a_d,
                                                          float* __restrict__ s_d) {
    __shared__ int sIdx[256];  // the block's rows * K <= (256 / M) * M entries
    __shared__ float sSc[256];
    const int rpb = 256 / M;
    const long r0 = long(blockIdx.x) * rpb;
    const long nr = rows - r0 < rpb ? rows - r0 : rpb;  // rows of this block
    const int ne = int(nr) * K;                          // <= 256 (K <= M, rpb * M = 256)
    for (int e = threadIdx.x; e < ne; e += 256) {
        sIdx[e] = idx[r0 * K + e];
        sSc[e] = score[r0 * K + e];
    }
    __syncthreads();
    const int rl = threadIdx.x / M, i = threadIdx.x % M;
    if (rl >= nr) return;
    const long r = r0 + rl;
    float a = 1.0f, sv = 0.0f;
    const float ft = f[r];
    for (int n = 0; n < K; ++n) {
        if (sIdx[rl * K + n] == i) {
            sv = sSc[rl * K + n];
            a = sv > 0.0f ? __expf(sv * ft) : 1.0f;  // as the forward router forms it
        }
    }
    a_d[r * M + i] = a;
    s_d[r * M + i] = sv;
}

constexpr int kPF = 8;  // tokens of loads in flight ahead of the one being applied

// Segments of the backward passes: S of them per head, L tokens each (the last may be short).
struct BwdSeg {
    int S;
    long L;
    float* Hs;  // [B*Hh][S-1][M][Dv]: forward end states from zero, folded into start states
    float* Es;  // [B*Hh][S-1][M]: alpha products of the segments
    float* Gs;  // [B*Hh][S-1][M][Dv]: backward carries, slot j for segment S-1-j, folded
    float* Ps;  // [B*Hh][S-1][M]
};

// Pass 2: rows forward.  Block = (head, group of 16 slots, segment), 256 threads: slot
// 16*g + tid/16, columns (tid%16)*CG .. +CG.  PRE: segments 0 .. S-2 from a zero state, their
// end states and alpha products into Hs / Es (nothing else); else every segment from its
// start state (H0, or the folded Hs), dq, and after the last one dH_T . H_{T-1} per slot.
template <typename T, int CG, bool PRE>
__global__ __launch_bounds__(256) void bwd_rows_fwd_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                           const float* __restrict__ H0, const float* __restrict__ dO,
                                                           const float* __restrict__ dHT,
                                                           const float* __restrict__ a_d, long T_len, int Hh,
                                                           int M, BwdSeg sg, float* __restrict__ dq,
                                                           float* __restrict__ Fst) {
    constexpr int Dv = 16 * CG;
    const int ng = M / 16;
    const int nsb = PRE ? sg.S - 1 : sg.S;
    const int seg = blockIdx.x % nsb;
    const long bh = (blockIdx.x / nsb) / ng;
    const int i = ((blockIdx.x / nsb) % ng) * 16 + threadIdx.x / 16, cg = threadIdx.x % 16;
    const long b = bh / Hh, h = bh % Hh;
    const long r0 = b * T_len * Hh + h;  // row of token t: r0 + t * Hh
    const long ta = seg * sg.L, tb = ta + sg.L < T_len ? ta + sg.L : T_len;
    float H[CG];
    {
        const float* hs = PRE ? nullptr : seg > 0 ? sg.Hs + ((bh * (sg.S - 1) + seg - 1) * M + i) * Dv : H0 ? H0 + (bh * M + i) * Dv : nullptr;
#pragma unroll
        for (int c = 0; c < CG; ++c) H[c] = hs ? hs[cg * CG + c] : 0.0f;
    }
    float E = 1.0f;
    float pa[kPF], pk[kPF], pv[kPF][CG], pd[kPF][CG];
    auto load = [&](int j, long t) __attribute__((always_inline)) {
        const long row = r0 + (t < tb ? t : tb - 1) * Hh;  // past the segment: a valid row, unused
        // (row pointers are uniform over the block: scalar base + 32-bit lane offset)
        pa[j] = (a_d + row * M)[i];
        pk[j] = ld(k + row * M, i);
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            pv[j][c] = ld(v + row * Dv, cg * CG + c);
            if (!PRE) pd[j][c] = (dO + row * Dv)[cg * CG + c];
        }
    };
#pragma unroll
    for (int j = 0; j < kPF; ++j) load(j, ta + j);
    for (long t0 = ta; t0 < tb; t0 += kPF) {
        unroll<kPF>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const long t = t0 + j;
            if (t < tb) {
                const float a = pa[j], kw = (1.0f - a) * pk[j];
                float p = 0.0f;
#pragma unroll
                for (int c = 0; c < CG; ++c) {
                    // (an unselected row, a = 1 and kw = 0, keeps its value; the state here only
                    // feeds gradients, so no select for the sign of a zero)
                    H[c] = fmaf(a, H[c], kw * pv[j][c]);
                    if (!PRE) p = fmaf(pd[j][c], H[c], p);
                }
                if (PRE) {
                    E *= a;
                } else {
                    p = row16_sum(p);
                    if (cg == 0) (dq + (r0 + t * Hh) * M)[i] = p;
                }
            }
            load(j, t + kPF);
        });
    }
    if (PRE) {
        const long sr = (bh * (sg.S - 1) + seg) * M + i;
#pragma unroll
        for (int c = 0; c < CG; ++c) sg.Hs[sr * Dv + cg * CG + c] = H[c];
        if (cg == 0) sg.Es[sr] = E;
        return;
    }
    if (seg != sg.S - 1) return;
    float F = 0.0f;
    if (dHT) {
#pragma unroll
        for (int c = 0; c < CG; ++c) F = fmaf(dHT[(bh * M + i) * Dv + cg * CG + c], H[c], F);
    }
    F = row16_sum(F);
    if (cg == 0) Fst[bh * M + i] = F;
}

// Pass 3: rows backward (layout of pass 2) -> dk, dz, dg s, dH0.  PRE: segments 1 .. S-1 from
// a zero carry, their local carries and alpha products into Gs / Ps (slot S-1-s); else every
// segment from its carry (dH_T, or the folded Gs) with the outputs.
// (the rows-backward pass keeps four tokens of loads in flight: with eight its many
// per-token scalars spill scalar registers)
constexpr int kPFR = 4;

template <typename T, int CG, bool PRE>
__global__ __launch_bounds__(256) void bwd_rows_rev_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const float* __restrict__ f,
                                                           const float* __restrict__ dO, const float* __restrict__ dHT,
                                                           const float* __restrict__ a_d, const float* __restrict__ s_d,
                                                           const float* __restrict__ dq, const float* __restrict__ Fst,
                                                           long T_len, int Hh, int M, BwdSeg sg,
                                                           float* __restrict__ dk, float* __restrict__ dz,
                                                           float* __restrict__ dgs, float* __restrict__ dH0) {
    constexpr int Dv = 16 * CG;
    const int ng = M / 16;
    const int nsb = PRE ? sg.S - 1 : sg.S;
    const int seg = PRE ? 1 + int(blockIdx.x % nsb) : int(blockIdx.x % nsb);
    const long bh = (blockIdx.x / nsb) / ng;
    const int i = ((blockIdx.x / nsb) % ng) * 16 + threadIdx.x / 16, cg = threadIdx.x % 16;
    const long b = bh / Hh, h = bh % Hh;
    const long r0 = b * T_len * Hh + h;
    const long ta = seg * sg.L, tb = ta + sg.L < T_len ? ta + sg.L : T_len;
    float G[CG];
    float R = 0.0f;  // D_{t+1} - k_{t+1} dk_{t+1}: carry . state after the segment's last token
    if (!PRE) {
        const bool last = seg == sg.S - 1;
        const float* gs = last ? (dHT ? dHT + (bh * M + i) * Dv : nullptr)
                               : sg.Gs + ((bh * (sg.S - 1) + (sg.S - 2 - seg)) * M + i) * Dv;
#pragma unroll
        for (int c = 0; c < CG; ++c) G[c] = gs ? gs[cg * CG + c] : 0.0f;
        if (last) {
            R = Fst[bh * M + i];  // dH_T . H_{T-1}
        } else {
            const float* hs = sg.Hs + ((bh * (sg.S - 1) + seg) * M + i) * Dv;  // H_start(seg + 1)
#pragma unroll
            for (int c = 0; c < CG; ++c) R = fmaf(G[c], hs[cg * CG + c], R);
            R = row16_sum(R);
        }
    } else {
#pragma unroll
        for (int c = 0; c < CG; ++c) G[c] = 0.0f;
    }
    float E = 1.0f;
    float pq[kPFR], pk[kPFR], pa[kPFR], ps[kPFR], pdq[kPFR], pf[kPFR], pv[kPFR][CG], pd[kPFR][CG];
    auto load = [&](int j, long t) __attribute__((always_inline)) {
        const long row = r0 + (t >= ta ? t : ta) * Hh;
        pq[j] = ld(q, row * M + i);
        pa[j] = a_d[row * M + i];
        if (!PRE) {
            pk[j] = ld(k, row * M + i);
            ps[j] = s_d[row * M + i];
            pdq[j] = dq[row * M + i];
            pf[j] = f[row];
        }
#pragma unroll
        for (int c = 0; c < CG; ++c) {
            if (!PRE) pv[j][c] = ld(v, row * Dv + cg * CG + c);
            pd[j][c] = dO[row * Dv + cg * CG + c];
        }
    };
#pragma unroll
    for (int j = 0; j < kPFR; ++j) load(j, tb - 1 - j);
    for (long t0 = tb - 1; t0 >= ta; t0 -= kPFR) {
        unroll<kPFR>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const long t = t0 - j;
            if (t >= ta) {
                const long row = r0 + t * Hh;
                const float qi = pq[j], a = pa[j];
#pragma unroll
                for (int c = 0; c < CG; ++c) G[c] = fmaf(qi, pd[j][c], G[c]);
                if (!PRE) {
                    const float ki = pk[j], s = ps[j];
                    float u = 0.0f;
#pragma unroll
                    for (int c = 0; c < CG; ++c) u = fmaf(G[c], pv[j][c], u);
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
                } else {
                    E *= a;
                }
                // (a gradient, not a state: multiplying by a = 1 leaves it unchanged exactly)
#pragma unroll
                for (int c = 0; c < CG; ++c) G[c] *= a;
            }
            load(j, t - kPFR);
        });
    }
    if (PRE) {
        const long sr = (bh * (sg.S - 1) + (sg.S - 1 - seg)) * M + i;
#pragma unroll
        for (int c = 0; c < CG; ++c) sg.Gs[sr * Dv + cg * CG + c] = G[c];
        if (cg == 0) sg.Ps[sr] = E;
        return;
    }
    if (dH0 && seg == 0) {
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
                                                           BwdSeg bs, float* __restrict__ dv) {
    constexpr int M = 16 * SPT;
    const int nt = Dv / CT;
    const int seg = blockIdx.x % bs.S;
    const long bh = (blockIdx.x / bs.S) / nt;
    const int c = ((blockIdx.x / bs.S) % nt) * CT + threadIdx.x / 16, sg = threadIdx.x % 16;
    const long b = bh / Hh, h = bh % Hh;
    const long r0 = b * T_len * Hh + h;
    const long ta = seg * bs.L, tb = ta + bs.L < T_len ? ta + bs.L : T_len;
    float G[SPT];
    {
        const bool last = seg == bs.S - 1;
        const float* gs = last ? (dHT ? dHT + bh * M * Dv : nullptr)
                               : bs.Gs + (bh * (bs.S - 1) + (bs.S - 2 - seg)) * M * Dv;
#pragma unroll
        for (int j = 0; j < SPT; ++j) G[j] = gs ? gs[(sg * SPT + j) * Dv + c] : 0.0f;
    }
    float pdo[kPF], pq[kPF][SPT], pw[kPF][SPT], pa[kPF][SPT];
    auto load = [&](int j, long t) __attribute__((always_inline)) {
        const long row = r0 + (t >= ta ? t : ta) * Hh;
        pdo[j] = (dO + row * Dv)[c];
#pragma unroll
        for (int x = 0; x < SPT; ++x) {
            const int i = sg * SPT + x;
            pq[j][x] = ld(q + row * M, i);
            pa[j][x] = (a_d + row * M)[i];
            pw[j][x] = (1.0f - pa[j][x]) * ld(k + row * M, i);
        }
    };
#pragma unroll
    for (int j = 0; j < kPF; ++j) load(j, tb - 1 - j);
    for (long t0 = tb - 1; t0 >= ta; t0 -= kPF) {
        unroll<kPF>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value;
            const long t = t0 - j;
            if (t >= ta) {
                float p = 0.0f;
#pragma unroll
                for (int x = 0; x < SPT; ++x) {
                    G[x] = fmaf(pq[j][x], pdo[j], G[x]);
                    p = fmaf(pw[j][x], G[x], p);
                    G[x] *= pa[j][x];  // (a = 1 leaves it unchanged exactly)
                }
                p = row16_sum(p);
                if (sg == 0) dv[(r0 + t * Hh) * Dv + c] = p;
            }
            load(j, t - kPF);
        });
    }
}

// Pass 4 for M <= 64: columns backward with a lane per (column, half of the slots).  Block =
// (head, segment, 128 columns), 256 threads: column 128*tile + (lane % 32) + 32*(wave), slots
// h*M/2 .. +M/2 with h = lane / 32, the thread's column of G for those slots in registers.
// The slot data of a block of TB tokens (q, w = (1 - alpha) k, alpha, as fp32) is staged in
// LDS by the whole block and read back as broadcasts; dO of the thread's column is read into
// registers per block.  dv_t = sum over slots of w_t G_t (after the q_t dO_t update): the two
// halves' partial sums meet by a lane exchange.
template <typename T, int M>
__global__ __launch_bounds__(256) void bwd_cols_lane_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                            const float* __restrict__ dO,
                                                            const float* __restrict__ dHT,
                                                            const float* __restrict__ a_d, long T_len, int Hh, int Dv,
                                                            BwdSeg bs, float* __restrict__ dv) {
    constexpr int TB = 32, HM = M / 2;
    __shared__ __align__(16) float sQ[TB * M];
    __shared__ __align__(16) float sW[TB * M];
    __shared__ __align__(16) float sA[TB * M];
    const int nt = (Dv + 127) / 128;
    const int seg = blockIdx.x % bs.S;
    const long bh = (blockIdx.x / bs.S) / nt;
    const int tile = (blockIdx.x / bs.S) % nt;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int c = tile * 128 + wv * 32 + (lane & 31);
    const bool col_ok = c < Dv;
    const long b = bh / Hh, hh = bh % Hh;
    const long r0 = b * T_len * Hh + hh;
    const long ta = seg * bs.L, tb = ta + bs.L < T_len ? ta + bs.L : T_len;
    float G[HM];
    {
        const bool last = seg == bs.S - 1;
        const float* gs = last ? (dHT ? dHT + bh * M * Dv : nullptr)
                               : bs.Gs + (bh * (bs.S - 1) + (bs.S - 2 - seg)) * M * Dv;
#pragma unroll
        for (int x = 0; x < HM; ++x) G[x] = (gs && col_ok) ? gs[(h * HM + x) * Dv + c] : 0.0f;
    }
    for (long t1 = tb; t1 > ta; t1 -= TB) {  // blocks of tokens [t0, t1), from the end
        const long t0 = t1 - TB > ta ? t1 - TB : ta;
        const int nb = int(t1 - t0);
        __syncthreads();  // the previous block's LDS reads are done
        for (int e = threadIdx.x; e < nb * M; e += 256) {
            const int tt = e / M, x = e % M;
            const long row = r0 + (t0 + tt) * Hh;
            const float a = (a_d + row * M)[x];
            sQ[e] = ld(q + row * M, x);
            sW[e] = (1.0f - a) * ld(k + row * M, x);
            sA[e] = a;
        }
        float d[TB];
#pragma unroll
        for (int tt = 0; tt < TB; ++tt) d[tt] = (tt < nb && col_ok) ? dO[(r0 + (t0 + tt) * Hh) * Dv + c] : 0.0f;
        __syncthreads();
#pragma unroll
        for (int tt = TB - 1; tt >= 0; --tt) {
            if (tt < nb) {
                const float* qv = sQ + tt * M + h * HM;
                const float* wq = sW + tt * M + h * HM;
                const float* av = sA + tt * M + h * HM;
                float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
                for (int x = 0; x < HM; x += 4) {
                    const float4 q4v = *reinterpret_cast<const float4*>(qv + x);
                    const float4 w4v = *reinterpret_cast<const float4*>(wq + x);
                    const float4 a4v = *reinterpret_cast<const float4*>(av + x);
                    G[x] = fmaf(q4v.x, d[tt], G[x]);
                    G[x + 1] = fmaf(q4v.y, d[tt], G[x + 1]);
                    G[x + 2] = fmaf(q4v.z, d[tt], G[x + 2]);
                    G[x + 3] = fmaf(q4v.w, d[tt], G[x + 3]);
                    p0 = fmaf(w4v.x, G[x], p0);
                    p1 = fmaf(w4v.y, G[x + 1], p1);
                    p0 = fmaf(w4v.z, G[x + 2], p0);
                    p1 = fmaf(w4v.w, G[x + 3], p1);
                    G[x] *= a4v.x;  // (a = 1 leaves it unchanged exactly)
                    G[x + 1] *= a4v.y;
                    G[x + 2] *= a4v.z;
                    G[x + 3] *= a4v.w;
                }
                float p = p0 + p1;
                p += __shfl_xor(p, 32);
                if (h == 0 && col_ok) dv[(r0 + (t0 + tt) * Hh) * Dv + c] = p;
            }
        }
    }
}

// df_t = sum over slots of dg s: 16 lanes per row, each summing M/16 consecutive slots, then
// a DPP sum over the 16 lanes (a block of 256 threads takes 16 rows, reads coalesced).
__global__ __launch_bounds__(256) void df_kernel(const float* __restrict__ dgs, long rows, int M,
                                                 float* __restrict__ df) {
    const long r = long(blockIdx.x) * 16 + threadIdx.x / 16;
    const int l = threadIdx.x % 16, per = M / 16;
    float acc = 0.0f;
    if (r < rows)
        for (int x = 0; x < per; ++x) acc += dgs[r * M + l * per + x];
    acc = row16_sum(acc);
    if (r < rows && l == 0) df[r] = acc;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

__global__ void zero_kernel(float* __restrict__ x, long n) {
    const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) x[i] = 0.0f;
}

}  // namespace

template <typename X>
struct ElemTag {
    using type = X;
};

// Segments per head: enough workgroups for the rows passes (about 2048: eight per compute
// unit), at least 64 tokens per segment, a power of two.
static int bwd_segments(long BH, long T, int M) {
    const long wg = BH * (M / 16);
    int S = 1;
    while (wg * S < 2048 && (T / (2 * S)) >= 64) S *= 2;
    return S;
}

size_t backward_workspace(long B, long T, long Hh, int M, int Dv, int K) {
    const size_t rows = size_t(B) * size_t(T) * size_t(Hh), BH = size_t(B) * size_t(Hh);
    const int S = bwd_segments(long(BH), T, M);
    const size_t segs = BH * size_t(S - 1);
    return align256(rows * K * 4) * 2 + align256(rows * M * 4) * 3 + align256(BH * M * 4) +
           2 * (align256(segs * M * Dv * 4) + align256(segs * M * 4));
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
    BwdSeg bs{};
    bs.S = bwd_segments(BH, T, M);
    bs.L = (T + bs.S - 1) / bs.S;
    {
        const size_t segs = size_t(BH) * size_t(bs.S - 1);
        bs.Hs = reinterpret_cast<float*>(take(segs * M * Dv * 4));
        bs.Es = reinterpret_cast<float*>(take(segs * M * 4));
        bs.Gs = reinterpret_cast<float*>(take(segs * M * Dv * 4));
        bs.Ps = reinterpret_cast<float*>(take(segs * M * 4));
    }
    const RouterOpts op{0, 0, 0, nullptr};
    int st = route_topk_launch(z, dtype, rows, M, K, idx, sc, op, s);
    if (st != RSM_OK) return st;
    const long rpb = 256 / M;
    hipLaunchKernelGGL(dense_route_kernel, dim3(unsigned((rows + rpb - 1) / rpb)), dim3(256), 0, s, idx, sc, f, rows,
                       M, K, a_d, s_d);
    const bool bf = dtype == RSM_BF16;
    const unsigned gr = unsigned(BH * (M / 16) * bs.S), gc = unsigned(BH * (Dv / 16) * bs.S);
    const unsigned gp = unsigned(BH * (M / 16) * (bs.S - 1));  // the passes over all segments but one
    // fold of the segments' (alpha product, state) pairs: forward from H0, backward from dH_T
    const SegArgs fold_f{0, bs.S, 0, bs.Hs, bs.Es}, fold_b{0, bs.S, 0, bs.Gs, bs.Ps};
    auto rows_passes = [&](auto tag, auto cgc) -> int {
        using EL = typename decltype(tag)::type;
        constexpr int CGV = decltype(cgc)::value;
        const EL *qq = static_cast<const EL*>(q), *kk = static_cast<const EL*>(k), *vv = static_cast<const EL*>(v);
        if (bs.S > 1) {
            hipLaunchKernelGGL((bwd_rows_fwd_kernel<EL, CGV, true>), dim3(gp), dim3(256), 0, s, kk, vv, H0, dO, dHT, a_d,
                               T, int(Hh), M, bs, dq, Fst);
            if (seg_fold_launch(H0, fold_f, BH, M, Dv, s) != RSM_OK) return RSM_ERR_HIP;
        }
        hipLaunchKernelGGL((bwd_rows_fwd_kernel<EL, CGV, false>), dim3(gr), dim3(256), 0, s, kk, vv, H0, dO, dHT, a_d, T,
                           int(Hh), M, bs, dq, Fst);
        if (bs.S > 1) {
            hipLaunchKernelGGL((bwd_rows_rev_kernel<EL, CGV, true>), dim3(gp), dim3(256), 0, s, qq, kk, vv, f, dO, dHT,
                               a_d, s_d, dq, Fst, T, int(Hh), M, bs, dk, dz, dgs, dH0);
            if (seg_fold_launch(dHT, fold_b, BH, M, Dv, s, false) != RSM_OK) return RSM_ERR_HIP;
        }
        hipLaunchKernelGGL((bwd_rows_rev_kernel<EL, CGV, false>), dim3(gr), dim3(256), 0, s, qq, kk, vv, f, dO, dHT, a_d,
                           s_d, dq, Fst, T, int(Hh), M, bs, dk, dz, dgs, dH0);
        return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
    };
    auto rows_dv = [&](auto tag) -> int {
        switch (Dv) {
            case 16: return rows_passes(tag, std::integral_constant<int, 1>{});
            case 32: return rows_passes(tag, std::integral_constant<int, 2>{});
            case 64: return rows_passes(tag, std::integral_constant<int, 4>{});
            case 128: return rows_passes(tag, std::integral_constant<int, 8>{});
            case 256: return rows_passes(tag, std::integral_constant<int, 16>{});
        }
        return RSM_ERR_UNSUPPORTED;
    };
    st = bf ? rows_dv(ElemTag<bf16_t>{}) : rows_dv(ElemTag<float>{});
    if (st != RSM_OK) return st;
#define RSM_COLS(SPTV)                                                                                                \
    if (bf)                                                                                                           \
        hipLaunchKernelGGL((bwd_cols_rev_kernel<bf16_t, SPTV, 16>), dim3(gc), dim3(256), 0, s,                        \
                           static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), dO, dHT, a_d, T, int(Hh),    \
                           Dv, bs, dv);                                                                               \
    else                                                                                                              \
        hipLaunchKernelGGL((bwd_cols_rev_kernel<float, SPTV, 16>), dim3(gc), dim3(256), 0, s,                         \
                           static_cast<const float*>(q), static_cast<const float*>(k), dO, dHT, a_d, T, int(Hh), Dv, \
                           bs, dv);
    const unsigned gl = unsigned(BH * ((Dv + 127) / 128) * bs.S);
#define RSM_COLS_LANE(MV)                                                                                            \
    if (bf)                                                                                                          \
        hipLaunchKernelGGL((bwd_cols_lane_kernel<bf16_t, MV>), dim3(gl), dim3(256), 0, s,                            \
                           static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), dO, dHT, a_d, T, int(Hh),   \
                           Dv, bs, dv);                                                                              \
    else                                                                                                             \
        hipLaunchKernelGGL((bwd_cols_lane_kernel<float, MV>), dim3(gl), dim3(256), 0, s,                             \
                           static_cast<const float*>(q), static_cast<const float*>(k), dO, dHT, a_d, T, int(Hh), Dv, \
                           bs, dv);
    switch (M) {
        case 16: RSM_COLS_LANE(16) break;
        case 32: RSM_COLS_LANE(32) break;
        case 64: RSM_COLS_LANE(64) break;
        case 128: RSM_COLS(8) break;
        case 256: RSM_COLS(16) break;
        default: return RSM_ERR_UNSUPPORTED;
    }
#undef RSM_COLS_LANE
#undef RSM_COLS
    hipLaunchKernelGGL(df_kernel, dim3(unsigned((rows + 15) / 16)), dim3(256), 0, s, dgs, rows, M, df);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

}  // namespace rsm
