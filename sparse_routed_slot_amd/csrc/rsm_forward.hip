// rsm_forward.hip -- chunked forward of the RSM mixer: route, sparse decay, intra-chunk
// and chunk-state contractions on MFMA, inter-chunk state scan.
//
// The method (Raven README page, "How Raven Works"): per token the top-K slots by sigmoid
// score are decayed by alpha = exp(s*f) and written with (1-alpha)*k_i*v, and o = q . H is
// read after the update.  The Raven paper summary (appendix A.5) evaluates it chunkwise,
// T = n*C.  Unrolling the recurrence over a chunk that starts from state H_c, with the
// per-slot cumulative log-decay b_t = sum_{tau <= t} g_tau taken from the chunk start
// (g = s*f on selected slots, 0 elsewhere) and k~ = (1-alpha)*k:
//
//     o_t     = sum_i q_ti e^{b_ti} H_c[i,:] + sum_{j<=t} ( sum_i q_ti e^{b_ti - b_ji} k~_ji ) v_j
//     H_{c+1} = diag(e^{b_last}) ( H_c + sum_j diag(e^{-b_j}) k~_j v_j^T )
//
// Factoring e^{b_t - b_j} = e^{b_t} e^{-b_j} turns the double sum into dense products of
// Qh = q o e^{b} and Kh = k~ o e^{-b}:  O^T = V^T P^T + H_c^T Qh^T with P = tril(Qh Kh^T),
// and U^T = V^T Kh gives the state update H_{c+1} = diag(e^{b_last}) (H_c + U).
//
// Two kernels:
//  * fwd_prep (one workgroup per (batch, head, chunk), fully parallel): routes every token
//    (wave64 exact top-K), forms e^{b} as running products of the clamped per-step decay,
//    and writes Qh, Kh (input precision) and e^{b_last} to the workspace.  Doing this once
//    per chunk keeps the router and the exponentials off the sequential scan.
//  * fwd_scan (one workgroup per (batch, head, Dv tile)): walks the chunks in order with
//    the fp32 state tile in registers, runs the three contractions on MFMA 16x16 tiles
//    from LDS, writes o, and applies the state update.  Rows of slots untouched in a chunk
//    (e^{b_last} == 1) are not written, so they keep their exact bits.
//
// Overflow guard: e^{-b_j} grows with the decay accumulated in a chunk.  The per-step
// log-decay is clamped at -30 on the factored path (alpha = e^{-30} ~ 1e-13 instead of
// 0), and a chunk whose decay product for any slot falls below 2^-100 is flagged; the
// scan evaluates such a chunk token by token with the exact alphas instead.
#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

constexpr float kGMin = -30.0f;               // clamp of s*f on the factored path
constexpr float kSafeMin = 7.8886091e-31f;    // 2^-100, smallest e^{b_last} kept factored

template <typename T> __device__ __forceinline__ T to_elem(float x);
template <> __device__ __forceinline__ float to_elem<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t to_elem<bf16_t>(float x) { return bf16_t{float_to_bf16(x)}; }

// ------------------------------------------------------------------------------------
// MFMA traits: 16x16 output tiles; a k-block of KB along the contraction, EPL = KB/4
// consecutive k per lane (lane l holds row/col l%16 and k = EPL*(l/16) + e).
// ------------------------------------------------------------------------------------
template <typename T> struct MfmaT;

template <> struct MfmaT<bf16_t> {
    static constexpr int KB = 32, EPL = 8;
    typedef bf16x8 frag;
    __device__ static __forceinline__ frag load_row(const bf16_t* p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
    }
    // k-slot f = kb*EPL + e of a contraction over chunk rows j maps to j = 16(f/4) + 4*q4 + f%4:
    // two runs of four consecutive j.
    __device__ static __forceinline__ frag load_perm(const bf16_t* row, int kb, int q4) {
        const uint2 a = *reinterpret_cast<const uint2*>(row + 32 * kb + 4 * q4);
        const uint2 b = *reinterpret_cast<const uint2*>(row + 32 * kb + 16 + 4 * q4);
        return __builtin_bit_cast(frag, make_uint4(a.x, a.y, b.x, b.y));
    }
    template <int NT>
    __device__ static __forceinline__ frag pack_perm(const floatx4 (&st)[NT], int kb) {
        const floatx4 x = st[2 * kb], y = st[2 * kb + 1];
        uint4 u;
        u.x = uint32_t(float_to_bf16(x[0])) | (uint32_t(float_to_bf16(x[1])) << 16);
        u.y = uint32_t(float_to_bf16(x[2])) | (uint32_t(float_to_bf16(x[3])) << 16);
        u.z = uint32_t(float_to_bf16(y[0])) | (uint32_t(float_to_bf16(y[1])) << 16);
        u.w = uint32_t(float_to_bf16(y[2])) | (uint32_t(float_to_bf16(y[3])) << 16);
        return __builtin_bit_cast(frag, u);
    }
    __device__ static __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct MfmaT<float> {
    static constexpr int KB = 4, EPL = 1;
    typedef float frag;
    __device__ static __forceinline__ frag load_row(const float* p) { return *p; }
    __device__ static __forceinline__ frag load_perm(const float* row, int kb, int q4) {
        return row[16 * (kb >> 2) + 4 * q4 + (kb & 3)];
    }
    template <int NT>
    __device__ static __forceinline__ frag pack_perm(const floatx4 (&st)[NT], int kb) {
        return st[kb >> 2][kb & 3];
    }
    __device__ static __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// LDS plan of the scan kernel (element pitches padded by one 16-byte vector).
template <typename T, int M, int C, int DT>
struct ScanCfg {
    static constexpr int KB = MfmaT<T>::KB;
    static constexpr int MP = M > KB ? M : KB;  // padded slot dimension
    static constexpr int CP = C > KB ? C : KB;  // padded chunk dimension
    static constexpr int EV = 16 / int(sizeof(T));
    static constexpr int QP = MP + EV;  // pitch of sQ, sK, sHt rows
    static constexpr int TP = CP + EV;  // pitch of sKt, sVt rows
    static constexpr int szQ = C * QP * int(sizeof(T));
    static constexpr int szHf = M * DT * 4;
    static constexpr int reg0 = (2 * szQ > szHf ? 2 * szQ : szHf);
    static constexpr int offQ = 0;
    static constexpr int offK = szQ;
    static constexpr int offKt = (reg0 + 15) / 16 * 16;
    static constexpr int offVt = offKt + MP * TP * int(sizeof(T));
    static constexpr int offHt = offVt + DT * TP * int(sizeof(T));
    static constexpr int offE = offHt + DT * QP * int(sizeof(T));
    static constexpr int total = (offE + M * 4 + 15) / 16 * 16;
};

// ------------------------------------------------------------------------------------
// Prep: one workgroup per (b, h, chunk); wave w owns tokens [w*C/4, (w+1)*C/4) of the chunk,
// lane = slot (slots r*64 + lane in register r).
// ------------------------------------------------------------------------------------
template <typename T, int M, int C>
__global__ __launch_bounds__(256) void fwd_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ z, const float* __restrict__ f,
    long T_len, int Hh, int K, long nC, T* __restrict__ tiles, float* __restrict__ elast,
    int* __restrict__ flags, int32_t* __restrict__ idx_out) {
    constexpr int SPL = M > kWave ? M / kWave : 1;
    constexpr int NB = Elem<T>::kKeyBits;
    constexpr int TPW = C / 4;
    __shared__ float s_tot[4][SPL * kWave];
    const int lane = lane_id(), w = threadIdx.x >> 6;
    const long bhc = blockIdx.x;
    const long c = bhc % nC, bh = bhc / nC;
    const long h = bh % Hh, b = bh / Hh;
    const long tok0 = c * C + w * TPW;

    float g[TPW][SPL];  // s*f on selected slots (may be -inf), 0 elsewhere
    float E[TPW][SPL];  // running product of the clamped decay inside this wave's tokens
    float run[SPL];
#pragma unroll
    for (int r = 0; r < SPL; ++r) run[r] = 1.0f;

#pragma unroll
    for (int tt = 0; tt < TPW; ++tt) {
        const long tok = tok0 + tt;
        if (tok < T_len) {
            const long row = (b * T_len + tok) * Hh + h;
            uint32_t key[SPL];
            float zv[SPL];
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = r * kWave + lane;
                zv[r] = slot < M ? Elem<T>::load(z + row * M, slot) : 0.0f;
                key[r] = slot < M ? order_key<NB>(zv[r]) : 0u;
            }
            bool sel[SPL];
            wave_topk<SPL, NB>(key, K, sel);
            const float ft = f[row];
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                float gg = 0.0f;
                if (sel[r]) {
                    const float s = sigmoidf_dev(zv[r]);
                    if (s > 0.0f) gg = s * ft;
                }
                g[tt][r] = gg;
            }
            if (idx_out) {
                int pos[SPL];
                wave_compact<SPL>(sel, pos);
#pragma unroll
                for (int r = 0; r < SPL; ++r)
                    if (sel[r]) idx_out[row * K + pos[r]] = r * kWave + lane;
            }
        } else {
#pragma unroll
            for (int r = 0; r < SPL; ++r) g[tt][r] = 0.0f;
        }
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            run[r] *= __expf(fmaxf(g[tt][r], kGMin));
            E[tt][r] = run[r];
        }
    }
#pragma unroll
    for (int r = 0; r < SPL; ++r) s_tot[w][r * kWave + lane] = run[r];
    __syncthreads();

    float pre[SPL], last[SPL];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
        const int slot = r * kWave + lane;
        float p = 1.0f, l = 1.0f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (u < w) p *= s_tot[u][slot];
            l *= s_tot[u][slot];
        }
        pre[r] = p;
        last[r] = l;
        bad |= !(l >= kSafeMin);
    }
    const bool unsafe = __ballot(bad) != 0ull;  // identical in every wave

    T* tq = tiles + bhc * 2 * C * M;
    T* tk = tq + C * M;
    if (!unsafe) {
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const long tok = tok0 + tt;
            const int trow = w * TPW + tt;
            const long row = (b * T_len + tok) * Hh + h;
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = r * kWave + lane;
                if (slot >= M) continue;
                float qh = 0.0f, kh = 0.0f;
                if (tok < T_len) {
                    const float ev = pre[r] * E[tt][r];
                    qh = Elem<T>::load(q + row * M, slot) * ev;
                    if (g[tt][r] != 0.0f) {
                        const float a = __expf(fmaxf(g[tt][r], kGMin));
                        kh = Elem<T>::load(k + row * M, slot) * (1.0f - a) * __builtin_amdgcn_rcpf(ev);
                    }
                }
                tq[trow * M + slot] = to_elem<T>(qh);
                tk[trow * M + slot] = to_elem<T>(kh);
            }
        }
        if (w == 0) {
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = r * kWave + lane;
                if (slot < M) elast[bhc * M + slot] = last[r];
            }
        }
        if (threadIdx.x == 0) flags[bhc] = 0;
    } else {
        float* ta = reinterpret_cast<float*>(tq);  // dense exact alpha [C][M] over both tiles
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int trow = w * TPW + tt;
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = r * kWave + lane;
                if (slot < M) ta[trow * M + slot] = g[tt][r] != 0.0f ? __expf(g[tt][r]) : 1.0f;
            }
        }
        if (threadIdx.x == 0) flags[bhc] = 1;
    }
}

// ------------------------------------------------------------------------------------
// Scan: one workgroup per (b, h, Dv tile of DT columns); sequential over chunks.
// ------------------------------------------------------------------------------------
template <typename T, int M, int C, int DT>
__global__ __launch_bounds__(256) void fwd_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ H0,
    long T_len, int Hh, int Dv, long nC, const T* __restrict__ tiles, const float* __restrict__ elast,
    const int* __restrict__ flags, float* __restrict__ o, float* __restrict__ H_out) {
    using Cfg = ScanCfg<T, M, C, DT>;
    using MT = MfmaT<T>;
    typedef typename MT::frag frag;
    constexpr int KB = MT::KB, EPL = MT::EPL;
    constexpr int MP = Cfg::MP, CP = Cfg::CP, QP = Cfg::QP, TP = Cfg::TP, EV = Cfg::EV;
    constexpr int NTC = C / 16, NTCP = CP / 16, NTD = DT / 16, NTM = M / 16;
    constexpr int NU = NTD * NTM, UPW = (NU + 3) / 4;
    constexpr int NKM = MP / KB, NKC = CP / KB;

    extern __shared__ __align__(16) unsigned char smem[];
    T* sQ = reinterpret_cast<T*>(smem + Cfg::offQ);
    T* sK = reinterpret_cast<T*>(smem + Cfg::offK);
    float* sHf = reinterpret_cast<float*>(smem + Cfg::offQ);  // fallback state, aliases sQ/sK
    T* sKt = reinterpret_cast<T*>(smem + Cfg::offKt);
    T* sVt = reinterpret_cast<T*>(smem + Cfg::offVt);
    T* sHt = reinterpret_cast<T*>(smem + Cfg::offHt);
    float* sE = reinterpret_cast<float*>(smem + Cfg::offE);

    // workgroup -> (head, Dv tile); the Dv tiles of one head land on the same XCD
    // (workgroups are dealt to the 8 XCDs round-robin) so they share Qh/Kh in its L2.
    const int nDT = Dv / DT;
    const long nblk = gridDim.x;
    long id = blockIdx.x;
    if (nblk % 8 == 0) id = (long(blockIdx.x) % 8) * (nblk / 8) + long(blockIdx.x) / 8;
    const long bh = id / nDT;
    const int d0 = int(id % nDT) * DT;
    const long h = bh % Hh, b = bh / Hh;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;

    for (int i = tid * 16; i < Cfg::total; i += 256 * 16)
        *reinterpret_cast<uint4*>(smem + i) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();

    // state tile u = w + 4*j holds H[i = 16*I + l16][d = 16*D + 4*q4 + r], r = 0..3
    floatx4 Hreg[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
        const int u = w + 4 * j;
        if (u < NU) {
            const int D = u / NTM, I = u % NTM, i = 16 * I + l16;
            if (H0) {
                const float4 x = *reinterpret_cast<const float4*>(H0 + (bh * M + i) * Dv + d0 + 16 * D + 4 * q4);
                Hreg[j] = floatx4{x.x, x.y, x.z, x.w};
            } else {
                Hreg[j] = floatx4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sHt[(16 * D + 4 * q4 + r) * QP + i] = to_elem<T>(Hreg[j][r]);
        }
    }

    for (long c = 0; c < nC; ++c) {
        __syncthreads();
        const long bhc = bh * nC + c;
        const int unsafe = flags[bhc];
        const long tokc = c * C;
        if (!unsafe) {
            const T* tq = tiles + bhc * 2 * C * M;
            const T* tk = tq + C * M;
            for (int p = tid; p < C * M / EV; p += 256) {
                const int row = (p * EV) / M, col = (p * EV) % M;
                const uint4 x = *reinterpret_cast<const uint4*>(tq + p * EV);
                const uint4 y = *reinterpret_cast<const uint4*>(tk + p * EV);
                *reinterpret_cast<uint4*>(sQ + row * QP + col) = x;
                *reinterpret_cast<uint4*>(sK + row * QP + col) = y;
                const T* ye = reinterpret_cast<const T*>(&y);
#pragma unroll
                for (int e = 0; e < EV; ++e) sKt[(col + e) * TP + row] = ye[e];
            }
            for (int p = tid; p < C * DT / EV; p += 256) {
                const int row = (p * EV) / DT, col = (p * EV) % DT;
                const long tok = tokc + row;
                uint4 x = make_uint4(0u, 0u, 0u, 0u);
                if (tok < T_len) x = *reinterpret_cast<const uint4*>(v + ((b * T_len + tok) * Hh + h) * Dv + d0 + col);
                const T* xe = reinterpret_cast<const T*>(&x);
#pragma unroll
                for (int e = 0; e < EV; ++e) sVt[(col + e) * TP + row] = xe[e];
            }
            for (int i = tid; i < M; i += 256) sE[i] = elast[bhc * M + i];
        }
        __syncthreads();

        if (unsafe) {
            // exact token-by-token recurrence with the dense alphas written by the prep
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int u = w + 4 * j;
                if (u < NU) {
                    const int D = u / NTM, I = u % NTM, i = 16 * I + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sHf[i * DT + 16 * D + 4 * q4 + r] = Hreg[j][r];
                }
            }
            __syncthreads();
            const float* ta = reinterpret_cast<const float*>(tiles + bhc * 2 * C * M);
            for (int tt = 0; tt < C; ++tt) {
                const long tok = tokc + tt;
                if (tok >= T_len) break;
                const long row = (b * T_len + tok) * Hh + h;
                for (int e = tid; e < M * DT; e += 256) {
                    const int i = e / DT, dd = e % DT;
                    const float a = ta[tt * M + i];
                    if (a != 1.0f) {
                        const float wk = (1.0f - a) * Elem<T>::load(k + row * M, i);
                        sHf[e] = fmaf(a, sHf[e], wk * Elem<T>::load(v + row * Dv + d0, dd));
                    }
                }
                __syncthreads();
                if (tid < DT) {
                    float acc = 0.0f;
                    for (int i = 0; i < M; ++i) acc = fmaf(Elem<T>::load(q + row * M, i), sHf[i * DT + tid], acc);
                    o[row * Dv + d0 + tid] = acc;
                }
                __syncthreads();
            }
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int u = w + 4 * j;
                if (u < NU) {
                    const int D = u / NTM, I = u % NTM, i = 16 * I + l16;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        Hreg[j][r] = sHf[i * DT + 16 * D + 4 * q4 + r];
                        sHt[(16 * D + 4 * q4 + r) * QP + i] = to_elem<T>(Hreg[j][r]);
                    }
                }
            }
            continue;
        }

        // ---- S^T = Kh Qh^T (masked) and O^T = V^T P^T + H_c^T Qh^T, one t-tile per wave
        for (int Tt = w; Tt < NTC; Tt += 4) {
            frag qf[NKM];
#pragma unroll
            for (int kb = 0; kb < NKM; ++kb) qf[kb] = MT::load_row(sQ + (16 * Tt + l16) * QP + kb * KB + EPL * q4);
            floatx4 st[NTCP];
#pragma unroll
            for (int J = 0; J < NTCP; ++J) {
                st[J] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (J <= Tt && J < NTC) {
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb) {
                        const frag a = MT::load_row(sK + (16 * J + l16) * QP + kb * KB + EPL * q4);
                        st[J] = MT::mma(a, qf[kb], st[J]);
                    }
                    if (J == Tt) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * q4 + r > l16) st[J][r] = 0.0f;  // j > t
                    }
                }
            }
            frag pf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) pf[kb] = MT::pack_perm(st, kb);
            const long tok = tokc + 16 * Tt + l16;
#pragma unroll
            for (int D = 0; D < NTD; ++D) {
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    if (kb * KB < 16 * (Tt + 1)) {
                        const frag a = MT::load_perm(sVt + (16 * D + l16) * TP, kb, q4);
                        acc = MT::mma(a, pf[kb], acc);
                    }
                }
#pragma unroll
                for (int kb = 0; kb < NKM; ++kb) {
                    const frag a = MT::load_row(sHt + (16 * D + l16) * QP + kb * KB + EPL * q4);
                    acc = MT::mma(a, qf[kb], acc);
                }
                if (tok < T_len)
                    *reinterpret_cast<float4*>(o + ((b * T_len + tok) * Hh + h) * Dv + d0 + 16 * D + 4 * q4) =
                        make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }

        // ---- U^T = V^T Kh on the state tiles this wave owns
        floatx4 U[UPW];
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int u = w + 4 * j;
            U[j] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (u < NU) {
                const int D = u / NTM, I = u % NTM;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    const frag a = MT::load_perm(sVt + (16 * D + l16) * TP, kb, q4);
                    const frag bb = MT::load_perm(sKt + (16 * I + l16) * TP, kb, q4);
                    U[j] = MT::mma(a, bb, U[j]);
                }
            }
        }
        __syncthreads();  // every read of H_c (sHt) is done
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int u = w + 4 * j;
            if (u < NU) {
                const int D = u / NTM, I = u % NTM, i = 16 * I + l16;
                const float e = sE[i];
                if (e < 1.0f) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Hreg[j][r] = e * (Hreg[j][r] + U[j][r]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sHt[(16 * D + 4 * q4 + r) * QP + i] = to_elem<T>(Hreg[j][r]);
                }
            }
        }
    }

    if (H_out) {
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int u = w + 4 * j;
            if (u < NU) {
                const int D = u / NTM, I = u % NTM, i = 16 * I + l16;
                *reinterpret_cast<float4*>(H_out + (bh * M + i) * Dv + d0 + 16 * D + 4 * q4) =
                    make_float4(Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
            }
        }
    }
}

// H_out = H0 (or zeros) for empty sequences.
__global__ void copy_state_kernel(const float* __restrict__ H0, float* __restrict__ H_out, long n) {
    const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) H_out[i] = H0 ? H0[i] : 0.0f;
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

FwdLayout forward_layout(int dtype, long B, long T, long Hh, int M, int Dv, int C) {
    (void)Dv;
    FwdLayout L{};
    const size_t es = dtype == RSM_F32 ? 4 : 2;
    L.n_chunks = (T + C - 1) / C;
    const size_t nbhc = size_t(B) * size_t(Hh) * size_t(L.n_chunks);
    L.tiles_off = 0;
    L.elast_off = align256(nbhc * 2 * size_t(C) * size_t(M) * es);
    L.flags_off = L.elast_off + align256(nbhc * size_t(M) * 4);
    L.total = L.flags_off + align256(nbhc * 4);
    if (nbhc == 0) L.total = 0;
    return L;
}

template <typename T, int M, int C, int DT>
static int launch_forward(const T* q, const T* k, const T* z, const T* v, const float* f, const float* H0,
                          long B, long T_len, long Hh, int Dv, int K, float* o, float* H_out,
                          int32_t* idx_out, unsigned char* ws, const FwdLayout& L, hipStream_t s) {
    using Cfg = ScanCfg<T, M, C, DT>;
    const long nC = L.n_chunks, BH = B * Hh;
    T* tiles = reinterpret_cast<T*>(ws + L.tiles_off);
    float* el = reinterpret_cast<float*>(ws + L.elast_off);
    int* fl = reinterpret_cast<int*>(ws + L.flags_off);
    hipLaunchKernelGGL((fwd_prep_kernel<T, M, C>), dim3(unsigned(BH * nC)), dim3(256), 0, s, q, k, z, f, T_len,
                       int(Hh), K, nC, tiles, el, fl, idx_out);
    if (hipGetLastError() != hipSuccess) return RSM_ERR_HIP;
    static bool attr_done = false;
    if (!attr_done) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_scan_kernel<T, M, C, DT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::total) != hipSuccess)
            return RSM_ERR_HIP;
        attr_done = true;
    }
    hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT>), dim3(unsigned(BH * (Dv / DT))), dim3(256), Cfg::total, s,
                       q, k, v, H0, T_len, int(Hh), Dv, nC, tiles, el, fl, o, H_out);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

template <typename T, int M, int C>
static int dispatch_dt(const T* q, const T* k, const T* z, const T* v, const float* f, const float* H0, long B,
                       long T_len, long Hh, int Dv, int K, float* o, float* H_out, int32_t* idx_out,
                       unsigned char* ws, const FwdLayout& L, hipStream_t s) {
    if (Dv % 32 == 0)
        return launch_forward<T, M, C, 32>(q, k, z, v, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
    return launch_forward<T, M, C, 16>(q, k, z, v, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
}

template <typename T, int M>
static int dispatch_c(int C, const T* q, const T* k, const T* z, const T* v, const float* f, const float* H0,
                      long B, long T_len, long Hh, int Dv, int K, float* o, float* H_out, int32_t* idx_out,
                      unsigned char* ws, const FwdLayout& L, hipStream_t s) {
    switch (C) {
        case 16: return dispatch_dt<T, M, 16>(q, k, z, v, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
        case 32: return dispatch_dt<T, M, 32>(q, k, z, v, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
        case 64: return dispatch_dt<T, M, 64>(q, k, z, v, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
    }
    return RSM_ERR_UNSUPPORTED;
}

template <typename T>
static int dispatch_m(int M, int C, const void* q, const void* k, const void* z, const void* v, const float* f,
                      const float* H0, long B, long T_len, long Hh, int Dv, int K, float* o, float* H_out,
                      int32_t* idx_out, unsigned char* ws, const FwdLayout& L, hipStream_t s) {
    const T *qq = static_cast<const T*>(q), *kk = static_cast<const T*>(k), *zz = static_cast<const T*>(z),
            *vv = static_cast<const T*>(v);
    switch (M) {
        case 16: return dispatch_c<T, 16>(C, qq, kk, zz, vv, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
        case 32: return dispatch_c<T, 32>(C, qq, kk, zz, vv, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
        case 64: return dispatch_c<T, 64>(C, qq, kk, zz, vv, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
        case 128: return dispatch_c<T, 128>(C, qq, kk, zz, vv, f, H0, B, T_len, Hh, Dv, K, o, H_out, idx_out, ws, L, s);
    }
    return RSM_ERR_UNSUPPORTED;
}

int forward_chunked_launch(const void* q, const void* k, const void* z, const void* v, int dtype,
                           const float* f, const float* H0, long B, long T, long Hh, int M, int Dv, int K,
                           int C, float* o, float* H_out, int32_t* idx_out, void* workspace,
                           hipStream_t stream) {
    const long BH = B * Hh;
    if (BH == 0) return RSM_OK;
    if (T == 0) {
        if (!H_out || H_out == H0) return RSM_OK;
        const long n = BH * M * Dv;
        hipLaunchKernelGGL(copy_state_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, H0, H_out, n);
        return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
    }
    const FwdLayout L = forward_layout(dtype, B, T, Hh, M, Dv, C);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if (dtype == RSM_F32)
        return dispatch_m<float>(M, C, q, k, z, v, f, H0, B, T, Hh, Dv, K, o, H_out, idx_out, ws, L, stream);
    return dispatch_m<bf16_t>(M, C, q, k, z, v, f, H0, B, T, Hh, Dv, K, o, H_out, idx_out, ws, L, stream);
}

}  // namespace rsm
