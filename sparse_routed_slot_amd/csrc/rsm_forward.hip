// rsm_forward.hip -- chunked forward of the RSM mixer: sparse decay, intra-chunk and
// chunk-state contractions on MFMA, inter-chunk state scan.
//
// The method (Raven README page, "How Raven Works"): per token the top-K slots by sigmoid
// score are decayed by alpha = exp(s*f) and written with (1-alpha)*k_i*v, and o = q . H is
// read after the update.  The Raven paper summary (appendix A.5) evaluates it chunkwise,
// T = n*C.  Unrolling the recurrence over a chunk that starts from state H_c, with the
// per-slot decay product E_t = prod_{tau <= t} alpha_tau taken from the chunk start
// (alpha = 1 on unselected slots) and k~ = (1-alpha)*k:
//
//     o_t     = sum_i q_ti E_ti H_c[i,:] + sum_{j<=t} ( sum_i q_ti (E_ti / E_ji) k~_ji ) v_j
//     H_{c+1} = diag(E_last) ( H_c + sum_j diag(1 / E_j) k~_j v_j^T )
//
// With Qh = q o E and Kh = k~ / E the double sum becomes dense products:
//     O^T = V^T P^T + H_c^T Qh^T   with P = tril(Qh Kh^T),      U^T = V^T Kh,
//     H_{c+1} = diag(E_last) (H_c + U).
//
// Kernels:
//  * route (rsm_route.hip, fully parallel): exact top-K per token-head and alpha, written as
//    a compact list (slot, alpha) per token -- the only intermediate in memory.
//  * fwd_scan (one workgroup per (batch, head, Dv tile)): walks the chunks in order with the
//    fp32 state tile in registers.  Per chunk it scatters the alphas into a dense tile in
//    LDS, forms the decay products E by prefix products along the chunk, builds Qh and Kh
//    in LDS, runs the three contractions on 16x16 MFMA tiles, writes o, and updates the
//    state.  Rows of slots untouched in a chunk (E_last == 1) are not written, so they keep
//    their exact bits.  The next chunk's inputs are loaded into registers while the current
//    chunk computes.
//
// Overflow guard: 1/E grows with the decay accumulated in a chunk.  On the factored path each
// alpha is clamped below at e^-30 (~1e-13 instead of 0); a chunk whose decay product falls
// below 2^-100 for some slot is evaluated token by token with the exact alphas instead.
#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

constexpr float kAlphaMin = 9.3576230e-14f;  // e^-30: clamp of alpha on the factored path
constexpr float kSafeMin = 7.8886091e-31f;   // 2^-100: smallest E_last kept factored

// ------------------------------------------------------------------------------------
// Operand policy.  16x16 MFMA output tiles; a k-block of KB along the contraction with
// EPL = KB/4 consecutive k per lane (lane l holds row/col l%16 and k = EPL*(l/16) + e).
//
// fp32 inputs: fp32 MFMA (16x16x4), every operand a plain float.
// bf16 inputs: bf16 MFMA (16x16x32).  q, k, v are exact bf16, but the derived operands
// Qh, Kh, P and the state copy are fp32 values: each is carried as a pair hi + lo of bf16
// (hi = bf16(x), lo = bf16(x - hi)), ~16 significant bits.  A product of two derived
// operands takes three MFMAs (hi*hi + hi*lo + lo*hi); V times a derived operand takes two.
// A single bf16 rounding of a derived operand costs up to 2^-9 of |o| wherever one term
// dominates an output -- the whole bf16 error budget.
// ------------------------------------------------------------------------------------
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Pol;

template <> struct Pol<float> {
    static constexpr int KB = 4, EPL = 1, NPL = 1;
    typedef float E;
    typedef float frag;
    struct dfrag {
        frag p[1];
    };
    __device__ static __forceinline__ frag ld(const E* p) { return *p; }
    // k-slot f = kb*EPL + e of a contraction over chunk rows j <-> j = 16(f/4) + 4*q4 + f%4
    __device__ static __forceinline__ int jperm(int kb, int q4, int e) { return 16 * (kb >> 2) + 4 * q4 + (kb & 3); }
    __device__ static __forceinline__ frag ld_perm(const E* row, int kb, int q4) { return row[jperm(kb, q4, 0)]; }
    __device__ static __forceinline__ frag ld_perm_strided(const E* col, int stride, int kb, int q4) {
        return col[jperm(kb, q4, 0) * stride];
    }
    __device__ static __forceinline__ void put(E* base, int ps, int i, float x) { base[i] = x; }
    __device__ static __forceinline__ void put_pair(E* base, int ps, int i0, int i1, float a, float b) {
        base[i0] = a;
        base[i1] = b;
    }
    // EVT = 4 consecutive values at base[i] (16-byte aligned)
    __device__ static __forceinline__ void put_vec(E* base, int ps, int i, const float* x) {
        *reinterpret_cast<float4*>(base + i) = make_float4(x[0], x[1], x[2], x[3]);
    }
    template <int NT>
    __device__ static __forceinline__ dfrag pack_perm(const floatx4 (&st)[NT], int kb) {
        return dfrag{{st[kb >> 2][kb & 3]}};
    }
    __device__ static __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ floatx4 mm_dd(const dfrag& a, const dfrag& b, floatx4 c) {
        return mma(a.p[0], b.p[0], c);
    }
    __device__ static __forceinline__ floatx4 mm_vd(frag v, const dfrag& b, floatx4 c) { return mma(v, b.p[0], c); }
};

template <> struct Pol<bf16_t> {
    static constexpr int KB = 32, EPL = 8, NPL = 2;
    typedef bf16_t E;
    typedef bf16x8 frag;
    struct dfrag {
        frag p[2];  // hi, lo
    };
    __device__ static __forceinline__ frag ld(const E* p) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(p));
    }
    __device__ static __forceinline__ int jperm(int kb, int q4, int e) {
        return 32 * kb + 16 * (e >> 2) + 4 * q4 + (e & 3);
    }
    // two runs of four consecutive j
    __device__ static __forceinline__ frag ld_perm(const E* row, int kb, int q4) {
        const uint2 a = *reinterpret_cast<const uint2*>(row + 32 * kb + 4 * q4);
        const uint2 b = *reinterpret_cast<const uint2*>(row + 32 * kb + 16 + 4 * q4);
        return __builtin_bit_cast(frag, make_uint4(a.x, a.y, b.x, b.y));
    }
    __device__ static __forceinline__ frag ld_perm_strided(const E* col, int stride, int kb, int q4) {
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t lo = col[jperm(kb, q4, 2 * p) * stride].bits;
            const uint32_t hi = col[jperm(kb, q4, 2 * p + 1) * stride].bits;
            w[p] = lo | (hi << 16);
        }
        return __builtin_bit_cast(frag, make_uint4(w[0], w[1], w[2], w[3]));
    }
    __device__ static __forceinline__ uint32_t split2(float a, float b, uint32_t& lo) {
        const floatx2 x = {a, b};
        const bf16x2 hi = __builtin_convertvector(x, bf16x2);
        const floatx2 r = x - __builtin_convertvector(hi, floatx2);
        lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
        return __builtin_bit_cast(uint32_t, hi);
    }
    __device__ static __forceinline__ void put(E* base, int ps, int i, float x) {
        uint32_t lo;
        const uint32_t hi = split2(x, 0.0f, lo);
        base[i].bits = uint16_t(hi);
        base[ps + i].bits = uint16_t(lo);
    }
    __device__ static __forceinline__ void put_pair(E* base, int ps, int i0, int i1, float a, float b) {
        uint32_t lo;
        const uint32_t hi = split2(a, b, lo);
        base[i0].bits = uint16_t(hi);
        base[i1].bits = uint16_t(hi >> 16);
        base[ps + i0].bits = uint16_t(lo);
        base[ps + i1].bits = uint16_t(lo >> 16);
    }
    // EVT = 8 consecutive values at base[i] (16-byte aligned): one 16-byte store per plane
    __device__ static __forceinline__ void put_vec(E* base, int ps, int i, const float* x) {
        uint32_t l0, l1, l2, l3;
        const uint32_t h0 = split2(x[0], x[1], l0), h1 = split2(x[2], x[3], l1);
        const uint32_t h2 = split2(x[4], x[5], l2), h3 = split2(x[6], x[7], l3);
        *reinterpret_cast<uint4*>(base + i) = make_uint4(h0, h1, h2, h3);
        *reinterpret_cast<uint4*>(base + ps + i) = make_uint4(l0, l1, l2, l3);
    }
    template <int NT>
    __device__ static __forceinline__ dfrag pack_perm(const floatx4 (&st)[NT], int kb) {
        const floatx4 x = st[2 * kb], y = st[2 * kb + 1];
        uint32_t l0, l1, l2, l3;
        const uint32_t h0 = split2(x[0], x[1], l0), h1 = split2(x[2], x[3], l1);
        const uint32_t h2 = split2(y[0], y[1], l2), h3 = split2(y[2], y[3], l3);
        dfrag r;
        r.p[0] = __builtin_bit_cast(frag, make_uint4(h0, h1, h2, h3));
        r.p[1] = __builtin_bit_cast(frag, make_uint4(l0, l1, l2, l3));
        return r;
    }
    __device__ static __forceinline__ floatx4 mma(frag a, frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ floatx4 mm_dd(const dfrag& a, const dfrag& b, floatx4 c) {
        c = mma(a.p[1], b.p[0], c);
        c = mma(a.p[0], b.p[1], c);
        return mma(a.p[0], b.p[0], c);
    }
    __device__ static __forceinline__ floatx4 mm_vd(frag v, const dfrag& b, floatx4 c) {
        c = mma(v, b.p[1], c);
        return mma(v, b.p[0], c);
    }
};

// 16 bytes of input elements -> fp32 values
__device__ __forceinline__ void unpack16(const uint4& x, float (&v)[8], bf16_t) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        v[2 * p] = __uint_as_float(w[p] << 16);
        v[2 * p + 1] = __uint_as_float(w[p] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void unpack16(const uint4& x, float (&v)[8], float) {
    v[0] = __uint_as_float(x.x);
    v[1] = __uint_as_float(x.y);
    v[2] = __uint_as_float(x.z);
    v[3] = __uint_as_float(x.w);
}

// LDS plan of the scan kernel (byte offsets).  Row pitches padded by one 16-byte vector.
template <typename T, int M, int C, int DT>
struct ScanCfg {
    typedef Pol<T> P;
    typedef typename P::E E;
    static constexpr int KB = P::KB, NPL = P::NPL;
    static constexpr int MP = M > KB ? M : KB;  // padded slot dimension
    static constexpr int CP = C > KB ? C : KB;  // padded chunk dimension
    static constexpr int EVE = 16 / int(sizeof(E));
    static constexpr int EVT = 16 / int(sizeof(T));
    static constexpr int QP = MP + EVE;      // pitch of sQ, sK, sHt rows
    static constexpr int TP = CP + EVT;      // pitch of sVt rows
    static constexpr int NPART = 256 / M;    // token parts of the prefix product
    static constexpr int TPP = C / NPART;    // tokens per part
    static constexpr int psQ = C * QP;       // plane sizes (elements)
    static constexpr int psHt = DT * QP;
    static constexpr int szQ = NPL * psQ * int(sizeof(E));
    static constexpr int szX = (M * DT * 4 + C * M + 15) / 16 * 16;     // exact-path scratch
    static constexpr int offQ = 0;
    static constexpr int offK = szQ;
    static constexpr int offA = 2 * szQ > szX ? 2 * szQ : szX;           // float [C][M]
    static constexpr int offKr = offA + C * M * 4;                        // T [C][M]
    static constexpr int offVt = offKr + C * M * int(sizeof(T));          // T [DT][TP]
    static constexpr int offHt = offVt + DT * TP * int(sizeof(T));        // E planes [DT][QP]
    static constexpr int offTot = offHt + NPL * psHt * int(sizeof(E));    // float [NPART][M]
    static constexpr int offE = offTot + NPART * M * 4;                   // float [M]
    static constexpr int total = (offE + M * 4 + 15) / 16 * 16;
    // exact-path scratch: state [M][DT] fp32 and slots [C][K] (uint8) inside sQ/sK; the exact
    // alphas [C][K] go to sA
    static constexpr int offHf = 0;
    static constexpr int offRa = M * DT * 4;
    static_assert(offRa + C * M <= offA, "exact-path scratch must fit below sA");
};

// floor(n / K) for 0 <= n < 2^20 from a float reciprocal, corrected to the exact quotient
__device__ __forceinline__ int div_small(int n, int K, float invK) {
    int qt = int(float(n) * invK);
    qt -= (qt * K > n) ? 1 : 0;
    qt += ((qt + 1) * K <= n) ? 1 : 0;
    return qt;
}

// ------------------------------------------------------------------------------------
// Scan: one workgroup (4 waves) per (b, h, Dv tile of DT columns); sequential over chunks.
// ------------------------------------------------------------------------------------
template <typename T, int M, int C, int DT>
__global__ __launch_bounds__(256) void fwd_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ H0,
    long T_len, int Hh, int Dv, int K, long nC, const uint8_t* __restrict__ ridx, const float* __restrict__ ralpha,
    float* __restrict__ o, float* __restrict__ H_out) {
    typedef ScanCfg<T, M, C, DT> Cfg;
    typedef typename Cfg::P P;
    typedef typename P::E E;
    typedef typename P::frag frag;
    typedef typename P::dfrag dfrag;
    constexpr int KB = P::KB, EPL = P::EPL, NPL = P::NPL;
    constexpr int MP = Cfg::MP, CP = Cfg::CP, QP = Cfg::QP, TP = Cfg::TP, EVT = Cfg::EVT;
    constexpr int psQ = Cfg::psQ, psHt = Cfg::psHt;
    constexpr int NTC = C / 16, NTCP = CP / 16, NTD = DT / 16, NTM = M / 16;
    constexpr int NIW = (NTM + 3) / 4;   // slot tiles owned per wave (I = w + 4*jI)
    constexpr int UPW = NIW * NTD;       // state tiles per wave: (I, D) for D = 0..NTD-1
    constexpr int NKM = MP / KB, NKC = CP / KB;
    constexpr int NPART = Cfg::NPART, TPP = Cfg::TPP;
    constexpr int NVQ = (C * M / EVT + 255) / 256;   // q / k tile vectors per thread
    constexpr int NVV = (C * DT / EVT + 255) / 256;  // v tile vectors per thread
    constexpr int MAXRA = (C * M / 4 + 255) / 256;   // route vectors (4 entries) per thread, K <= M

    extern __shared__ __align__(16) unsigned char smem[];
    E* sQ = reinterpret_cast<E*>(smem + Cfg::offQ);
    E* sK = reinterpret_cast<E*>(smem + Cfg::offK);
    float* sA = reinterpret_cast<float*>(smem + Cfg::offA);
    T* sKr = reinterpret_cast<T*>(smem + Cfg::offKr);
    T* sVt = reinterpret_cast<T*>(smem + Cfg::offVt);
    E* sHt = reinterpret_cast<E*>(smem + Cfg::offHt);
    float* sTot = reinterpret_cast<float*>(smem + Cfg::offTot);
    float* sE = reinterpret_cast<float*>(smem + Cfg::offE);
    float* sHf = reinterpret_cast<float*>(smem + Cfg::offHf);       // exact path: state [M][DT]
    uint8_t* sRi = reinterpret_cast<uint8_t*>(smem + Cfg::offRa);   // exact path: slots [C][K]
    float* sRa = sA;                                                // exact path: alphas [C][K]

    // workgroup -> (head, Dv tile); the Dv tiles of one head land on the same XCD
    // (workgroups are dealt to the 8 XCDs round-robin) so they share inputs in its L2.
    const int nDT = Dv / DT;
    const long nblk = gridDim.x;
    long id = blockIdx.x;
    if (nblk % 8 == 0) id = (long(blockIdx.x) % 8) * (nblk / 8) + long(blockIdx.x) / 8;
    const long bh = id / nDT;
    const int d0 = int(id % nDT) * DT;
    const long h = bh % Hh, b = bh / Hh;
    const long T_pad = nC * C;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    const int nra = (C * K / 4 + 255) / 256;  // route vectors per thread (uniform)
    const float invK = 1.0f / float(K);
    const long tstride = long(Hh);            // rows between consecutive tokens of a head

    for (int i = tid * 16; i < Cfg::total; i += 256 * 16)
        *reinterpret_cast<uint4*>(smem + i) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    for (int i = tid; i < C * M; i += 256) sA[i] = 1.0f;

    // state tile j = jI*NTD + D holds H[i = 16*I + l16][d = 16*D + 4*q4 + r], I = w + 4*jI
    floatx4 Hreg[UPW];
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
        const int I = w + 4 * (j / NTD), D = j % NTD, i = 16 * I + l16;
        Hreg[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (I < NTM) {
            if (H0) {
                const float4 x = *reinterpret_cast<const float4*>(H0 + (bh * M + i) * Dv + d0 + 16 * D + 4 * q4);
                Hreg[j] = floatx4{x.x, x.y, x.z, x.w};
            }
            const int r0 = (16 * D + 4 * q4) * QP + i;
            P::put_pair(sHt, psHt, r0, r0 + QP, Hreg[j][0], Hreg[j][1]);
            P::put_pair(sHt, psHt, r0 + 2 * QP, r0 + 3 * QP, Hreg[j][2], Hreg[j][3]);
        }
    }

    // ---- register prefetch of one chunk's inputs
    uint4 pq[NVQ], pk[NVQ], pv[NVV];
    float4 pa[MAXRA];
    uint32_t pi[MAXRA];
    auto load_qk = [&](long c, uint4 (&dst)[NVQ], const T* src) {
        const T* base = src + ((b * T_len + c * C) * tstride + h) * M;
        const int nv = int(T_len - c * C < C ? T_len - c * C : C);
#pragma unroll
        for (int r = 0; r < NVQ; ++r) {
            const int u = tid + 256 * r;
            const int t = (u * EVT) / M, i0 = (u * EVT) % M;
            dst[r] = make_uint4(0u, 0u, 0u, 0u);
            if (u < C * M / EVT && t < nv) dst[r] = *reinterpret_cast<const uint4*>(base + t * tstride * M + i0);
        }
    };
    auto load_v = [&](long c) {
        const T* base = v + ((b * T_len + c * C) * tstride + h) * Dv + d0;
        const int nv = int(T_len - c * C < C ? T_len - c * C : C);
#pragma unroll
        for (int r = 0; r < NVV; ++r) {
            const int u = tid + 256 * r;
            const int t = (u * EVT) / DT, c0 = (u * EVT) % DT;
            pv[r] = make_uint4(0u, 0u, 0u, 0u);
            if (u < C * DT / EVT && t < nv) pv[r] = *reinterpret_cast<const uint4*>(base + t * tstride * Dv + c0);
        }
    };
    auto load_route = [&](long c) {
        const long base = (bh * T_pad + c * C) * K;
#pragma unroll
        for (int r = 0; r < MAXRA; ++r) {
            const int u = tid + 256 * r;
            if (r < nra && u < C * K / 4) {
                pa[r] = *reinterpret_cast<const float4*>(ralpha + base + 4 * u);
                pi[r] = *reinterpret_cast<const uint32_t*>(ridx + base + 4 * u);
            } else {
                pa[r] = make_float4(1.f, 1.f, 1.f, 1.f);
                pi[r] = 0u;
            }
        }
    };
    if (nC > 0) {
        load_qk(0, pq, q);
        load_qk(0, pk, k);
        load_v(0);
        load_route(0);
    }

    for (long c = 0; c < nC; ++c) {
        const long tokc = c * C;
        const int nvalid = int(T_len - tokc < C ? T_len - tokc : C);
        __syncthreads();  // previous chunk: every read of sQ, sK, sVt, sKr is done

        // ---- stage raw k and V^T, scatter the clamped alphas, clear Kh
#pragma unroll
        for (int r = 0; r < NVQ; ++r) {
            const int u = tid + 256 * r;
            if (u < C * M / EVT) *reinterpret_cast<uint4*>(sKr + u * EVT) = pk[r];
        }
#pragma unroll
        for (int r = 0; r < NVV; ++r) {
            const int u = tid + 256 * r;
            if (u < C * DT / EVT) {
                const int t = (u * EVT) / DT, c0 = (u * EVT) % DT;
                const T* xe = reinterpret_cast<const T*>(&pv[r]);
#pragma unroll
                for (int e = 0; e < EVT; ++e) sVt[(c0 + e) * TP + t] = xe[e];
            }
        }
#pragma unroll
        for (int r = 0; r < MAXRA; ++r) {
            if (r < nra) {
                const int u = tid + 256 * r;
                const float av[4] = {pa[r].x, pa[r].y, pa[r].z, pa[r].w};
                int t = div_small(4 * u, K, invK), n = 4 * u - t * K;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (t < nvalid && u < C * K / 4) sA[t * M + ((pi[r] >> (8 * e)) & 0xFF)] = fmaxf(av[e], kAlphaMin);
                    if (++n == K) {
                        n = 0;
                        ++t;
                    }
                }
            }
        }
        for (int i = Cfg::offK + tid * 16; i < 2 * Cfg::szQ; i += 256 * 16)
            *reinterpret_cast<uint4*>(smem + i) = make_uint4(0u, 0u, 0u, 0u);
        if (c + 1 < nC) {
            load_qk(c + 1, pk, k);
            load_v(c + 1);
        }
        __syncthreads();

        // ---- decay products: thread (slot i, part p) runs over its TPP tokens
        const int pslot = tid % M, ppart = tid / M;
        float Eloc[TPP];
        {
            float run = 1.0f;
#pragma unroll
            for (int tt = 0; tt < TPP; ++tt) {
                run *= sA[(ppart * TPP + tt) * M + pslot];
                Eloc[tt] = run;
            }
            sTot[ppart * M + pslot] = run;
        }
        __syncthreads();
        int bad = 0;
        {
            float pre = 1.0f, last = 1.0f;
#pragma unroll
            for (int p = 0; p < NPART; ++p) {
                const float tp = sTot[p * M + pslot];
                if (p < ppart) pre *= tp;
                last *= tp;
            }
#pragma unroll
            for (int tt = 0; tt < TPP; ++tt) sA[(ppart * TPP + tt) * M + pslot] = pre * Eloc[tt];
            if (ppart == 0) sE[pslot] = last;
            bad = !(last >= kSafeMin);
        }
        const int unsafe = __syncthreads_or(bad);

        if (unsafe) {
            // ---- exact token-by-token recurrence with the exact alphas
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int I = w + 4 * (j / NTD), D = j % NTD, i = 16 * I + l16;
                if (I < NTM) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sHf[i * DT + 16 * D + 4 * q4 + r] = Hreg[j][r];
                }
            }
#pragma unroll
            for (int r = 0; r < MAXRA; ++r) {
                const int u = tid + 256 * r;
                if (r < nra && u < C * K / 4) {
                    const float av[4] = {pa[r].x, pa[r].y, pa[r].z, pa[r].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        sRa[4 * u + e] = av[e];
                        sRi[4 * u + e] = uint8_t((pi[r] >> (8 * e)) & 0xFF);
                    }
                }
            }
            __syncthreads();
            for (int tt = 0; tt < nvalid; ++tt) {
                const long row = (b * T_len + tokc + tt) * Hh + h;
                for (int e = tid; e < K * DT; e += 256) {
                    const int n = e / DT, dd = e % DT;
                    const float a = sRa[tt * K + n];
                    const int i = sRi[tt * K + n];
                    if (a != 1.0f) {
                        const float wk = (1.0f - a) * Elem<T>::load(sKr, tt * M + i);
                        const float vv = Elem<T>::load(sVt, dd * TP + tt);
                        sHf[i * DT + dd] = fmaf(a, sHf[i * DT + dd], wk * vv);
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
                const int I = w + 4 * (j / NTD), D = j % NTD, i = 16 * I + l16;
                if (I < NTM) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Hreg[j][r] = sHf[i * DT + 16 * D + 4 * q4 + r];
                    const int r0 = (16 * D + 4 * q4) * QP + i;
                    P::put_pair(sHt, psHt, r0, r0 + QP, Hreg[j][0], Hreg[j][1]);
                    P::put_pair(sHt, psHt, r0 + 2 * QP, r0 + 3 * QP, Hreg[j][2], Hreg[j][3]);
                }
            }
            __syncthreads();
            for (int i = tid; i < C * M; i += 256) sA[i] = 1.0f;
            if (c + 1 < nC) {
                load_qk(c + 1, pq, q);
                load_route(c + 1);
            }
            continue;
        }

        // ---- Qh = q o E (split planes) and Kh = k (1 - alpha) / E at the selected entries
#pragma unroll
        for (int r = 0; r < NVQ; ++r) {
            const int u = tid + 256 * r;
            if (u < C * M / EVT) {
                const int t = (u * EVT) / M, i0 = (u * EVT) % M;
                float qv[8];
                unpack16(pq[r], qv, T());
                const float* Ep = sA + t * M + i0;
#pragma unroll
                for (int e = 0; e < EVT; ++e) qv[e] *= Ep[e];
                P::put_vec(sQ, psQ, t * QP + i0, qv);
            }
        }
#pragma unroll
        for (int r = 0; r < MAXRA; ++r) {
            if (r < nra) {
                const int u = tid + 256 * r;
                const float av[4] = {pa[r].x, pa[r].y, pa[r].z, pa[r].w};
                int t = div_small(4 * u, K, invK), n = 4 * u - t * K;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int slot = (pi[r] >> (8 * e)) & 0xFF;
                    const float a = fmaxf(av[e], kAlphaMin);
                    if (t < nvalid && u < C * K / 4 && a < 1.0f) {
                        const float kh = Elem<T>::load(sKr, t * M + slot) * (1.0f - a) *
                                         __builtin_amdgcn_rcpf(sA[t * M + slot]);
                        P::put(sK, psQ, t * QP + slot, kh);
                    }
                    if (++n == K) {
                        n = 0;
                        ++t;
                    }
                }
            }
        }
        __syncthreads();
        for (int i = tid; i < C * M; i += 256) sA[i] = 1.0f;  // ready for the next chunk's scatter
        if (c + 1 < nC) {
            load_qk(c + 1, pq, q);
            load_route(c + 1);
        }

        // ---- S^T = Kh Qh^T (masked) and O^T = V^T P^T + H_c^T Qh^T, one t-tile per wave
        float* obase = o + ((b * T_len + tokc) * tstride + h) * Dv + d0;
        for (int Tt = w; Tt < NTC; Tt += 4) {
            dfrag qf[NKM];
#pragma unroll
            for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
                    qf[kb].p[pl] = P::ld(sQ + pl * psQ + (16 * Tt + l16) * QP + kb * KB + EPL * q4);
            floatx4 st[NTCP];
#pragma unroll
            for (int J = 0; J < NTCP; ++J) {
                st[J] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (J <= Tt && J < NTC) {
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb) {
                        dfrag a;
#pragma unroll
                        for (int pl = 0; pl < NPL; ++pl)
                            a.p[pl] = P::ld(sK + pl * psQ + (16 * J + l16) * QP + kb * KB + EPL * q4);
                        st[J] = P::mm_dd(a, qf[kb], st[J]);
                    }
                    if (J == Tt) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * q4 + r > l16) st[J][r] = 0.0f;  // j > t
                    }
                }
            }
            dfrag pf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) pf[kb] = P::pack_perm(st, kb);
            const int tl = 16 * Tt + l16;
#pragma unroll
            for (int D = 0; D < NTD; ++D) {
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    if (kb * KB < 16 * (Tt + 1)) {
                        const frag a = P::ld_perm(reinterpret_cast<const E*>(sVt) + (16 * D + l16) * TP, kb, q4);
                        acc = P::mm_vd(a, pf[kb], acc);
                    }
                }
#pragma unroll
                for (int kb = 0; kb < NKM; ++kb) {
                    dfrag a;
#pragma unroll
                    for (int pl = 0; pl < NPL; ++pl)
                        a.p[pl] = P::ld(sHt + pl * psHt + (16 * D + l16) * QP + kb * KB + EPL * q4);
                    acc = P::mm_dd(a, qf[kb], acc);
                }
                if (tl < nvalid)
                    *reinterpret_cast<float4*>(obase + tl * tstride * Dv + 16 * D + 4 * q4) =
                        make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }

        // ---- U^T = V^T Kh on the state tiles this wave owns (Kh fragments shared across D)
        floatx4 U[UPW];
#pragma unroll
        for (int jI = 0; jI < NIW; ++jI) {
            const int I = w + 4 * jI;
#pragma unroll
            for (int D = 0; D < NTD; ++D) U[jI * NTD + D] = floatx4{0.f, 0.f, 0.f, 0.f};
            if (I < NTM) {
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
                    dfrag bb;
#pragma unroll
                    for (int pl = 0; pl < NPL; ++pl)
                        bb.p[pl] = P::ld_perm_strided(sK + pl * psQ + 16 * I + l16, QP, kb, q4);
#pragma unroll
                    for (int D = 0; D < NTD; ++D) {
                        const frag a = P::ld_perm(reinterpret_cast<const E*>(sVt) + (16 * D + l16) * TP, kb, q4);
                        U[jI * NTD + D] = P::mm_vd(a, bb, U[jI * NTD + D]);
                    }
                }
            }
        }
        __syncthreads();  // every read of H_c (sHt) is done
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int I = w + 4 * (j / NTD), D = j % NTD, i = 16 * I + l16;
            if (I < NTM) {
                const float e = sE[i];
                if (e < 1.0f) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Hreg[j][r] = e * (Hreg[j][r] + U[j][r]);
                    const int r0 = (16 * D + 4 * q4) * QP + i;
                    P::put_pair(sHt, psHt, r0, r0 + QP, Hreg[j][0], Hreg[j][1]);
                    P::put_pair(sHt, psHt, r0 + 2 * QP, r0 + 3 * QP, Hreg[j][2], Hreg[j][3]);
                }
            }
        }
    }

    if (H_out) {
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int I = w + 4 * (j / NTD), D = j % NTD, i = 16 * I + l16;
            if (I < NTM)
                *reinterpret_cast<float4*>(H_out + (bh * M + i) * Dv + d0 + 16 * D + 4 * q4) =
                    make_float4(Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
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

FwdLayout forward_layout(int dtype, long B, long T, long Hh, int M, int Dv, int C, int K) {
    (void)dtype;
    (void)Dv;
    (void)M;
    FwdLayout L{};
    L.n_chunks = (T + C - 1) / C;
    const size_t rows = size_t(B) * size_t(Hh) * size_t(L.n_chunks) * size_t(C);  // padded token-heads
    L.ridx_off = 0;
    L.ralpha_off = align256(rows * size_t(K));
    L.total = L.ralpha_off + align256(rows * size_t(K) * 4);
    if (rows == 0) L.total = 0;
    return L;
}

// Dv tile of the scan: 32 columns, 16 for M = 128 (LDS budget) or when Dv is 16.
static int pick_dt(int M, int Dv) { return (M >= 128 || Dv % 32 != 0) ? 16 : 32; }

template <typename T, int M, int C, int DT>
static int launch_scan(const T* q, const T* k, const T* v, const float* H0, long B, long T_len, long Hh, int Dv,
                       int K, long nC, const uint8_t* ridx, const float* ralpha, float* o, float* H_out,
                       hipStream_t s) {
    typedef ScanCfg<T, M, C, DT> Cfg;
    static bool attr_done = false;
    if (!attr_done) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(&fwd_scan_kernel<T, M, C, DT>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::total) != hipSuccess)
            return RSM_ERR_HIP;
        attr_done = true;
    }
    hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT>), dim3(unsigned(B * Hh * (Dv / DT))), dim3(256), Cfg::total, s,
                       q, k, v, H0, T_len, int(Hh), Dv, K, nC, ridx, ralpha, o, H_out);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

template <typename T, int M, int C>
static int dispatch_dt(const T* q, const T* k, const T* v, const float* H0, long B, long T_len, long Hh, int Dv,
                       int K, long nC, const uint8_t* ridx, const float* ralpha, float* o, float* H_out,
                       hipStream_t s) {
    if (pick_dt(M, Dv) == 32)
        return launch_scan<T, M, C, 32>(q, k, v, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
    return launch_scan<T, M, C, 16>(q, k, v, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
}

template <typename T, int M>
static int dispatch_c(int C, const T* q, const T* k, const T* v, const float* H0, long B, long T_len, long Hh,
                      int Dv, int K, long nC, const uint8_t* ridx, const float* ralpha, float* o, float* H_out,
                      hipStream_t s) {
    switch (C) {
        case 16: return dispatch_dt<T, M, 16>(q, k, v, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
        case 32: return dispatch_dt<T, M, 32>(q, k, v, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
        case 64: return dispatch_dt<T, M, 64>(q, k, v, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
    }
    return RSM_ERR_UNSUPPORTED;
}

template <typename T>
static int dispatch_m(int M, int C, const void* q, const void* k, const void* v, const float* H0, long B,
                      long T_len, long Hh, int Dv, int K, long nC, const uint8_t* ridx, const float* ralpha, float* o,
                      float* H_out, hipStream_t s) {
    const T *qq = static_cast<const T*>(q), *kk = static_cast<const T*>(k), *vv = static_cast<const T*>(v);
    switch (M) {
        case 16: return dispatch_c<T, 16>(C, qq, kk, vv, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
        case 32: return dispatch_c<T, 32>(C, qq, kk, vv, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
        case 64: return dispatch_c<T, 64>(C, qq, kk, vv, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
        case 128: return dispatch_c<T, 128>(C, qq, kk, vv, H0, B, T_len, Hh, Dv, K, nC, ridx, ralpha, o, H_out, s);
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
    const FwdLayout L = forward_layout(dtype, B, T, Hh, M, Dv, C, K);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    uint8_t* ridx = ws + L.ridx_off;
    float* ralpha = reinterpret_cast<float*>(ws + L.ralpha_off);
    const long T_pad = L.n_chunks * C;
    int st = route_fwd_launch(z, dtype, f, B, T, Hh, T_pad, M, K, idx_out, ridx, ralpha, stream);
    if (st != RSM_OK) return st;
    if (dtype == RSM_F32)
        return dispatch_m<float>(M, C, q, k, v, H0, B, T, Hh, Dv, K, L.n_chunks, ridx, ralpha, o, H_out, stream);
    return dispatch_m<bf16_t>(M, C, q, k, v, H0, B, T, Hh, Dv, K, L.n_chunks, ridx, ralpha, o, H_out, stream);
}

}  // namespace rsm
