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
//    a compact list (slot, alpha) per token, or as dense alphas when K is a large fraction
//    of M -- the only intermediate in memory.
//  * fwd_scan (one workgroup per (batch, head, Dv tile)): walks the chunks in order with the
//    fp32 state tile in registers.  The chunk's raw q, k, v tiles and its route arrive in
//    LDS by direct global->LDS loads issued while the previous chunk computes.  Per chunk it
//    scatters the alphas into a dense tile in LDS, forms the decay products E by prefix
//    products along the chunk, builds Qh and Kh in LDS, runs the three contractions on
//    16x16 MFMA tiles, writes o, and updates the state.  Rows of slots untouched in a chunk
//    (E_last == 1) are not written, so they keep their exact bits.
//
// Overflow guard: 1/E grows with the decay accumulated in a chunk.  On the factored path each
// alpha is clamped below at e^-30 (~1e-13 instead of 0); a chunk whose decay product falls
// below 2^-100 for some slot is evaluated token by token with the exact alphas instead.
#include <type_traits>

#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

constexpr float kAlphaMin = 9.3576230e-14f;  // e^-30: clamp of alpha on the factored path
constexpr float kSafeMin = 7.8886091e-31f;   // 2^-100: smallest E_last kept factored

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

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
//
// Contractions over chunk rows j use the k-slot order j = jperm(kb, q4, e), the row order in
// which the S^T accumulator tiles hold P^T (rows 16*J + 4*q4 + r).  Contractions over slots
// use the natural order i = KB*kb + EPL*q4 + e.  A "column" fragment (k along the rows of a
// row-major LDS array) is gathered with ds_read_b64_tr_b16 for bf16: within each 16-lane
// group, lane 4a+b receives element b of the 8-byte blocks addressed by lanes a, a+4, a+8,
// a+12; so lane (a + 4e) addresses row rho(e), columns 4a..4a+3.
// ------------------------------------------------------------------------------------
//
// Every LDS access is written as one offset from its array (arr + off): the compiler then
// keeps track of which array each access touches and does not make it wait for the direct
// global->LDS loads still in flight into other arrays.
template <typename T> struct Pol;

template <> struct Pol<float> {
    static constexpr int KB = 4, EPL = 1, NPL = 1;
    typedef float E;
    typedef float frag;
    struct dfrag {
        frag p[1];
    };
    __device__ static __forceinline__ int jperm(int kb, int q4, int e) { return 16 * (kb >> 2) + 4 * q4 + (kb & 3); }
    __device__ static __forceinline__ int inat(int kb, int q4, int e) { return 4 * kb + q4; }
    __device__ static __forceinline__ frag ld(const E* arr, int off) { return arr[off]; }
    // column fragment: rows rho(kb, q4, e) of a row-major array with `pitch`, columns from
    // element offset off0 (plane + first column)
    template <bool PERM>
    __device__ static __forceinline__ frag ld_col(const E* arr, int off0, int pitch, int kb, int q4, int l16) {
        const int row = PERM ? jperm(kb, q4, 0) : inat(kb, q4, 0);
        return arr[off0 + row * pitch + l16];
    }
    __device__ static __forceinline__ void put(E* arr, int ps, int i, float x) { arr[i] = x; }
    // 4 consecutive values (16-byte aligned)
    __device__ static __forceinline__ void put4(E* arr, int ps, int i, float a, float b, float c, float d) {
        *reinterpret_cast<float4*>(arr + i) = make_float4(a, b, c, d);
    }
    // EVT = 4 consecutive values (16-byte aligned)
    __device__ static __forceinline__ void put_vec(E* arr, int ps, int i, const float* x) {
        *reinterpret_cast<float4*>(arr + i) = make_float4(x[0], x[1], x[2], x[3]);
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
    __device__ static __forceinline__ int jperm(int kb, int q4, int e) {
        return 32 * kb + 16 * (e >> 2) + 4 * q4 + (e & 3);
    }
    __device__ static __forceinline__ int inat(int kb, int q4, int e) { return 32 * kb + 8 * q4 + e; }
    __device__ static __forceinline__ frag ld(const E* arr, int off) {
        return __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(arr + off));
    }
    template <bool PERM>
    __device__ static __forceinline__ frag ld_col(const E* arr, int off0, int pitch, int kb, int q4, int l16) {
        const int er = l16 >> 2, c4 = 4 * (l16 & 3);
        const int r0 = PERM ? jperm(kb, q4, er) : inat(kb, q4, er);
        const int r1 = PERM ? jperm(kb, q4, 4 + er) : inat(kb, q4, 4 + er);
        const shortx4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(arr + (off0 + r0 * pitch + c4)));
        const shortx4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(arr + (off0 + r1 * pitch + c4)));
        const uint2 xa = __builtin_bit_cast(uint2, x), ya = __builtin_bit_cast(uint2, y);
        return __builtin_bit_cast(frag, make_uint4(xa.x, xa.y, ya.x, ya.y));
    }
    __device__ static __forceinline__ uint32_t split2(float a, float b, uint32_t& lo) {
        const floatx2 x = {a, b};
        const bf16x2 hi = __builtin_convertvector(x, bf16x2);
        const floatx2 r = x - __builtin_convertvector(hi, floatx2);
        lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2));
        return __builtin_bit_cast(uint32_t, hi);
    }
    __device__ static __forceinline__ void put(E* arr, int ps, int i, float x) {
        uint32_t lo;
        const uint32_t hi = split2(x, 0.0f, lo);
        arr[i].bits = uint16_t(hi);
        arr[ps + i].bits = uint16_t(lo);
    }
    __device__ static __forceinline__ void put4(E* arr, int ps, int i, float a, float b, float c, float d) {
        uint32_t l0, l1;
        const uint32_t h0 = split2(a, b, l0), h1 = split2(c, d, l1);
        *reinterpret_cast<uint2*>(arr + i) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(arr + (ps + i)) = make_uint2(l0, l1);
    }
    __device__ static __forceinline__ void put_vec(E* arr, int ps, int i, const float* x) {
        uint32_t l0, l1, l2, l3;
        const uint32_t h0 = split2(x[0], x[1], l0), h1 = split2(x[2], x[3], l1);
        const uint32_t h2 = split2(x[4], x[5], l2), h3 = split2(x[6], x[7], l3);
        *reinterpret_cast<uint4*>(arr + i) = make_uint4(h0, h1, h2, h3);
        *reinterpret_cast<uint4*>(arr + (ps + i)) = make_uint4(l0, l1, l2, l3);
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

// f(i) for i = tid, tid + NT, ... below N, with a trip count known at compile time.
template <int N, int NT, typename F>
__device__ __forceinline__ void for_each_tid(int tid, F f) {
#pragma unroll
    for (int it = 0; it < (N + NT - 1) / NT; ++it) {
        const int i = tid + NT * it;
        if (N % NT == 0 || i < N) f(i);
    }
}

// Direct global->LDS copy of a chunk tile: wave-instruction r moves LDS bytes
// [r*1024, r*1024 + 1024) of `lds`, lane l the 16 bytes at r*1024 + 16*l, taken from the
// global address src(byte offset).  `nbytes` is a multiple of 1024 (the LDS array is padded).
template <int NW, typename F>
__device__ __forceinline__ void dma_tile(void* lds, int nbytes, int w, int lane, F src) {
    for (int r = w; r * 1024 < nbytes; r += NW) {
        const void* g = src(r * 1024 + 16 * lane);
        __builtin_amdgcn_global_load_lds(g, (lds_void*)(static_cast<unsigned char*>(lds) + r * 1024), 16, 0, 0);
    }
}

constexpr int pad1k(int bytes) { return (bytes + 1023) / 1024 * 1024; }

// Workgroup barrier without a memory fence.  A workgroup-scope release fence would also
// wait for every direct global->LDS load still in flight; the scan waits for those
// explicitly, one chunk later.  LDS is coherent inside the workgroup, so each wave's own
// LDS accesses having completed (lgkmcnt = 0) before s_barrier is what makes them visible.
// The signal fences keep the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void wg_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Compact route capacity: K up to KC uses (slot, alpha) lists, larger K dense alphas.
constexpr int compact_cap(int M) { return M / 2 < 32 ? M / 2 : 32; }

// ------------------------------------------------------------------------------------
// Sequence segments.  A head's chunks are cut into S consecutive segments so that a launch
// has enough workgroups.  Segment s starts from the state the segments before it leave:
//     H_start(s+1) = diag(E_s) H_start(s) + dH_s,
// with E_s the product of the decay factors over segment s and dH_s the state segment s
// reaches from a zero state (the recurrence is linear in the state).  Pass A computes
// (E_s, dH_s) for every segment but the last and emits nothing else; pass B folds them into
// its start state and runs its segment with outputs.  With S = 1 there is only pass B.
// ------------------------------------------------------------------------------------
struct SegArgs {
    long nC;    // chunks in the sequence
    int S;      // segments
    int cps;    // chunks per segment
    float* dH;  // [B*Hh][S-1][M][Dv]
    float* dE;  // [B*Hh][S-1][M]
};

// ------------------------------------------------------------------------------------
// Chunk scan: one workgroup (8 waves) per (b, h, Dv tile of DT columns, segment); it walks
// the segment's chunks in order with the fp32 state tile in registers.
// DENSE: the route arrives as dense alphas [C][M] instead of (slot, alpha) lists.
// pass_a: pass A of the segment split (no Qh, no outputs; writes dH, dE).
//
// Wave roles (w = 0..7, all uniform):
//  * chunk-row tile Tt of S^T and O^T: waves w and w + NTC*g share Tt; odd groups take the
//    tiles in reverse so that the two waves of a SIMD (w, w+4) get a cheap and a costly tile;
//  * slot tile I = w % NTM of U^T and of the state, column tiles gI, gI + GI, ...
// ------------------------------------------------------------------------------------
template <typename T, int M, int C, int DT, bool DENSE>
__global__ __launch_bounds__(512) void fwd_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ H0,
    long T_len, int Hh, int Dv, int K, SegArgs sg, int pass_a, const uint8_t* __restrict__ ridx,
    const float* __restrict__ ralpha, float* __restrict__ o, float* __restrict__ H_out) {
    typedef Pol<T> P;
    typedef typename P::E E;
    typedef typename P::frag frag;
    typedef typename P::dfrag dfrag;
    constexpr int NW = 8, NT = 64 * NW;
    constexpr int KB = P::KB, EPL = P::EPL, NPL = P::NPL;
    constexpr int MP = M > KB ? M : KB;        // padded slot dimension (k of slot contractions)
    constexpr int CP = C > KB ? C : KB;        // padded chunk dimension (k of row contractions)
    constexpr int EVE = 16 / int(sizeof(E));   // elements per 16 bytes
    constexpr int QP = MP + EVE;               // pitch of Qh / Kh rows
    constexpr int HP = DT + EVE;               // pitch of state rows
    constexpr int NTC = C / 16, NTCP = CP / 16, NTD = DT / 16, NTM = M / 16;
    constexpr int NKM = MP / KB, NKC = CP / KB;
    constexpr int GT = NW / NTC;               // waves per chunk-row tile
    constexpr int NOD = (NTD + GT - 1) / GT;   // output column tiles per wave
    constexpr int GI = NW / NTM;               // waves per slot tile
    constexpr int UPW = (NTD + GI - 1) / GI;   // state tiles per wave
    constexpr int NPART = NT / M < C ? NT / M : C;  // token parts of the decay products
    constexpr int TPP = C / NPART;
    constexpr int KC = compact_cap(M);
    constexpr int RPT = NT / C;                // threads per token for the compact route
    constexpr int psQ = CP * QP + 8;           // plane stride of Qh / Kh
    constexpr int oK = NPL * psQ;              // Kh planes start here
    constexpr int psH = MP * HP;               // plane stride of the state copy
    constexpr int SZQK = 2 * NPL * psQ;
    constexpr int SZHF = M * DT * 4 / int(sizeof(E));
    static_assert(NW % NTC == 0 && NW % NTM == 0 && NT % C == 0, "tile split");

    // LDS.  Raw inputs land by direct loads (tile arrays padded to 1 KB); every array is a
    // separate object so the compiler can tell the direct loads from the other accesses.
    __shared__ __align__(16) T rq[pad1k(C * M * int(sizeof(T))) / int(sizeof(T))];
    __shared__ __align__(16) T rk[pad1k(C * M * int(sizeof(T))) / int(sizeof(T))];
    __shared__ __align__(16) T rv0[pad1k(CP * DT * int(sizeof(T))) / int(sizeof(T))];  // v, even chunks
    __shared__ __align__(16) T rv1[pad1k(CP * DT * int(sizeof(T))) / int(sizeof(T))];  // v, odd chunks
    __shared__ __align__(16) float rA[DENSE ? 4 : pad1k(C * KC * 4) / 4];
    __shared__ __align__(16) uint8_t rI[DENSE ? 16 : pad1k(C * KC)];
    __shared__ __align__(16) float sA[pad1k(C * M * 4) / 4];        // exact alphas of the chunk
    __shared__ __align__(16) E sQK[SZQK > SZHF ? SZQK : SZHF];      // Qh planes, then Kh planes
    __shared__ __align__(16) E sH[NPL * psH];                       // state copy, row-major [i][d]
    __shared__ float sTot[NPART * M];
    __shared__ float sE[M];
    __shared__ int sFlag[NW];
    float* sHf = reinterpret_cast<float*>(sQK);  // exact path: fp32 state [M][DT]

    // workgroup -> (head, segment, Dv tile); consecutive ids (the Dv tiles of one head and
    // segment) land on the same XCD (workgroups are dealt to the 8 XCDs round-robin)
    const int nDT = Dv / DT;
    const int nseg = pass_a ? sg.S - 1 : sg.S;
    const long nblk = gridDim.x;
    long id = blockIdx.x;
    if (nblk % 8 == 0) id = (long(blockIdx.x) % 8) * (nblk / 8) + long(blockIdx.x) / 8;
    const int dtile = int(id % nDT);
    const long rest = id / nDT;
    const int seg = int(rest % nseg);
    const long bh = rest / nseg;
    const int d0 = dtile * DT;
    const long h = bh % Hh, b = bh / Hh;
    const long T_pad = sg.nC * C;
    const long c_begin = long(seg) * sg.cps;
    const long c_end = c_begin + sg.cps < sg.nC ? c_begin + sg.cps : sg.nC;
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    // wave index in a scalar register: every branch on it is a uniform scalar branch (no
    // EXEC masking around the MFMAs, which would not be skipped lane by lane)
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gT = w / NTC;
    const int Tt = (gT & 1) ? NTC - 1 - w % NTC : w % NTC;
    const int I = w % NTM, gI = w / NTM;
    const int rt = tid / RPT, rsub = tid % RPT;     // compact route entries: token, first entry
    const int pslot = tid % M, ppart = tid / M;     // decay products: slot, token part
    const long rstride = long(Hh);                  // rows between consecutive tokens of one head
    const long segrow = (bh * (sg.S - 1) + seg) * M;  // row of this segment in dH / dE

    // ---- direct loads of chunk c's inputs (rows past the sequence end repeat the last row;
    // their tokens carry no route entries, so they contribute nothing)
    auto issue_qk = [&](long c) {
        const int nv = int(T_len - c * C < C ? T_len - c * C : C);
        constexpr int RB = M * int(sizeof(T));
        const char* kb_ = reinterpret_cast<const char*>(k + ((b * T_len + c * C) * rstride + h) * M);
        dma_tile<NW>(rk, int(sizeof(rk)), w, lane, [&](int off) {
            const int t = min(off / RB, nv - 1), cb = off % RB;
            return static_cast<const void*>(kb_ + long(t) * rstride * RB + cb);
        });
        if (!pass_a) {
            const char* qb = reinterpret_cast<const char*>(q + ((b * T_len + c * C) * rstride + h) * M);
            dma_tile<NW>(rq, int(sizeof(rq)), w, lane, [&](int off) {
                const int t = min(off / RB, nv - 1), cb = off % RB;
                return static_cast<const void*>(qb + long(t) * rstride * RB + cb);
            });
        }
    };
    auto issue_v = [&](long c, T* dst) {
        const int nv = int(T_len - c * C < C ? T_len - c * C : C);
        const char* vb = reinterpret_cast<const char*>(v + ((b * T_len + c * C) * rstride + h) * Dv + d0);
        constexpr int RB = DT * int(sizeof(T));
        const long gpitch = rstride * Dv * long(sizeof(T));
        dma_tile<NW>(dst, int(sizeof(rv0)), w, lane, [&](int off) {
            const int t = min(off / RB, nv - 1), cb = off % RB;
            return static_cast<const void*>(vb + t * gpitch + cb);
        });
    };
    auto issue_route = [&](long c) {
        if (DENSE) {
            const char* ab = reinterpret_cast<const char*>(ralpha + (bh * T_pad + c * C) * M);
            dma_tile<NW>(sA, int(sizeof(sA)), w, lane,
                         [&](int off) { return static_cast<const void*>(ab + min(off, C * M * 4 - 16)); });
        } else {
            const char* ab = reinterpret_cast<const char*>(ralpha + (bh * T_pad + c * C) * K);
            const char* ib = reinterpret_cast<const char*>(ridx + (bh * T_pad + c * C) * K);
            const int na = C * K * 4, ni = C * K;
            dma_tile<NW>(rA, pad1k(na), w, lane,
                         [&](int off) { return static_cast<const void*>(ab + min(off, na - 16)); });
            dma_tile<NW>(rI, pad1k(ni), w, lane,
                         [&](int off) { return static_cast<const void*>(ib + min(off, ni - 16)); });
        }
    };

    // ---- start state in registers: tile j holds H[16*I + l16][16*D + 4*q4 + r], D = gI + GI*j.
    // Pass B starts from H0 (or zero) and folds in the segments before its own; pass A
    // starts from zero.  LDS padding (slot rows past M, chunk rows past C) stays zero.
    for (int i = tid; i < int(sizeof(sQK) / sizeof(E)); i += NT) sQK[i] = E{};
    for (int i = tid; i < int(sizeof(sH) / sizeof(E)); i += NT) sH[i] = E{};
    floatx4 Hreg[UPW];
    float Eseg = 1.0f;  // pass A: decay product over the segment of row 16*I + l16
#pragma unroll
    for (int j = 0; j < UPW; ++j) {
        const int D = gI + GI * j, i = 16 * I + l16, col = d0 + 16 * D + 4 * q4;
        Hreg[j] = floatx4{0.f, 0.f, 0.f, 0.f};
        if (!pass_a && D < NTD) {
            if (H0) {
                const float4 x = *reinterpret_cast<const float4*>(H0 + (bh * M + i) * Dv + col);
                Hreg[j] = floatx4{x.x, x.y, x.z, x.w};
            }
            for (int sj = 0; sj < seg; ++sj) {
                const long row = (bh * (sg.S - 1) + sj) * M + i;
                const float e = sg.dE[row];
                if (e != 1.0f) {  // rows untouched in segment sj keep their bits
                    const float4 x = *reinterpret_cast<const float4*>(sg.dH + row * Dv + col);
                    Hreg[j] = floatx4{fmaf(e, Hreg[j][0], x.x), fmaf(e, Hreg[j][1], x.y),
                                      fmaf(e, Hreg[j][2], x.z), fmaf(e, Hreg[j][3], x.w)};
                }
            }
        }
    }
    wg_barrier();  // the zero fill is done before the state copy is written
    if (!pass_a) {
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int D = gI + GI * j, i = 16 * I + l16;
            if (D < NTD) P::put4(sH, psH, i * HP + 16 * D + 4 * q4, Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
        }
    }
    if (c_begin < c_end) {
        issue_qk(c_begin);
        issue_v(c_begin, rv0);
        issue_route(c_begin);
    }
    if (!DENSE)
        for (int i = tid; i < C * M; i += NT) sA[i] = 1.0f;

    // One chunk.  CUR selects the v buffer statically (even chunks of the segment rv0, odd
    // rv1) so the compiler can tell the in-flight loads of the next chunk's v from this
    // chunk's reads.
    auto chunk = [&](auto cur, long c) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur)::value;
        const long tokc = c * C;
        const int nvalid = int(T_len - tokc < C ? T_len - tokc : C);
        const T* rvc = CUR ? rv1 : rv0;
        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of this chunk have landed
        wg_barrier();                   // ... and every other wave's
        if (c + 1 < c_end) issue_v(c + 1, CUR ? rv0 : rv1);

        // ---- compact route: scatter the exact alphas into the dense tile (1 elsewhere)
        if (!DENSE) {
            if (rt < nvalid) {
#pragma unroll
                for (int j = 0; j < (KC + RPT - 1) / RPT; ++j) {
                    const int n = rsub + RPT * j;
                    if (n < K) sA[rt * M + rI[rt * K + n]] = rA[rt * K + n];
                }
            }
            wg_barrier();
        }

        // ---- decay products: thread (slot pslot, part ppart) runs over its TPP tokens with
        // the clamped alphas; the parts' products are combined through LDS
        float Eloc[TPP], Aloc[TPP];
        if (ppart < NPART) {
            float run = 1.0f;
#pragma unroll
            for (int tt = 0; tt < TPP; ++tt) {
                const int t = ppart * TPP + tt;
                const float a = t < nvalid ? sA[t * M + pslot] : 1.0f;
                Aloc[tt] = a;
                run *= fmaxf(a, kAlphaMin);
                Eloc[tt] = run;
            }
            sTot[ppart * M + pslot] = run;
        }
        wg_barrier();

        // ---- E, and in the same pass Qh = q o E and Kh = k (1 - alpha) / E (0 where alpha = 1)
        int bad = 0;
        if (ppart < NPART) {
            float pre = 1.0f, last = 1.0f;
#pragma unroll
            for (int p = 0; p < NPART; ++p) {
                const float tp = sTot[p * M + pslot];
                pre = p < ppart ? pre * tp : pre;
                last *= tp;
            }
#pragma unroll
            for (int tt = 0; tt < TPP; ++tt) {
                const int t = ppart * TPP + tt;
                const float ev = pre * Eloc[tt];
                if (!pass_a) P::put(sQK, psQ, t * QP + pslot, Elem<T>::load(rq, t * M + pslot) * ev);
                const float a = fmaxf(Aloc[tt], kAlphaMin);
                const float kh =
                    a < 1.0f ? Elem<T>::load(rk, t * M + pslot) * (1.0f - a) * __builtin_amdgcn_rcpf(ev) : 0.0f;
                P::put(sQK, psQ, oK + t * QP + pslot, kh);
            }
            if (ppart == 0) sE[pslot] = last;
            bad = !(last >= kSafeMin);
        }
        {
            const bool wave_bad = __ballot(bad) != 0;
            if (lane == 0) sFlag[w] = wave_bad;
        }
        wg_barrier();
        int unsafe = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) unsafe |= sFlag[i];

        if (unsafe) {
            // ---- exact token-by-token recurrence with the exact alphas, on an fp32 copy
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int D = gI + GI * j, i = 16 * I + l16;
                if (D < NTD) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) sHf[i * DT + 16 * D + 4 * q4 + r] = Hreg[j][r];
                }
            }
            wg_barrier();
            for (int tt = 0; tt < nvalid; ++tt) {
                for (int e = tid; e < M * DT; e += NT) {
                    const int i = e / DT, dd = e % DT;
                    const float a = sA[tt * M + i];
                    if (a != 1.0f) {
                        const float wk = (1.0f - a) * Elem<T>::load(rk, tt * M + i);
                        sHf[e] = fmaf(a, sHf[e], wk * Elem<T>::load(rvc, tt * DT + dd));
                    }
                }
                wg_barrier();
                if (!pass_a && tid < DT) {
                    float acc = 0.0f;
                    for (int i = 0; i < M; ++i) acc = fmaf(Elem<T>::load(rq, tt * M + i), sHf[i * DT + tid], acc);
                    o[((b * T_len + tokc + tt) * rstride + h) * Dv + d0 + tid] = acc;
                }
                wg_barrier();
            }
            if (tid < M) {  // decay product of the chunk with the exact alphas
                float e = 1.0f;
                for (int tt = 0; tt < nvalid; ++tt) e *= sA[tt * M + tid];
                sE[tid] = e;
            }
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int D = gI + GI * j, i = 16 * I + l16;
                if (D < NTD) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Hreg[j][r] = sHf[i * DT + 16 * D + 4 * q4 + r];
                }
            }
            wg_barrier();  // every read of sHf (aliasing Qh/Kh) is done; sE is written
            if (MP > M || CP > C)
                for (int i = tid; i < int(sizeof(sQK) / sizeof(E)); i += NT) sQK[i] = E{};  // padding
            if (!pass_a) {
#pragma unroll
                for (int j = 0; j < UPW; ++j) {
                    const int D = gI + GI * j, i = 16 * I + l16;
                    if (D < NTD)
                        P::put4(sH, psH, i * HP + 16 * D + 4 * q4, Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
                }
            } else {
                Eseg *= sE[16 * I + l16];
            }
            if (!DENSE)
                for (int i = tid; i < C * M; i += NT) sA[i] = 1.0f;
            if (c + 1 < c_end) {
                issue_qk(c + 1);
                issue_route(c + 1);
            }
            return;
        }

        if (!DENSE)  // ready for the next chunk's scatter
            for_each_tid<C * M / 4, NT>(tid, [&](int i) {
                *reinterpret_cast<float4*>(sA + 4 * i) = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            });
        if (c + 1 < c_end) {
            issue_qk(c + 1);
            issue_route(c + 1);
        }

        // ---- S^T = Kh Qh^T (masked) and O^T = V^T P^T + H_c^T Qh^T for chunk-row tile Tt
        if (!pass_a) {
            float* obase = o + ((b * T_len + tokc) * rstride + h) * Dv + d0;
            dfrag qf[NKM];
#pragma unroll
            for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
                    qf[kb].p[pl] = P::ld(sQK, pl * psQ + (16 * Tt + l16) * QP + kb * KB + EPL * q4);
            floatx4 st[NTCP];
#pragma unroll
            for (int J = 0; J < NTCP; ++J) {
                st[J] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (J <= Tt && J < NTC) {
                    dfrag a[NKM];
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                        for (int pl = 0; pl < NPL; ++pl)
                            a[kb].p[pl] = P::ld(sQK, oK + pl * psQ + (16 * J + l16) * QP + kb * KB + EPL * q4);
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb) st[J] = P::mm_dd(a[kb], qf[kb], st[J]);
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
            for (int jd = 0; jd < NOD; ++jd) {
                const int D = gT + GT * jd;
                if (NTD % GT != 0 && D >= NTD) break;
                frag va[NKC];
                dfrag ha[NKM];
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)
                    va[kb] = P::template ld_col<true>(rvc, 16 * D, DT, kb, q4, l16);  // in bounds for every kb
#pragma unroll
                for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                    for (int pl = 0; pl < NPL; ++pl)
                        ha[kb].p[pl] = P::template ld_col<false>(sH, pl * psH + 16 * D, HP, kb, q4, l16);
                floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb)
                    if (kb * KB < 16 * (Tt + 1)) acc = P::mm_vd(va[kb], pf[kb], acc);
#pragma unroll
                for (int kb = 0; kb < NKM; ++kb) acc = P::mm_dd(ha[kb], qf[kb], acc);
                if (tl < nvalid)
                    *reinterpret_cast<float4*>(obase + tl * rstride * Dv + 16 * D + 4 * q4) =
                        make_float4(acc[0], acc[1], acc[2], acc[3]);
            }
        }

        // ---- U^T = V^T Kh on the state tiles of this wave (Kh fragments shared across D)
        floatx4 U[UPW];
        {
            dfrag kf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
                    kf[kb].p[pl] = P::template ld_col<true>(sQK, oK + pl * psQ + 16 * I, QP, kb, q4, l16);
#pragma unroll
            for (int j = 0; j < UPW; ++j) {
                const int D = gI + GI * j;
                U[j] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (D < NTD) {
                    frag va[NKC];
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb) va[kb] = P::template ld_col<true>(rvc, 16 * D, DT, kb, q4, l16);
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb) U[j] = P::mm_vd(va[kb], kf[kb], U[j]);
                }
            }
        }
        wg_barrier();  // every read of H_c (sH), Qh/Kh and this chunk's v is done
        const float e = sE[16 * I + l16];
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int D = gI + GI * j, i = 16 * I + l16;
            if (D < NTD && e < 1.0f) {
#pragma unroll
                for (int r = 0; r < 4; ++r) Hreg[j][r] = e * (Hreg[j][r] + U[j][r]);
                if (!pass_a)
                    P::put4(sH, psH, i * HP + 16 * D + 4 * q4, Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
            }
        }
        if (pass_a) Eseg *= e;
    };
    for (long c = c_begin; c < c_end; c += 2) {
        chunk(std::integral_constant<int, 0>{}, c);
        if (c + 1 < c_end) chunk(std::integral_constant<int, 1>{}, c + 1);
    }

    if (pass_a) {
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int D = gI + GI * j, i = 16 * I + l16;
            if (D < NTD)
                *reinterpret_cast<float4*>(sg.dH + (segrow + i) * Dv + d0 + 16 * D + 4 * q4) =
                    make_float4(Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
        }
        if (dtile == 0 && gI == 0 && q4 == 0) sg.dE[segrow + 16 * I + l16] = Eseg;
    } else if (H_out && seg == sg.S - 1) {
#pragma unroll
        for (int j = 0; j < UPW; ++j) {
            const int D = gI + GI * j, i = 16 * I + l16;
            if (D < NTD)
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

// Chunk length the kernels run: the requested C, except M = 128, whose C = 64 tiles do not
// fit in LDS and run as chunks of 32 (same result up to rounding).
static int scan_chunk(int M, int C) { return (M == 128 && C > 32) ? 32 : C; }

// Dv tile of a workgroup: the whole head up to 128 columns (bf16) / 64 (fp32), half that
// for M = 128, so the fp32 state tile is at most 32 KB.
static int pick_dt(int dtype, int M, int Dv) {
    int cap = dtype == RSM_F32 ? 64 : 128;
    if (M >= 128) cap /= 2;
    return Dv < cap ? Dv : cap;
}

// Enough workgroups to fill the chip: segments per head so that heads x Dv tiles x
// segments reaches 256, at least one chunk per segment.
static void pick_segments(long heads_x_tiles, long nC, int& S, int& cps) {
    long s = 1;
    while (heads_x_tiles * s < 256 && s * 2 <= nC) s *= 2;
    cps = int((nC + s - 1) / s);
    S = nC > 0 ? int((nC + cps - 1) / cps) : 1;
}

FwdLayout forward_layout(int dtype, long B, long T, long Hh, int M, int Dv, int C, int K) {
    C = scan_chunk(M, C);
    FwdLayout L{};
    L.chunk = C;
    L.dt = pick_dt(dtype, M, Dv);
    L.n_chunks = (T + C - 1) / C;
    L.dense = K > compact_cap(M) ? 1 : 0;
    pick_segments(B * Hh * (Dv / L.dt), L.n_chunks, L.S, L.cps);
    const size_t rows = size_t(B) * size_t(Hh) * size_t(L.n_chunks) * size_t(C);  // padded token-heads
    if (rows == 0) return L;
    size_t off = 0;
    if (L.dense) {
        L.ridx_off = 0;
        L.ralpha_off = 0;
        off = align256(rows * size_t(M) * 4);
    } else {
        L.ridx_off = 0;
        L.ralpha_off = align256(rows * size_t(K));
        off = L.ralpha_off + align256(rows * size_t(K) * 4);
    }
    const size_t segs = size_t(B) * size_t(Hh) * size_t(L.S - 1);
    L.dh_off = off;
    off += align256(segs * size_t(M) * size_t(Dv) * 4);
    L.de_off = off;
    off += align256(segs * size_t(M) * 4);
    L.total = off;
    return L;
}

template <typename T, int M, int C, int DT, bool DENSE>
static int launch_scan(const T* q, const T* k, const T* v, const float* H0, long B, long T_len, long Hh, int Dv,
                       int K, const SegArgs& sg, const uint8_t* ridx, const float* ralpha, float* o,
                       float* H_out, hipStream_t s) {
    const long tiles = B * Hh * (Dv / DT);
    if (sg.S > 1) {
        hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, DENSE>), dim3(unsigned(tiles * (sg.S - 1))), dim3(512), 0,
                           s, q, k, v, H0, T_len, int(Hh), Dv, K, sg, 1, ridx, ralpha, o, H_out);
        if (hipGetLastError() != hipSuccess) return RSM_ERR_HIP;
    }
    hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, DENSE>), dim3(unsigned(tiles * sg.S)), dim3(512), 0, s, q, k,
                       v, H0, T_len, int(Hh), Dv, K, sg, 0, ridx, ralpha, o, H_out);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

template <typename T, int M, int C>
static int dispatch_dt(int DT, bool dense, const T* q, const T* k, const T* v, const float* H0, long B, long T_len,
                       long Hh, int Dv, int K, const SegArgs& sg, const uint8_t* ridx, const float* ralpha, float* o,
                       float* H_out, hipStream_t s) {
#define RSM_SCAN(DTV)                                                                                           \
    return dense ? launch_scan<T, M, C, DTV, true>(q, k, v, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s) \
                 : launch_scan<T, M, C, DTV, false>(q, k, v, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s)
    constexpr int cap = (sizeof(T) == 4 ? 64 : 128) / (M >= 128 ? 2 : 1);
    switch (DT) {
        case 16: RSM_SCAN(16);
        case 32: RSM_SCAN(32);
        case 64:
            if constexpr (cap >= 64) { RSM_SCAN(64); }
            break;
        case 128:
            if constexpr (cap >= 128) { RSM_SCAN(128); }
            break;
    }
#undef RSM_SCAN
    return RSM_ERR_UNSUPPORTED;
}

template <typename T, int M>
static int dispatch_c(int C, int DT, bool dense, const T* q, const T* k, const T* v, const float* H0, long B,
                      long T_len, long Hh, int Dv, int K, const SegArgs& sg, const uint8_t* ridx, const float* ralpha,
                      float* o, float* H_out, hipStream_t s) {
    switch (C) {
        case 16:
            return dispatch_dt<T, M, 16>(DT, dense, q, k, v, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s);
        case 32:
            return dispatch_dt<T, M, 32>(DT, dense, q, k, v, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s);
        case 64:
            if constexpr (M < 128)
                return dispatch_dt<T, M, 64>(DT, dense, q, k, v, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out,
                                             s);
            break;
    }
    return RSM_ERR_UNSUPPORTED;
}

template <typename T>
static int dispatch_m(int M, int C, int DT, bool dense, const void* q, const void* k, const void* v, const float* H0,
                      long B, long T_len, long Hh, int Dv, int K, const SegArgs& sg, const uint8_t* ridx,
                      const float* ralpha, float* o, float* H_out, hipStream_t s) {
    const T *qq = static_cast<const T*>(q), *kk = static_cast<const T*>(k), *vv = static_cast<const T*>(v);
    switch (M) {
        case 16:
            return dispatch_c<T, 16>(C, DT, dense, qq, kk, vv, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s);
        case 32:
            return dispatch_c<T, 32>(C, DT, dense, qq, kk, vv, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s);
        case 64:
            return dispatch_c<T, 64>(C, DT, dense, qq, kk, vv, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out, s);
        case 128:
            return dispatch_c<T, 128>(C, DT, dense, qq, kk, vv, H0, B, T_len, Hh, Dv, K, sg, ridx, ralpha, o, H_out,
                                      s);
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
    const SegArgs sg{L.n_chunks, L.S, L.cps, reinterpret_cast<float*>(ws + L.dh_off),
                     reinterpret_cast<float*>(ws + L.de_off)};
    int st = route_fwd_launch(z, dtype, f, B, T, Hh, L.n_chunks * L.chunk, M, K, L.dense, idx_out, ridx, ralpha,
                              stream);
    if (st != RSM_OK) return st;
    if (dtype == RSM_F32)
        return dispatch_m<float>(M, L.chunk, L.dt, L.dense, q, k, v, H0, B, T, Hh, Dv, K, sg, ridx, ralpha, o, H_out,
                                 stream);
    return dispatch_m<bf16_t>(M, L.chunk, L.dt, L.dense, q, k, v, H0, B, T, Hh, Dv, K, sg, ridx, ralpha, o, H_out,
                              stream);
}

}  // namespace rsm
