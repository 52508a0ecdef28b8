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
//    a selection bit mask plus the alphas of the selected slots -- the only intermediate in
//    memory.
//  * fwd_scan (one workgroup per (batch, head, Dv tile)): walks the chunks in order with the
//    fp32 state tile in registers.  The chunk's raw q, k, v tiles and its route arrive in
//    LDS by direct global->LDS loads issued while the previous chunk computes.  Per chunk
//    each lane takes one token and each wave a group of slots: the lane gathers its alphas
//    from the route, the decay products E come from a product scan across the wave's lanes,
//    and the lane writes its rows of Qh and Kh.  Then the three contractions run on 16x16
//    MFMA tiles, o is written, and the state is updated.  Rows of slots untouched in a chunk
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
// Swizzled tiles.  The raw q, k and v tiles arrive in LDS by direct loads that fill 16-byte
// granules in order, so their rows cannot be padded; instead granule g of row `row` (GPR
// granules per row) sits at granule position row*GPR + swz(row, g), an XOR of g with a
// function of the row, so that the rows a wave reads at once fall into different banks:
//  * KIND 1 (q, k: lane = row, one granule each): g ^ ((row / RPB) % GPR);
//  * KIND 2 (v: 8-byte column pieces of 4 rows and 2 adjacent granules per 16 lanes):
//    g ^ 2*((row / RPB) % (GPR/2)), which keeps granule pairs together;
//  * KIND 3 (the state copy: 8-byte column pieces of rows 8*q4 + 0..3 per 16 lanes):
//    g ^ ((2*(row % 4) + 8*((row / 8) % 2)) % GPR);
// with RPB = max(1, 16 / GPR) rows per 256-byte bank sweep.
//
// Every LDS access is written as one offset from its array (arr + off): the compiler then
// keeps track of which array each access touches and does not make it wait for the direct
// global->LDS loads still in flight into other arrays.
template <int GPR, int KIND>
__device__ __forceinline__ int swz(int row, int g) {
    if constexpr (GPR <= 1 || KIND == 0) {
        return g;
    } else {
        constexpr int RPB = GPR >= 16 ? 1 : 16 / GPR;
        if constexpr (KIND == 1) return g ^ ((row / RPB) % GPR);
        else if constexpr (KIND == 3) return g ^ ((2 * (row & 3) + 8 * ((row >> 3) & 1)) & (GPR - 1));
        else if constexpr (GPR >= 4) return g ^ (2 * ((row / RPB) % (GPR / 2)));
        else return g;
    }
}
// element index of (row, col) in a swizzled tile of EPG elements per granule
template <int GPR, int KIND, int EPG>
__device__ __forceinline__ int swz_elem(int row, int col) {
    return (row * GPR + swz<GPR, KIND>(row, col / EPG)) * EPG + col % EPG;
}

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
    template <bool PERM, int GPR, int KIND>
    __device__ static __forceinline__ frag ld_col_swz(const E* arr, int base, int col0, int kb, int q4, int l16) {
        const int row = PERM ? jperm(kb, q4, 0) : inat(kb, q4, 0);
        return arr[base + swz_elem<GPR, KIND, 4>(row, col0 + l16)];
    }
    __device__ static __forceinline__ void put(E* arr, int ps, int i, float x) { arr[i] = x; }
    // 4 consecutive values (16-byte aligned)
    __device__ static __forceinline__ void put4(E* arr, int ps, int i, float a, float b, float c, float d) {
        *reinterpret_cast<float4*>(arr + i) = make_float4(a, b, c, d);
    }
    // N consecutive values (N*4 bytes aligned to min(16, N*4))
    template <int N>
    __device__ static __forceinline__ void put_row(E* arr, int ps, int i, const float (&x)[N]) {
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int g = 0; g < N / 4; ++g)
                *reinterpret_cast<float4*>(arr + (i + 4 * g)) = make_float4(x[4 * g], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]);
        } else {
#pragma unroll
            for (int g = 0; g < N / 2; ++g) *reinterpret_cast<float2*>(arr + (i + 2 * g)) = make_float2(x[2 * g], x[2 * g + 1]);
        }
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
    template <bool PERM, int GPR, int KIND>
    __device__ static __forceinline__ frag ld_col_swz(const E* arr, int base, int col0, int kb, int q4, int l16) {
        const int er = l16 >> 2, c = col0 + 4 * (l16 & 3);
        const int r0 = PERM ? jperm(kb, q4, er) : inat(kb, q4, er);
        const int r1 = PERM ? jperm(kb, q4, 4 + er) : inat(kb, q4, 4 + er);
        const shortx4 x =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(arr + (base + swz_elem<GPR, KIND, 8>(r0, c))));
        const shortx4 y =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(arr + (base + swz_elem<GPR, KIND, 8>(r1, c))));
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
    // N consecutive values as hi / lo planes (N*2 bytes aligned to min(16, N*2))
    template <int N>
    __device__ static __forceinline__ void put_row(E* arr, int ps, int i, const float (&x)[N]) {
        static_assert(N % 2 == 0, "pairs of bf16");
        uint32_t hi[N / 2], lo[N / 2];
#pragma unroll
        for (int p = 0; p < N / 2; ++p) hi[p] = split2(x[2 * p], x[2 * p + 1], lo[p]);
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int g = 0; g < N / 8; ++g) {
                *reinterpret_cast<uint4*>(arr + (i + 8 * g)) = make_uint4(hi[4 * g], hi[4 * g + 1], hi[4 * g + 2], hi[4 * g + 3]);
                *reinterpret_cast<uint4*>(arr + (ps + i + 8 * g)) =
                    make_uint4(lo[4 * g], lo[4 * g + 1], lo[4 * g + 2], lo[4 * g + 3]);
            }
        } else if constexpr (N == 4) {
            *reinterpret_cast<uint2*>(arr + i) = make_uint2(hi[0], hi[1]);
            *reinterpret_cast<uint2*>(arr + (ps + i)) = make_uint2(lo[0], lo[1]);
        } else {
            *reinterpret_cast<uint32_t*>(arr + i) = hi[0];
            *reinterpret_cast<uint32_t*>(arr + (ps + i)) = lo[0];
        }
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

// Direct loads of a swizzled chunk tile of NBYTES (a multiple of 1024) whose rows are RB
// bytes of a global row every gpitch bytes.  Wave w issues instructions r = w, w + NW, ...;
// instruction r fills tile granules 64r .. 64r + 63, lane l granule p = 64r + l, which holds
// granule swz(row, p % GPR) of row p / GPR (the swizzle is an XOR, its own inverse).  The
// per-lane global offsets are computed once; rows at or past the sequence end (only in a
// chunk with fewer than NBYTES / RB valid rows) repeat the last valid row.
template <int NBYTES, int RB, int NW, int KIND>
struct TileDma {
    static constexpr int NI = (NBYTES / 1024 + NW - 1) / NW;  // instructions per wave, at most
    static constexpr int ROWS = NBYTES / RB;                  // rows the tile spans, padding included
    static constexpr int GPR = RB / 16;
    long goff[NI];
    __device__ static __forceinline__ long offset(int p, int nrow_max, long gpitch) {
        const int row = p / GPR;
        const int g = swz<GPR, KIND>(row, p % GPR);
        return long(min(row, nrow_max)) * gpitch + 16 * g;
    }
    __device__ __forceinline__ void init(int w, int lane, long gpitch) {
#pragma unroll
        for (int j = 0; j < NI; ++j) goff[j] = offset((w + NW * j) * 64 + lane, ROWS, gpitch);
    }
    __device__ __forceinline__ void issue(void* lds, const char* base, int w, int lane, int nv, long gpitch) const {
#pragma unroll
        for (int j = 0; j < NI; ++j) {
            const int r = w + NW * j;
            if (NBYTES % (1024 * NW) == 0 || r * 1024 < NBYTES) {
                const long go = nv < ROWS ? offset(r * 64 + lane, nv - 1, gpitch) : goff[j];
                __builtin_amdgcn_global_load_lds(base + go, (lds_void*)(static_cast<unsigned char*>(lds) + r * 1024),
                                                 16, 0, 0);
            }
        }
    }
};

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

// Inclusive product scan across the 64 lanes of a wave (lane order): DPP row shifts by 1, 2,
// 4, 8 within rows of 16 lanes, then row broadcasts of lane 15 and lane 31.  Lanes without a
// source lane in a step multiply by 1 (the "old" operand of the DPP move).
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float scan_mul_step(float x) {
    const int y = __builtin_amdgcn_update_dpp(__float_as_int(1.0f), __float_as_int(x), CTRL, ROWMASK, 0xF, false);
    return x * __int_as_float(y);
}
__device__ __forceinline__ float wave_scan_mul(float x) {
    x = scan_mul_step<0x111, 0xF>(x);  // row_shr:1
    x = scan_mul_step<0x112, 0xF>(x);  // row_shr:2
    x = scan_mul_step<0x114, 0xF>(x);  // row_shr:4
    x = scan_mul_step<0x118, 0xF>(x);  // row_shr:8
    x = scan_mul_step<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x = scan_mul_step<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// The same scan on N independent values with the DPP folded into the multiply: a lane whose
// source lane is outside the row (or whose row is masked off) is not written and keeps its
// value.  A DPP read of a VGPR needs two instructions after the VALU write of that VGPR:
// the s_nop covers the writes before the first step, and with N >= 3 values interleaved
// every later step reads registers written N instructions earlier.
#define RSM_SCAN_STEP(CTRL)                                                                        \
    _Pragma("unroll") for (int i = 0; i < N; ++i) asm volatile("v_mul_f32_dpp %0, %0, %0 " CTRL   \
                                                               " bank_mask:0xf"                  \
                                                               : "+v"(x[i]));
template <int N>
__device__ __forceinline__ void wave_scan_mul_n(float (&x)[N]) {
    if constexpr (N < 3) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = wave_scan_mul(x[i]);
    } else {
        asm volatile("s_nop 1");
        RSM_SCAN_STEP("row_shr:1 row_mask:0xf")
        RSM_SCAN_STEP("row_shr:2 row_mask:0xf")
        RSM_SCAN_STEP("row_shr:4 row_mask:0xf")
        RSM_SCAN_STEP("row_shr:8 row_mask:0xf")
        RSM_SCAN_STEP("row_bcast:15 row_mask:0xa")
        RSM_SCAN_STEP("row_bcast:31 row_mask:0xc")
    }
}
#undef RSM_SCAN_STEP

// alpha clamped below at e^-30 for the factored path: alpha is in [0, 1], so the larger
// value is the larger bit pattern (one integer max, no NaN canonicalisation).
__device__ __forceinline__ float clamp_alpha(float a) {
    return __int_as_float(max(__float_as_int(a), __float_as_int(kAlphaMin)));
}

// N consecutive input elements (N*sizeof(T) a multiple of 4 bytes, aligned) -> fp32
template <int N>
__device__ __forceinline__ void load_row(const bf16_t* arr, int off, float (&x)[N]) {
    static_assert(N % 2 == 0, "pairs of bf16");
    uint32_t wds[N / 2];
    if constexpr (N % 8 == 0) {
#pragma unroll
        for (int g = 0; g < N / 8; ++g) {
            const uint4 u = *reinterpret_cast<const uint4*>(arr + (off + 8 * g));
            wds[4 * g] = u.x; wds[4 * g + 1] = u.y; wds[4 * g + 2] = u.z; wds[4 * g + 3] = u.w;
        }
    } else if constexpr (N == 4) {
        const uint2 u = *reinterpret_cast<const uint2*>(arr + off);
        wds[0] = u.x; wds[1] = u.y;
    } else {
        wds[0] = *reinterpret_cast<const uint32_t*>(arr + off);
    }
#pragma unroll
    for (int p = 0; p < N / 2; ++p) {
        x[2 * p] = __uint_as_float(wds[p] << 16);
        x[2 * p + 1] = __uint_as_float(wds[p] & 0xFFFF0000u);
    }
}
template <int N>
__device__ __forceinline__ void load_row(const float* arr, int off, float (&x)[N]) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int g = 0; g < N / 4; ++g) {
            const float4 u = *reinterpret_cast<const float4*>(arr + (off + 4 * g));
            x[4 * g] = u.x; x[4 * g + 1] = u.y; x[4 * g + 2] = u.z; x[4 * g + 3] = u.w;
        }
    } else {
#pragma unroll
        for (int g = 0; g < N / 2; ++g) {
            const float2 u = *reinterpret_cast<const float2*>(arr + (off + 2 * g));
            x[2 * g] = u.x; x[2 * g + 1] = u.y;
        }
    }
}

// N consecutive elements of row `row` from column col0 of a swizzled tile (col0 a multiple
// of min(N, elements per granule)); read granule piece by granule piece
template <int N, int GPR, int KIND, typename T>
__device__ __forceinline__ void load_row_swz(const T* arr, int row, int col0, float (&x)[N]) {
    constexpr int EPG = 16 / int(sizeof(T));
    constexpr int PE = N < EPG ? N : EPG;  // elements per piece
#pragma unroll
    for (int pc = 0; pc < N / PE; ++pc) {
        float y[PE];
        load_row<PE>(arr, swz_elem<GPR, KIND, EPG>(row, col0 + pc * PE), y);
#pragma unroll
        for (int e = 0; e < PE; ++e) x[pc * PE + e] = y[e];
    }
}


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
// pass_a: pass A of the segment split (no Qh, no outputs; writes dH, dE).
//
// Wave roles (w = 0..7, all uniform):
//  * decay products, Qh, Kh: lane = token of the chunk, wave w = slots w*SPW .. w*SPW+SPW-1;
//  * chunk-row tile Tt of S^T and O^T: waves w and w + NTC*g share Tt; odd groups take the
//    tiles in reverse so that the two waves of a SIMD (w, w+4) get a cheap and a costly tile;
//  * slot tile I = w % NTM of U^T and of the state, column tiles gI, gI + GI, ...
// ------------------------------------------------------------------------------------
template <typename T, int M, int C, int DT>
__global__ __launch_bounds__(512) void fwd_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ H0,
    long T_len, int Hh, int Dv, int K, SegArgs sg, int pass_a, const unsigned long long* __restrict__ rmask,
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
    constexpr int GH = DT * int(sizeof(E)) / 16;   // granules per row of the state copy (swizzled)
    constexpr int GQK = M * int(sizeof(T)) / 16;   // granules per row of the q / k tiles
    constexpr int GV = DT * int(sizeof(T)) / 16;   // granules per row of the v tile
    constexpr int EPG = 16 / int(sizeof(T));       // elements per granule
    constexpr int NTC = C / 16, NTCP = CP / 16, NTD = DT / 16, NTM = M / 16;
    constexpr int NKM = MP / KB, NKC = CP / KB;
    constexpr int GT = NW / NTC;               // waves per chunk-row tile
    constexpr int NOD = (NTD + GT - 1) / GT;   // output column tiles per wave
    constexpr int GI = NW / NTM;               // waves per slot tile
    constexpr int UPW = (NTD + GI - 1) / GI;   // state tiles per wave
    constexpr int SPW = M / NW;                // slots per wave in the decay-product pass
    constexpr int MW = (M + 63) / 64;          // 64-bit words of a token's selection mask
    constexpr int psQ = CP * QP + 8;           // plane stride of Qh / Kh
    constexpr int oK = NPL * psQ;              // Kh planes start here
    constexpr int psH = MP * DT;               // plane stride of the state copy
    constexpr int SZQK = 2 * NPL * psQ;
    constexpr int SZHF = M * DT * 4 / int(sizeof(E));
    static_assert(NW % NTC == 0 && NW % NTM == 0 && SPW >= 2 && SPW <= 16 && C <= 64, "tile split");

    // LDS.  Raw inputs land by direct loads (tile arrays padded to 1 KB); every array is a
    // separate object so the compiler can tell the direct loads from the other accesses.
    __shared__ __align__(16) T rq[pad1k(C * M * int(sizeof(T))) / int(sizeof(T))];
    __shared__ __align__(16) T rk[pad1k(C * M * int(sizeof(T))) / int(sizeof(T))];
    __shared__ __align__(16) T rv0[pad1k(CP * DT * int(sizeof(T))) / int(sizeof(T))];  // v, even chunks
    __shared__ __align__(16) T rv1[pad1k(CP * DT * int(sizeof(T))) / int(sizeof(T))];  // v, odd chunks
    __shared__ __align__(16) unsigned long long rMask[pad1k(C * MW * 8) / 8];  // selection masks
    __shared__ __align__(16) float rA[pad1k(C * M * 4) / 4];  // alpha lists; exact path: dense alphas [C][M]
    __shared__ __align__(16) E sQK[SZQK > SZHF ? SZQK : SZHF];      // Qh planes, then Kh planes
    __shared__ __align__(16) E sH[NPL * psH];                       // state copy, row-major [i][d]
    __shared__ __align__(16) float sE[M];
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
    __builtin_assume(w >= 0 && w < NW);
    const int gT = w / NTC;
    const int Tt = (gT & 1) ? NTC - 1 - w % NTC : w % NTC;
    const int I = w % NTM, gI = w / NTM;
    const int s0 = w * SPW;                         // first slot of this wave's decay products
    const long rstride = long(Hh);                  // rows between consecutive tokens of one head
    const long segrow = (bh * (sg.S - 1) + seg) * M;  // row of this segment in dH / dE

    // ---- direct loads of chunk c's inputs (rows past the sequence end repeat the last row;
    // their tokens carry no route entries, so they contribute nothing)
    const long qk_pitch = rstride * M * long(sizeof(T)), v_pitch = rstride * Dv * long(sizeof(T));
    TileDma<int(sizeof(rk)), M * int(sizeof(T)), NW, 1> dqk;
    TileDma<int(sizeof(rv0)), DT * int(sizeof(T)), NW, 2> dv;
    dqk.init(w, lane, qk_pitch);
    dv.init(w, lane, v_pitch);
    auto issue_qk = [&](long c) {
        const int nv = int(T_len - c * C < C ? T_len - c * C : C);
        const long row0 = ((b * T_len + c * C) * rstride + h) * M;
        dqk.issue(rk, reinterpret_cast<const char*>(k + row0), w, lane, nv, qk_pitch);
        if (!pass_a) dqk.issue(rq, reinterpret_cast<const char*>(q + row0), w, lane, nv, qk_pitch);
    };
    auto issue_v = [&](long c, T* dst) {
        const int nv = int(T_len - c * C < C ? T_len - c * C : C);
        dv.issue(dst, reinterpret_cast<const char*>(v + ((b * T_len + c * C) * rstride + h) * Dv + d0), w, lane, nv,
                 v_pitch);
    };
    auto issue_route = [&](long c) {
        const char* ab = reinterpret_cast<const char*>(ralpha + (bh * T_pad + c * C) * K);
        const char* mb = reinterpret_cast<const char*>(rmask + (bh * T_pad + c * C) * MW);
        const int na = C * K * 4, nm = C * MW * 8;
        dma_tile<NW>(rA, pad1k(na), w, lane, [&](int off) { return static_cast<const void*>(ab + min(off, na - 16)); });
        dma_tile<NW>(rMask, pad1k(nm), w, lane,
                     [&](int off) { return static_cast<const void*>(mb + min(off, nm - 16)); });
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
            if (D < NTD) P::put4(sH, psH, swz_elem<GH, 3, EVE>(i, 16 * D + 4 * q4), Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
        }
    }
    if (c_begin < c_end) {
        issue_qk(c_begin);
        issue_v(c_begin, rv0);
        issue_route(c_begin);
    }

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

        // ---- decay products, Qh = q o E and Kh = k (1 - alpha) / E (0 where alpha = 1).
        // Lane = token t of the chunk, this wave's slots s0 .. s0 + SPW - 1.  The lane gathers
        // its alphas through the token's selection mask (position in the alpha list = number
        // of selected slots below); E is an inclusive product scan across the lanes of the
        // clamped alphas.  Tokens past the sequence end have alpha = 1.
        float al[SPW], Ev[SPW];
        {
            const int tc = lane < C ? lane : C - 1;
            unsigned long long word = 0ull;
            int base = 0;
            if (lane < nvalid) {
                const unsigned long long w0 = rMask[tc * MW];
                if (MW == 1 || s0 < 64) {
                    word = w0;
                    base = __popcll(w0 & ((1ull << (s0 & 63)) - 1ull));
                } else {
                    word = rMask[tc * MW + 1];
                    base = __popcll(w0) + __popcll(word & ((1ull << (s0 & 63)) - 1ull));
                }
            }
            const uint32_t g = uint32_t(word >> (s0 & 63));
            int idx = base;
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                const bool sel = (g >> j) & 1u;
                const float a = rA[(idx < K ? idx : K - 1) * C + tc];
                al[j] = sel ? a : 1.0f;
                idx += sel ? 1 : 0;
            }
        }
        int bad = 0;
#pragma unroll
        for (int j = 0; j < SPW; ++j) Ev[j] = clamp_alpha(al[j]);
        wave_scan_mul_n<SPW>(Ev);
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const float el = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Ev[j]), 63));
            bad |= !(el >= kSafeMin);
        }
        if (lane == 63) {  // E at the chunk end, per slot
#pragma unroll
            for (int j = 0; j < SPW; ++j) sE[s0 + j] = Ev[j];
        }
        if (lane == 0) sFlag[w] = bad;
        if (lane < C) {
            float x[SPW];
            load_row_swz<SPW, GQK, 1>(rk, lane, s0, x);
#pragma unroll
            for (int j = 0; j < SPW; ++j) x[j] = x[j] * (1.0f - clamp_alpha(al[j])) * __builtin_amdgcn_rcpf(Ev[j]);
            P::template put_row<SPW>(sQK, psQ, oK + lane * QP + s0, x);
            if (!pass_a) {
                load_row_swz<SPW, GQK, 1>(rq, lane, s0, x);
#pragma unroll
                for (int j = 0; j < SPW; ++j) x[j] *= Ev[j];
                P::template put_row<SPW>(sQK, psQ, lane * QP + s0, x);
            }
        }
        wg_barrier();
        int unsafe = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) unsafe |= sFlag[i];

        if (unsafe) {
            // ---- exact token-by-token recurrence with the exact alphas, on an fp32 copy.
            // Dense exact alphas [C][M] go where the alpha lists were (all lists are read).
            if (lane < C) {
                float x[SPW];
#pragma unroll
                for (int j = 0; j < SPW; ++j) x[j] = al[j];
                Pol<float>::template put_row<SPW>(rA, 0, lane * M + s0, x);
            }
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
                    const float a = rA[tt * M + i];
                    if (a != 1.0f) {
                        const float wk = (1.0f - a) * Elem<T>::load(rk, swz_elem<GQK, 1, EPG>(tt, i));
                        sHf[e] = fmaf(a, sHf[e], wk * Elem<T>::load(rvc, swz_elem<GV, 2, EPG>(tt, dd)));
                    }
                }
                wg_barrier();
                if (!pass_a && tid < DT) {
                    float acc = 0.0f;
                    for (int i = 0; i < M; ++i)
                        acc = fmaf(Elem<T>::load(rq, swz_elem<GQK, 1, EPG>(tt, i)), sHf[i * DT + tid], acc);
                    o[((b * T_len + tokc + tt) * rstride + h) * Dv + d0 + tid] = acc;
                }
                wg_barrier();
            }
            if (tid < M) {  // decay product of the chunk with the exact alphas
                float e = 1.0f;
                for (int tt = 0; tt < nvalid; ++tt) e *= rA[tt * M + tid];
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
                        P::put4(sH, psH, swz_elem<GH, 3, EVE>(i, 16 * D + 4 * q4), Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
                }
            } else {
                Eseg *= sE[16 * I + l16];
            }
            if (c + 1 < c_end) {
                issue_qk(c + 1);
                issue_route(c + 1);
            }
            return;
        }

        if (c + 1 < c_end) {
            issue_qk(c + 1);
            issue_route(c + 1);
        }

        // ---- S^T = Kh Qh^T (masked) and O^T = V^T P^T + H_c^T Qh^T for chunk-row tile TT
        // (a compile-time tile index, so the masked tiles and k-blocks drop out statically)
        auto so_phase = [&](auto ttc) __attribute__((always_inline)) {
            constexpr int TT = decltype(ttc)::value;
            float* obase = o + ((b * T_len + tokc) * rstride + h) * Dv + d0;
            dfrag qf[NKM];
#pragma unroll
            for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
                    qf[kb].p[pl] = P::ld(sQK, pl * psQ + (16 * TT + l16) * QP + kb * KB + EPL * q4);
            floatx4 st[NTCP];
#pragma unroll
            for (int J = 0; J < NTCP; ++J) {
                st[J] = floatx4{0.f, 0.f, 0.f, 0.f};
                if constexpr (true) {
                    if (J <= TT && J < NTC) {
                        dfrag a[NKM];
#pragma unroll
                        for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                            for (int pl = 0; pl < NPL; ++pl)
                                a[kb].p[pl] = P::ld(sQK, oK + pl * psQ + (16 * J + l16) * QP + kb * KB + EPL * q4);
#pragma unroll
                        for (int kb = 0; kb < NKM; ++kb) st[J] = P::mm_dd(a[kb], qf[kb], st[J]);
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (4 * q4 + r > l16) st[TT][r] = 0.0f;  // j > t on the diagonal tile
            dfrag pf[NKC];
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb) pf[kb] = P::pack_perm(st, kb);
            const int tl = 16 * TT + l16;
            floatx4 acc[NOD];
#pragma unroll
            for (int jd = 0; jd < NOD; ++jd) {
                const int D = gT + GT * jd;
                acc[jd] = floatx4{0.f, 0.f, 0.f, 0.f};
                if (NTD % GT == 0 || D < NTD) {
                    frag va[NKC];
                    dfrag ha[NKM];
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        if (kb * KB < 16 * (TT + 1)) va[kb] = P::template ld_col_swz<true, GV, 2>(rvc, 0, 16 * D, kb, q4, l16);
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb)
#pragma unroll
                        for (int pl = 0; pl < NPL; ++pl)
                            ha[kb].p[pl] = P::template ld_col_swz<false, GH, 3>(sH, pl * psH, 16 * D, kb, q4, l16);
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        if (kb * KB < 16 * (TT + 1)) acc[jd] = P::mm_vd(va[kb], pf[kb], acc[jd]);
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb) acc[jd] = P::mm_dd(ha[kb], qf[kb], acc[jd]);
                }
            }
#pragma unroll
            for (int jd = 0; jd < NOD; ++jd) {
                const int D = gT + GT * jd;
                if ((NTD % GT == 0 || D < NTD) && tl < nvalid)
                    *reinterpret_cast<float4*>(obase + tl * rstride * Dv + 16 * D + 4 * q4) =
                        make_float4(acc[jd][0], acc[jd][1], acc[jd][2], acc[jd][3]);
            }
        };
        if (!pass_a) {
            switch (Tt) {
                case 0: so_phase(std::integral_constant<int, 0>{}); break;
                case 1: if constexpr (NTC > 1) so_phase(std::integral_constant<int, 1>{}); break;
                case 2: if constexpr (NTC > 2) so_phase(std::integral_constant<int, 2>{}); break;
                case 3: if constexpr (NTC > 3) so_phase(std::integral_constant<int, 3>{}); break;
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
                    for (int kb = 0; kb < NKC; ++kb) va[kb] = P::template ld_col_swz<true, GV, 2>(rvc, 0, 16 * D, kb, q4, l16);
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
                    P::put4(sH, psH, swz_elem<GH, 3, EVE>(i, 16 * D + 4 * q4), Hreg[j][0], Hreg[j][1], Hreg[j][2], Hreg[j][3]);
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
    pick_segments(B * Hh * (Dv / L.dt), L.n_chunks, L.S, L.cps);
    const size_t rows = size_t(B) * size_t(Hh) * size_t(L.n_chunks) * size_t(C);  // padded token-heads
    if (rows == 0) return L;
    const size_t mw = size_t(M + 63) / 64;
    size_t off = 0;
    L.rmask_off = off;
    off += align256(rows * mw * 8);
    L.ralpha_off = off;
    off += align256(rows * size_t(K) * 4);
    const size_t segs = size_t(B) * size_t(Hh) * size_t(L.S - 1);
    L.dh_off = off;
    off += align256(segs * size_t(M) * size_t(Dv) * 4);
    L.de_off = off;
    off += align256(segs * size_t(M) * 4);
    L.total = off;
    return L;
}

template <typename T, int M, int C, int DT>
static int launch_scan(const T* q, const T* k, const T* v, const float* H0, long B, long T_len, long Hh, int Dv,
                       int K, const SegArgs& sg, const unsigned long long* rmask, const float* ralpha, float* o,
                       float* H_out, hipStream_t s) {
    const long tiles = B * Hh * (Dv / DT);
    if (sg.S > 1) {
        hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT>), dim3(unsigned(tiles * (sg.S - 1))), dim3(512), 0, s, q, k,
                           v, H0, T_len, int(Hh), Dv, K, sg, 1, rmask, ralpha, o, H_out);
        if (hipGetLastError() != hipSuccess) return RSM_ERR_HIP;
    }
    hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT>), dim3(unsigned(tiles * sg.S)), dim3(512), 0, s, q, k, v, H0,
                       T_len, int(Hh), Dv, K, sg, 0, rmask, ralpha, o, H_out);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

struct ScanArgs {
    const void *q, *k, *v;
    const float* H0;
    long B, T_len, Hh;
    int Dv, K;
    SegArgs sg;
    const unsigned long long* rmask;
    const float* ralpha;
    float *o, *H_out;
    hipStream_t s;
};

template <typename T, int M, int C>
static int dispatch_dt(int DT, const ScanArgs& a) {
    const T *q = static_cast<const T*>(a.q), *k = static_cast<const T*>(a.k), *v = static_cast<const T*>(a.v);
#define RSM_SCAN(DTV) \
    return launch_scan<T, M, C, DTV>(q, k, v, a.H0, a.B, a.T_len, a.Hh, a.Dv, a.K, a.sg, a.rmask, a.ralpha, a.o, a.H_out, a.s)
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
static int dispatch_c(int C, int DT, const ScanArgs& a) {
    switch (C) {
        case 16: return dispatch_dt<T, M, 16>(DT, a);
        case 32: return dispatch_dt<T, M, 32>(DT, a);
        case 64:
            if constexpr (M < 128) return dispatch_dt<T, M, 64>(DT, a);
            break;
    }
    return RSM_ERR_UNSUPPORTED;
}

template <typename T>
static int dispatch_m(int M, int C, int DT, const ScanArgs& a) {
    switch (M) {
        case 16: return dispatch_c<T, 16>(C, DT, a);
        case 32: return dispatch_c<T, 32>(C, DT, a);
        case 64: return dispatch_c<T, 64>(C, DT, a);
        case 128: return dispatch_c<T, 128>(C, DT, a);
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
    auto* rmask = reinterpret_cast<unsigned long long*>(ws + L.rmask_off);
    auto* ralpha = reinterpret_cast<float*>(ws + L.ralpha_off);
    const SegArgs sg{L.n_chunks, L.S, L.cps, reinterpret_cast<float*>(ws + L.dh_off),
                     reinterpret_cast<float*>(ws + L.de_off)};
    int st = route_fwd_launch(z, dtype, f, B, T, Hh, L.n_chunks * L.chunk, M, K, L.chunk, idx_out, rmask, ralpha,
                              stream);
    if (st != RSM_OK) return st;
    const ScanArgs a{q, k, v, H0, B, T, Hh, Dv, K, sg, rmask, ralpha, o, H_out, stream};
    if (dtype == RSM_F32) return dispatch_m<float>(M, L.chunk, L.dt, a);
    return dispatch_m<bf16_t>(M, L.chunk, L.dt, a);
}

}  // namespace rsm
