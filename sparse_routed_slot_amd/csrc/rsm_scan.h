#pragma once
// rsm_scan.h -- chunked forward of the RSM mixer: sparse decay, intra-chunk and
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
//  * fwd_scan (one workgroup per (batch, head, Dv tile, sequence segment)): walks the
//    segment's chunks in order with the fp32 state tile in registers, split by column tiles
//    among the waves that own them.  The chunk's v tile and its route arrive in LDS by direct
//    global->LDS loads issued a phase ahead; q and k come into registers.  For the decay
//    products each lane takes one token and each wave a group of slots: the lane gathers its
//    alphas from the route, E comes from a product scan across the wave's lanes, and the lane
//    writes its rows of Qh and Kh.  The contractions run on 16x16 MFMA tiles, o is written,
//    and the state is updated.  Rows of slots untouched in a chunk (E_last == 1) keep their
//    exact bits.
//
// Overflow guard: 1/E grows with the decay accumulated in a chunk.  On the factored path each
// alpha is clamped below at e^-30 (~1e-13 instead of 0); a chunk whose decay product falls
// below 2^-100 for some slot is evaluated token by token with the exact alphas instead.
#include <type_traits>
#include <utility>

#include "rsm_device.h"
#include "rsm_launch.h"
#include "rsm_scan_args.h"
#include "rsm_route_row.h"

namespace rsm {

constexpr float kAlphaMin = 9.3576230e-14f;  // e^-30: clamp of alpha on the factored path
constexpr float kSafeMin = 7.8886091e-31f;   // 2^-100: smallest E_last kept factored
// Raw buffer resources for the output stores: no stride, range kOutRange bytes from the chunk's
// first output row (far past any row of a chunk); an offset past it drops the store.
constexpr int kOutRange = 0x7FFFFF00;
constexpr int kBufferFlags = 0x00020000;  // dword 3 of a gfx9 buffer resource
typedef uint32_t uint32x4 __attribute__((ext_vector_type(4)));
// Pass B folds up to this many earlier segment states itself; beyond that a separate kernel
// folds them between the passes.
constexpr int kFoldMax = 3;

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
// Qh, Kh, P and the state are fp32 values: each is carried as a pair hi + lo of bf16
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
// Swizzled tiles.  The raw v tile arrives in LDS by direct loads that fill 16-byte granules
// in order, so its rows cannot be padded; instead granule g of row `row` (GPR granules per
// row) sits at granule position row*GPR + swz(row, g), an XOR of g with a function of the
// row, so that the rows a wave reads at once fall into different banks.  KIND 2 (8-byte
// column pieces of 4 rows and 2 adjacent granules per 16 lanes): g ^ 2*((row / RPB) %
// (GPR/2)), which keeps granule pairs together, with RPB = max(1, 16 / GPR) rows per
// 256-byte bank sweep.  KIND 0: no swizzle.
//
// Every LDS access is written as one offset from its array (arr + off): the compiler then
// keeps track of which array each access touches and does not make it wait for the direct
// global->LDS loads still in flight into other arrays.
template <int GPR, int KIND>
__device__ __forceinline__ int swz(int row, int g) {
    if constexpr (GPR <= 1 || KIND == 0) {
        return g;
    } else {
        static_assert(KIND == 2, "swizzle kind");
        constexpr int RPB = GPR >= 16 ? 1 : 16 / GPR;
        if constexpr (GPR >= 4) return g ^ (2 * ((row / RPB) % (GPR / 2)));
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
    __device__ static __forceinline__ floatx4 mm_dv(const dfrag& a, frag v, floatx4 c) { return mma(a.p[0], v, c); }
    // k-fragment kb of a row (element offset off) in the slot order jperm
    __device__ static __forceinline__ frag ld_jrow(const E* arr, int off, int kb, int q4) {
        return arr[off + jperm(kb, q4, 0)];
    }
    // P^T fragments: block (TT, kb) of 64 values, lane l's at l; accumulator tile J of row
    // tile TT holds the fragments kb = 4J + r
    template <int NKC>
    __device__ static __forceinline__ void put_pfrag(E* arr, int psP, int TT, int J, int lane, floatx4 x) {
#pragma unroll
        for (int r = 0; r < 4; ++r) arr[(TT * NKC + 4 * J + r) * 64 + lane] = x[r];
    }
    template <int NKC>
    __device__ static __forceinline__ dfrag ld_pfrag(const E* arr, int psP, int TT, int kb, int lane) {
        return dfrag{{arr[(TT * NKC + kb) * 64 + lane]}};
    }
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
    __device__ static __forceinline__ floatx4 mm_dv(const dfrag& a, frag v, floatx4 c) {
        c = mma(a.p[1], v, c);
        return mma(a.p[0], v, c);
    }
    // k-fragment kb of a row (element offset off, 8-byte aligned) in the slot order jperm:
    // slots 32kb + 4q4 + 0..3 and 32kb + 16 + 4q4 + 0..3
    __device__ static __forceinline__ frag ld_jrow(const E* arr, int off, int kb, int q4) {
        const uint2 x = *reinterpret_cast<const uint2*>(arr + (off + 32 * kb + 4 * q4));
        const uint2 y = *reinterpret_cast<const uint2*>(arr + (off + 32 * kb + 16 + 4 * q4));
        return __builtin_bit_cast(frag, make_uint4(x.x, x.y, y.x, y.y));
    }
    // P^T fragments: block (TT, kb) of 64 lanes x 8 values per plane, lane l's at 8l;
    // accumulator tile J of row tile TT is the k-half J % 2 of the fragments kb = J / 2
    template <int NKC>
    __device__ static __forceinline__ void put_pfrag(E* arr, int psP, int TT, int J, int lane, floatx4 x) {
        uint32_t l0, l1;
        const uint32_t h0 = split2(x[0], x[1], l0), h1 = split2(x[2], x[3], l1);
        const int off = (TT * NKC + (J >> 1)) * 512 + lane * 8 + (J & 1) * 4;
        *reinterpret_cast<uint2*>(arr + off) = make_uint2(h0, h1);
        *reinterpret_cast<uint2*>(arr + (psP + off)) = make_uint2(l0, l1);
    }
    template <int NKC>
    __device__ static __forceinline__ dfrag ld_pfrag(const E* arr, int psP, int TT, int kb, int lane) {
        const int off = (TT * NKC + kb) * 512 + lane * 8;
        dfrag r;
        r.p[0] = ld(arr, off);
        r.p[1] = ld(arr, psP + off);
        return r;
    }
};



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

// s_waitcnt vmcnt(N) only (expcnt and lgkmcnt unconstrained): all but the N most recent
// vector memory instructions of this wave have completed (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x70 | 0xF00);
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
// FULL = false: separate scans over lanes 0-31 and 32-63 (the row_bcast:31 step left out).
template <bool FULL>
__device__ __forceinline__ float wave_scan_mul(float x) {
    x = scan_mul_step<0x111, 0xF>(x);  // row_shr:1
    x = scan_mul_step<0x112, 0xF>(x);  // row_shr:2
    x = scan_mul_step<0x114, 0xF>(x);  // row_shr:4
    x = scan_mul_step<0x118, 0xF>(x);  // row_shr:8
    x = scan_mul_step<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    if constexpr (FULL) x = scan_mul_step<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return x;
}

// The same scan on N independent values with the DPP folded into the multiply: a lane whose
// source lane is outside the row (or whose row is masked off) is not written and keeps its
// value.  A DPP read of a VGPR needs two wait states after a VALU write of that VGPR, which
// the compiler does not check for inline assembly, so the whole scan is one asm block: its
// leading s_nop covers whatever the compiler wrote last (copies into the operand registers
// included), and inside it every step reads a register written N >= 4 instructions earlier.
#define RSM_DPP(CTRL, I) "v_mul_f32_dpp %" #I ", %" #I ", %" #I " " CTRL " bank_mask:0xf\n"
#define RSM_DPP4(CTRL, A, B, C, D) RSM_DPP(CTRL, A) RSM_DPP(CTRL, B) RSM_DPP(CTRL, C) RSM_DPP(CTRL, D)
#define RSM_STEPS4(CTRL) RSM_DPP4(CTRL, 0, 1, 2, 3)
#define RSM_STEPS8(CTRL) RSM_STEPS4(CTRL) RSM_DPP4(CTRL, 4, 5, 6, 7)
#define RSM_STEPS16(CTRL) RSM_STEPS8(CTRL) RSM_DPP4(CTRL, 8, 9, 10, 11) RSM_DPP4(CTRL, 12, 13, 14, 15)
#define RSM_SCAN_ASM32(STEPS)                                                                     \
    "s_nop 1\n" STEPS("row_shr:1 row_mask:0xf") STEPS("row_shr:2 row_mask:0xf")                 \
        STEPS("row_shr:4 row_mask:0xf") STEPS("row_shr:8 row_mask:0xf")                          \
            STEPS("row_bcast:15 row_mask:0xa")
#define RSM_SCAN_ASM(STEPS) RSM_SCAN_ASM32(STEPS) STEPS("row_bcast:31 row_mask:0xc")
// FULL = false: separate scans over lanes 0-31 and 32-63.
template <int N, bool FULL = true>
__device__ __forceinline__ void wave_scan_mul_n(float (&x)[N]) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "scan width");
    if constexpr (N == 32) {  // two blocks of 16 independent values
        wave_scan_mul_n<16, FULL>(*reinterpret_cast<float(*)[16]>(&x[0]));
        wave_scan_mul_n<16, FULL>(*reinterpret_cast<float(*)[16]>(&x[16]));
    } else if constexpr (N == 2) {
        x[0] = wave_scan_mul<FULL>(x[0]);
        x[1] = wave_scan_mul<FULL>(x[1]);
    } else if constexpr (N == 4) {
        if constexpr (FULL)
            asm volatile(RSM_SCAN_ASM(RSM_STEPS4) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
        else
            asm volatile(RSM_SCAN_ASM32(RSM_STEPS4) : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
    } else if constexpr (N == 8) {
        if constexpr (FULL)
            asm volatile(RSM_SCAN_ASM(RSM_STEPS8)
                         : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                           "+v"(x[7]));
        else
            asm volatile(RSM_SCAN_ASM32(RSM_STEPS8)
                         : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                           "+v"(x[7]));
    } else {
        if constexpr (FULL)
            asm volatile(RSM_SCAN_ASM(RSM_STEPS16)
                         : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                           "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),
                           "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
        else
            asm volatile(RSM_SCAN_ASM32(RSM_STEPS16)
                         : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                           "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),
                           "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
    }
}
#undef RSM_SCAN_ASM
#undef RSM_SCAN_ASM32
#undef RSM_STEPS16
#undef RSM_STEPS8
#undef RSM_STEPS4
#undef RSM_DPP4
#undef RSM_DPP

// alpha clamped below at e^-30 for the factored path: alpha is in [0, 1], so the larger
// value is the larger bit pattern (one integer max, no NaN canonicalisation).
__device__ __forceinline__ float clamp_alpha(float a) {
    return __int_as_float(max(__float_as_int(a), __float_as_int(kAlphaMin)));
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

// ------------------------------------------------------------------------------------
// Chunk scan: one workgroup (8 or 16 waves) per (b, h, Dv tile of DT columns, segment); it walks
// the segment's chunks in order.
//
// The fp32 state tile stays in registers, split by column tiles: wave w owns column tile
// D = w % NTD for every slot, as 16x16 accumulator tiles H[16*I + 4*q4 + r][16*D + l16]
// (the NW / NTD waves of one column tile keep identical copies).  In that layout the tiles
// 2*kb and 2*kb + 1 are, element for element, the k-fragment kb of H^T in the slot order
// jperm, so the state feeds the output contraction without going through LDS.
//
// A chunk c takes two phases, each closed by a workgroup barrier:
//  X (pass B only): S^T = Kh Qh^T on its lower-triangular 16x16 tiles, spread over the
//    waves, masked, and stored as ready-made MFMA fragments of P^T;
//  Y: O^T = V^T P^T + H_c^T Qh^T for the wave's column tile (pass B), U = Kh^T V and the
//    update H_{c+1} = diag(E_last)(H_c + U), and, independent of those, the decay products,
//    Qh and Kh of chunk c+1 (lane = token, or two lanes per token with chunks of 32; wave =
//    group of SPW slots).
// Qh / Kh, the decay products, the alpha lists, the masks and the v tile are double-
// buffered; the buffer is a compile-time index (even / odd chunk of the segment), so the
// compiler can tell the direct global->LDS loads in flight from the other LDS accesses.
// v of chunk c+1 and the route of chunk c+2 are loaded directly into LDS at the start of
// phase Y(c); q and k of chunk c+2 come into registers right after chunk c+1 is prepared.
// ------------------------------------------------------------------------------------
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// row tile of the s-th lower-triangular tile (row-major order: (0,0), (1,0), (1,1), ...)
constexpr int tri_row(int s) {
    int r = 0;
    while ((r + 1) * (r + 2) / 2 <= s) ++r;
    return r;
}

// Waves per workgroup: 16 for pass B with M <= 64 (8 state waves and 8 decay-product waves,
// two of each per SIMD), else 8.
template <typename T, bool PASS_A, int M>
constexpr int scan_waves() { return (!PASS_A && M <= 64) ? 16 : 8; }
// Wave roles split (state waves / decay-product waves) in pass B: M <= 64 (16 waves), and
// bf16 M = 128 and 256 with chunks of 32 (8 waves: one of each kind per SIMD; 16 would not
// fit the state and its split operands in 128 registers per wave).
template <typename T, bool PASS_A, int M, int C>
constexpr bool scan_split() { return !PASS_A && (M <= 64 || (M >= 128 && C == 32 && sizeof(T) == 2)); }
// Alpha-list entries per token the LDS route buffers hold: K <= M up to 128 slots, K <= 32 at
// M = 256 (the host takes the token-by-token form beyond that).
template <int M>
constexpr int route_kcap() { return M <= 128 ? M : kRouteKCap256; }

// FUSE (pass A only, bf16 inputs, default router, K <= 16, one Dv tile per head): the pass routes the
// tokens itself -- each workgroup its own segment before the walk, and one extra workgroup
// per head (past the scan's grid) the last segment, which pass B alone reads -- in place of
// the separate router kernel; z, f and idx_out are the router's inputs and optional output.
// (rmask and ralpha carry no __restrict__: the fused pass writes the route through them.)
// DENSE (K = M with the default router: every slot selected every token): no route in memory;
// the decay-product waves form alpha = exp(sigmoid(z) f) from z and f themselves, loaded
// beside k (the router's formula, so the same alphas).
template <typename T, int M, int C, int DT, bool PASS_A, bool FUSE, bool DENSE = false>
__global__ __launch_bounds__((64 * scan_waves<T, PASS_A, M>())) void fwd_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ H0,
    long T_len, int Hh, int Dv, int K, SegArgs sg, const unsigned long long* rmask,
    const float* ralpha, float* __restrict__ o, float* __restrict__ H_out, const T* __restrict__ z,
    const float* __restrict__ f, int32_t* __restrict__ idx_out) {
    static_assert(!FUSE || PASS_A, "only the first pass routes");
    static_assert(!(FUSE && DENSE), "dense mode has no route");
    typedef Pol<T> P;
    typedef typename P::E E;
    typedef typename P::frag frag;
    typedef typename P::dfrag dfrag;
    constexpr int NW = scan_waves<T, PASS_A, M>(), NT = 64 * NW;
    constexpr int KB = P::KB, EPL = P::EPL, NPL = P::NPL;
    constexpr int MP = M > KB ? M : KB;        // padded slot dimension (k of slot contractions)
    constexpr int CP = C > KB ? C : KB;        // padded chunk dimension (k of row contractions)
    constexpr int EVE = 16 / int(sizeof(E));   // elements per 16 bytes
    constexpr int QP = MP + EVE;               // pitch of Qh / Kh rows
    constexpr int GV = DT * int(sizeof(T)) / 16;   // granules per row of the v tile
    constexpr int EPG = 16 / int(sizeof(T));       // input elements per granule
    constexpr int NTC = C / 16, NTD = DT / 16, NTM = M / 16, NTMP = MP / 16;
    constexpr int NKM = MP / KB, NKC = CP / KB;
    // Wave roles.  Pass B with M <= 64 (and bf16 M = 128): the first half of the waves own
    // the state columns (MFMA work), the second half compute the decay products; wave w runs
    // on SIMD w % 4, so each SIMD runs both kinds and their vector and matrix work overlap.
    // Otherwise every wave does both.
    constexpr bool SPLIT = scan_split<T, PASS_A, M, C>();
    constexpr int NMW = SPLIT ? NW / 2 : NW;         // state-column (MFMA) waves: 0 .. NMW-1
    constexpr int NPW = SPLIT ? NW / 2 : NW;         // decay-product waves: PW0 .. NW-1
    constexpr int PW0 = NW - NPW;
    constexpr int DPW = NTD > NMW ? NTD / NMW : 1;   // column tiles per MFMA wave
    constexpr int GT = NTD >= NMW ? 1 : NMW / NTD;   // MFMA waves per column tile
    constexpr int NTT = (NTC + GT - 1) / GT;         // output row tiles per MFMA wave, at most
    constexpr int SPW = M / NPW;                     // slots per decay-product wave
    // lanes per token in the decay-product pass: with chunks of 32 a token's SPW slots are
    // split between lanes t and t + 32 (every lane busy), else lane = token
    constexpr int LPT = (C == 32 && SPW >= 4) ? 2 : 1;
    constexpr int SPL = SPW / LPT;                   // slots per lane
    constexpr int MW = (M + 63) / 64;          // 64-bit words of a token's selection mask
    constexpr int NS = NTC * (NTC + 1) / 2;    // lower-triangular tiles of S^T
    constexpr int psQ = CP * QP + 8;           // plane stride of Qh / Kh
    constexpr int oK = NPL * psQ;              // Kh planes start here
    constexpr int SZQK = 2 * NPL * psQ;
    constexpr int psP = NTC * NKC * 64 * EPL;  // plane stride of the P^T fragments
    constexpr int NWD = SPL * int(sizeof(T)) / 4;  // 32-bit words of a lane's q (or k) piece
    static_assert((NMW % NTD == 0 || NTD % NMW == 0) && SPL >= 2 && SPL <= 32 && C <= 64 && NMW <= 8,
                  "tile split");
    constexpr int KCAP = route_kcap<M>();
    static_assert(2 * SZQK * int(sizeof(E)) >= 12 * C * M, "exact-path scratch");

    // LDS.  Every array is a separate object so the compiler can tell the direct loads from
    // the other accesses.  Route arrays are sized for K = KCAP.
    __shared__ __align__(16) T rv0[pad1k(CP * DT * int(sizeof(T))) / int(sizeof(T))];  // v, even chunks
    __shared__ __align__(16) T rv1[pad1k(CP * DT * int(sizeof(T))) / int(sizeof(T))];  // v, odd chunks
    __shared__ __align__(16) float rA0[pad1k(C * KCAP * 4) / 4];  // alpha lists, slot-major
    __shared__ __align__(16) float rA1[pad1k(C * KCAP * 4) / 4];
    __shared__ __align__(16) unsigned long long rM0[pad1k(C * MW * 8) / 8];  // selection masks
    __shared__ __align__(16) unsigned long long rM1[pad1k(C * MW * 8) / 8];
    __shared__ __align__(16) E sQK0[SZQK];  // Qh planes, then Kh planes
    __shared__ __align__(16) E sQK1[SZQK];
    __shared__ __align__(16) E sP[NPL * psP];  // P^T fragments
    __shared__ __align__(16) float sE0[M];     // decay products at the chunk end
    __shared__ __align__(16) float sE1[M];
    __shared__ int sF0[NW];                    // per wave: a decay product below the factored range
    __shared__ int sF1[NW];

    // workgroup -> (head, segment, Dv tile); consecutive ids (the Dv tiles of one head and
    // segment) land on the same XCD (workgroups are dealt to the 8 XCDs round-robin)
    const int nDT = Dv / DT;
    const int nseg = PASS_A ? sg.S - 1 : sg.S;
    long nblk = gridDim.x;
    // routing segment sgi of head bhr: one token per thread, rows past the sequence end skipped
    auto route_segment = [&](auto bhr, long sgi) {  // (generic: instantiated only where FUSE calls it)
        const long t_lo = sgi * sg.cps * C;
        const long t_end = (sgi + 1) * sg.cps * C;
        const long t_hi = t_end < T_len ? t_end : T_len;
        const long hb = bhr / Hh, hh = bhr % Hh;
        for (long t = t_lo + long(threadIdx.x); t < t_hi; t += 64 * NW)
            route_row<T, M, true, true>(z, f, (hb * T_len + t) * Hh + hh, bhr, t, sg.nC * C, K, C, idx_out, nullptr,
                                        const_cast<unsigned long long*>(rmask), const_cast<float*>(ralpha));
    };
    if constexpr (FUSE) {
        const long heads = nblk / (long(nseg) * nDT + 1);
        nblk -= heads;
        if (long(blockIdx.x) >= nblk) {  // route-only workgroup: the last segment of one head
            route_segment(long(blockIdx.x) - nblk, sg.S - 1);
            return;
        }
    }
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
    const bool mwave = w < NMW, pwave = w >= PW0;  // roles (both for every wave unless split)
    const int g = GT == 1 ? 0 : w / NTD;           // MFMA wave: token-tile group
    // column tile j of an MFMA wave
    auto Dj = [&](int j) { return GT == 1 ? w + NMW * j : w % NTD; };
    // decay-product lane: token tl of the chunk, slots s0 .. s0 + SPL - 1
    const int tl = LPT == 1 ? lane : (lane & (C - 1));
    const int s0 = (w - PW0) * SPW + (LPT == 1 ? 0 : (lane / C) * SPL);
    const long rstride = long(Hh);                  // rows between consecutive tokens of one head
    const long segrow = (bh * (sg.S - 1) + seg) * M;  // row of this segment in dH / dE
    auto valid_rows = [&](long c) { return int(T_len - c * C < C ? T_len - c * C : C); };

    // ---- direct loads of v (rows past the sequence end repeat the last row; their tokens
    // carry no route entries, so they contribute nothing) and of the route
    const long v_pitch = rstride * Dv * long(sizeof(T));
    // The direct loads are issued by the decay-product waves only (instruction r by wave
    // PW0 + r % NPW), right after their last read of the route buffer in a phase: the
    // compiler then never has a direct load in flight ahead of another wave's LDS reads.
    const int pw_i = w - PW0;
    TileDma<int(sizeof(rv0)), DT * int(sizeof(T)), NPW, 2> dv;
    dv.init(pw_i, lane, v_pitch);
    const T* vbase = v + (b * T_len * rstride + h) * Dv + d0;
    auto issue_v = [&](long c, T* dst) {
        dv.issue(dst, reinterpret_cast<const char*>(vbase + c * C * rstride * Dv), pw_i, lane, valid_rows(c), v_pitch);
    };
    const float* abase = ralpha + bh * T_pad * K;
    const unsigned long long* mbase = rmask + bh * T_pad * MW;
    auto issue_route = [&](long c, float* dA, unsigned long long* dM) {
        if constexpr (DENSE) return;
        const char* ab = reinterpret_cast<const char*>(abase + c * C * K);
        const char* mb = reinterpret_cast<const char*>(mbase + c * C * MW);
        const int na = C * K * 4, nm = C * MW * 8;
        dma_tile<NPW>(dA, pad1k(na), pw_i, lane, [&](int off) { return static_cast<const void*>(ab + min(off, na - 16)); });
        dma_tile<NPW>(dM, pad1k(nm), pw_i, lane,
                     [&](int off) { return static_cast<const void*>(mb + min(off, nm - 16)); });
    };

    // ---- q and k pieces of the decay-product pass: token tl, SPL slots from s0
    struct Seg {
        uint32_t wd[NWD];
        uint32_t zw[DENSE ? NWD : 1];  // dense mode, the k piece: the same slots of z, and f
        float f;
    };
    const T* qbase = q + (b * T_len * rstride + h) * M + s0;
    const T* kbase = k + (b * T_len * rstride + h) * M + s0;
    const T* zbase = z + (b * T_len * rstride + h) * M + s0;
    auto load_piece = [&](const T* src, Seg& s) {
        if constexpr (NWD % 4 == 0) {
#pragma unroll
            for (int p = 0; p < NWD / 4; ++p) {
                const uint4 u = reinterpret_cast<const uint4*>(src)[p];
                s.wd[4 * p] = u.x; s.wd[4 * p + 1] = u.y; s.wd[4 * p + 2] = u.z; s.wd[4 * p + 3] = u.w;
            }
        } else if constexpr (NWD == 2) {
            const uint2 u = *reinterpret_cast<const uint2*>(src);
            s.wd[0] = u.x; s.wd[1] = u.y;
        } else {
            s.wd[0] = *reinterpret_cast<const uint32_t*>(src);
        }
    };
    // (lanes past the chunk or the sequence get zeros; they load a valid row and select, so
    // the pieces are never assigned under a branch and stay in registers)
    // number of load instructions load_qk issues
    constexpr int NQK = (NWD % 4 == 0 ? NWD / 4 : 1) * (PASS_A ? 1 : 2) + (DENSE ? (NWD % 4 == 0 ? NWD / 4 : 1) + 1 : 0);
    auto load_qk = [&](long c, Seg& qs, Seg& ks) {
        // after every direct load of the phase: the waits for those skip these NQK loads
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        const long t = c * C + tl;
        const bool ok = tl < C && t < T_len;
        const long row = (ok ? t : 0) * rstride * M;
        Seg x, y, zz;
        load_piece(kbase + row, x);
        if (!PASS_A) load_piece(qbase + row, y);
        if constexpr (DENSE) {
            load_piece(zbase + row, zz);
            ks.f = f[(b * T_len + (ok ? t : 0)) * rstride + h];
        }
#pragma unroll
        for (int p = 0; p < NWD; ++p) {
            ks.wd[p] = ok ? x.wd[p] : 0u;
            qs.wd[p] = PASS_A ? 0u : ok ? y.wd[p] : 0u;
            if constexpr (DENSE) ks.zw[p] = zz.wd[p];
        }
    };
    auto unpack = [&](const Seg& s, float (&x)[SPL]) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int p = 0; p < NWD; ++p) {
                x[2 * p] = __uint_as_float(s.wd[p] << 16);
                x[2 * p + 1] = __uint_as_float(s.wd[p] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int p = 0; p < NWD; ++p) x[p] = __uint_as_float(s.wd[p]);
        }
    };

    // ---- the alphas of this lane's token for slots s0 .. s0+SPL-1: through the token's
    // selection mask (position in the alpha list = number of selected slots below); 1 for
    // unselected slots and for tokens past the sequence end.  A list position read for an
    // unselected slot may be past the list (stale LDS) and is discarded.
    auto gather = [&](const float* rA, const unsigned long long* rM, int nvalid, float (&al)[SPL]) {
        const int tc = tl < C ? tl : C - 1;
        // the mask word holding slots s0 .. s0+SPL-1 (SPL <= 32 slots never straddle two),
        // and the selected slots in the words below it
        const int wi = s0 >> 6;
        unsigned long long word = rM[tc * MW + wi];
        int base = __popcll(word & ((1ull << (s0 & 63)) - 1ull));
#pragma unroll
        for (int j = 0; j + 1 < MW; ++j) base += j < wi ? __popcll(rM[tc * MW + j]) : 0;
        if (tl >= nvalid) word = 0ull;
        const uint32_t gsel = uint32_t(word >> (s0 & 63));
        int idx = base;
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const bool sel = (gsel >> j) & 1u;
            const float a = rA[idx * C + tc];
            al[j] = sel ? a : 1.0f;
            idx += sel ? 1 : 0;
        }
    };

    // ---- dense mode: every slot's alpha from z and f of the lane's token (1 past the sequence)
    auto gather_dense = [&](const Seg& ks, int nvalid, float (&al)[SPL]) {
        float zf[SPL];
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int p = 0; p < NWD; ++p) {
                zf[2 * p] = __uint_as_float(ks.zw[p] << 16);
                zf[2 * p + 1] = __uint_as_float(ks.zw[p] & 0xFFFF0000u);
            }
        } else {
#pragma unroll
            for (int p = 0; p < NWD; ++p) zf[p] = __uint_as_float(ks.zw[p]);
        }
        const bool in = tl < nvalid;
#pragma unroll
        for (int j = 0; j < SPL; ++j) {
            const float sc = sigmoidf_dev(zf[j]);
            al[j] = (in && sc > 0.0f) ? __expf(sc * ks.f) : 1.0f;
        }
    };

    // ---- decay products, Qh = q o E and Kh = k (1 - alpha) / E (0 where alpha = 1) of
    // chunk c into buffer NB.  E is an inclusive product scan across the lanes of the clamped
    // alphas.  Also the per-slot E at the chunk end and the flag of a product that left the
    // factored range.
    // pre(): called first (direct loads into buffers prep does not read); mid(): called once
    // the route of chunk c has been read (the direct loads go there)
    auto prep = [&](auto nb, long c, const Seg& qs, const Seg& ks, float (&Ev)[SPL], auto&& pre, auto&& mid)
                    __attribute__((always_inline)) {
        constexpr int NB = decltype(nb)::value;
        E* sQK = NB ? sQK1 : sQK0;
        float al[SPL];
        // q / k of this chunk are in: no later use of them has to wait behind the direct
        // loads issued next
        wait_vm<0>();
        pre();
        if constexpr (DENSE) gather_dense(ks, valid_rows(c), al);
        else gather(NB ? rA1 : rA0, NB ? rM1 : rM0, valid_rows(c), al);
        mid();
#pragma unroll
        for (int j = 0; j < SPL; ++j) Ev[j] = clamp_alpha(al[j]);
        wave_scan_mul_n<SPL, LPT == 1>(Ev);
        if (LPT == 2 || C == 64 || lane < C) {
            float x[SPL];
            unpack(ks, x);
#pragma unroll
            for (int j = 0; j < SPL; ++j) x[j] = x[j] * (1.0f - clamp_alpha(al[j])) * __builtin_amdgcn_rcpf(Ev[j]);
            P::template put_row<SPL>(sQK, psQ, oK + tl * QP + s0, x);
            if (!PASS_A) {
                unpack(qs, x);
#pragma unroll
                for (int j = 0; j < SPL; ++j) x[j] *= Ev[j];
                P::template put_row<SPL>(sQK, psQ, tl * QP + s0, x);
            }
        }
    };
    // the last lane of each token group (lane 63; lanes 31 and 63 with two lanes per token)
    // holds the decay products at the chunk end: store them, and the wave's flag of one below
    // the factored range
    const bool tail_lane = LPT == 1 ? lane == 63 : tl == C - 1;
    auto prep_tail = [&](auto nb, const float (&Ev)[SPL]) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb)::value;
        int bad = 0;
#pragma unroll
        for (int j = 0; j < SPL; ++j) bad |= !(Ev[j] >= kSafeMin);
        const bool wbad = __builtin_amdgcn_ballot_w64(tail_lane && bad) != 0ull;
        if (tail_lane) Pol<float>::template put_row<SPL>(NB ? sE1 : sE0, 0, s0, Ev);
        if (lane == 63) (NB ? sF1 : sF0)[w] = wbad;
    };

    // ---- phase X: S^T tiles (J, TT), J <= TT, dealt to the state waves round-robin
    auto s_phase = [&](auto cur) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur)::value;
        const E* sQK = CUR ? sQK1 : sQK0;
        static_for<NS>([&](auto sc) {
            constexpr int S = decltype(sc)::value;
            constexpr int TT = tri_row(S), J = S - TT * (TT + 1) / 2;
            if (S % NMW == w) {
                // (with more than two k-blocks the fragments are loaded a pair of k-blocks at a
                // time, so the state waves' registers hold the state besides them)
                constexpr int KG = NKM > 2 ? 2 : NKM;
                floatx4 st = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k0 = 0; k0 < NKM; k0 += KG) {
                    dfrag a[KG], bq[KG];
#pragma unroll
                    for (int kk = 0; kk < KG; ++kk)
#pragma unroll
                        for (int pl = 0; pl < NPL; ++pl) {
                            const int kb = k0 + kk;
                            a[kk].p[pl] = P::ld(sQK, oK + pl * psQ + (16 * J + l16) * QP + kb * KB + EPL * q4);
                            bq[kk].p[pl] = P::ld(sQK, pl * psQ + (16 * TT + l16) * QP + kb * KB + EPL * q4);
                        }
#pragma unroll
                    for (int kk = 0; kk < KG; ++kk) st = P::mm_dd(a[kk], bq[kk], st);
                }
                if (J == TT) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (4 * q4 + r > l16) st[r] = 0.0f;  // j > t
                }
                P::template put_pfrag<NKC>(sP, psP, TT, J, lane, st);
            }
        });
    };

    // ---- the state: Hreg[I][r] = H[16*I + 4*q4 + r][d0 + 16*D + l16]; slot tiles past M
    // (padding of the k-blocks) stay zero.  Pass B starts from H0 (or zero) and folds in the
    // segments before its own; pass A starts from zero.
    floatx4 Hreg[DPW][NTMP];
#pragma unroll
    for (int j = 0; j < DPW; ++j)
#pragma unroll
        for (int I = 0; I < NTMP; ++I) Hreg[j][I] = floatx4{0.f, 0.f, 0.f, 0.f};
    float Eseg = 1.0f;  // pass A: decay product over the segment of slot tid (tid < M)

    // LDS padding (slot columns past M, chunk rows past C, P^T fragments above the diagonal)
    // stays zero; everything else of Qh / Kh is written before it is read
    auto zero16 = [&](void* arr, int nbytes) {
        for (int i = tid; i < nbytes / 16; i += NT) reinterpret_cast<uint4*>(arr)[i] = make_uint4(0u, 0u, 0u, 0u);
    };
    auto zero_qk = [&]() {
        zero16(sQK0, int(sizeof(sQK0)));
        zero16(sQK1, int(sizeof(sQK1)));
    };

    // ---- phase Y, factored path: output tiles, U, state update
    auto y_phase = [&](auto cur, auto gc, long c, int nvalid) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur)::value, G = decltype(gc)::value;
        const E* sQK = CUR ? sQK1 : sQK0;
        const T* rvc = CUR ? rv1 : rv0;
        const float* sE = CUR ? sE1 : sE0;
        frag va[DPW][NKC];  // V^T rows of the column tiles (k = chunk rows in the order jperm)
#pragma unroll
        for (int j = 0; j < DPW; ++j)
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
                va[j][kb] = P::template ld_col_swz<true, GV, 2>(rvc, 0, 16 * Dj(j), kb, q4, l16);
        // more than four k-blocks of slots (M = 256): k-block outer, the state split one
        // k-block at a time and applied to every output row tile (few live registers, the
        // accumulators of the row tiles independent)
        constexpr bool KOUTER = NKM > 4;
        if constexpr (!PASS_A && KOUTER) {
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                o + ((b * T_len + c * C) * rstride + h) * Dv + d0, short(0), kOutRange, kBufferFlags);
            floatx4 acc[NTT][DPW];
            static_for<NTT>([&](auto nc) {
                constexpr int N = decltype(nc)::value, TT = G + GT * N;
#pragma unroll
                for (int j = 0; j < DPW; ++j) acc[N][j] = floatx4{0.f, 0.f, 0.f, 0.f};
                if constexpr (TT < NTC) {
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        if (kb * KB < 16 * (TT + 1)) {
                            const dfrag pf = P::template ld_pfrag<NKC>(sP, psP, TT, kb, lane);
#pragma unroll
                            for (int j = 0; j < DPW; ++j) acc[N][j] = P::mm_vd(va[j][kb], pf, acc[N][j]);
                        }
                }
            });
#pragma unroll
            for (int kb = 0; kb < NKM; ++kb) {
                dfrag hk[DPW];
#pragma unroll
                for (int j = 0; j < DPW; ++j) hk[j] = P::pack_perm(Hreg[j], kb);
                static_for<NTT>([&](auto nc) {
                    constexpr int N = decltype(nc)::value, TT = G + GT * N;
                    if constexpr (TT < NTC) {
                        dfrag qk;
#pragma unroll
                        for (int pl = 0; pl < NPL; ++pl)
                            qk.p[pl] = P::ld_jrow(sQK, pl * psQ + (16 * TT + l16) * QP, kb, q4);
#pragma unroll
                        for (int j = 0; j < DPW; ++j) acc[N][j] = P::mm_dd(hk[j], qk, acc[N][j]);
                    }
                });
            }
            static_for<NTT>([&](auto nc) {
                constexpr int N = decltype(nc)::value, TT = G + GT * N;
                if constexpr (TT < NTC) {
                    const int tl = 16 * TT + l16;
#pragma unroll
                    for (int j = 0; j < DPW; ++j) {
                        const int off =
                            tl < nvalid ? int((tl * rstride * Dv + 16 * Dj(j) + 4 * q4) * 4) : kOutRange + 16;
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint32x4, acc[N][j]), orsrc, off, 0,
                                                               0);
                    }
                }
            });
        }
        if (!PASS_A && !KOUTER) {
            // the state as hi / lo MFMA operands: split once when the wave has several output
            // row tiles, else at its use, one k-block at a time (fewer live registers)
            constexpr bool HPRE = NTT > 1;
            dfrag hf[HPRE ? DPW : 1][HPRE ? NKM : 1];
            if constexpr (HPRE) {
#pragma unroll
                for (int j = 0; j < DPW; ++j)
#pragma unroll
                    for (int kb = 0; kb < NKM; ++kb) hf[j][kb] = P::pack_perm(Hreg[j], kb);
            }
            // outputs go out by buffer stores whose offset is out of range for rows past the
            // sequence end (dropped by the hardware), so no branch splits this block
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                o + ((b * T_len + c * C) * rstride + h) * Dv + d0, short(0), kOutRange, kBufferFlags);
            static_for<NTT>([&](auto nc) {
                constexpr int N = decltype(nc)::value, TT = G + GT * N;
                if constexpr (TT < NTC) {
                    dfrag qf[NKM], pf[NKC];  // shared by the wave's column tiles
                    auto load_qf = [&](int kb) __attribute__((always_inline)) {
#pragma unroll
                        for (int pl = 0; pl < NPL; ++pl)
                            qf[kb].p[pl] = P::ld_jrow(sQK, pl * psQ + (16 * TT + l16) * QP, kb, q4);
                    };
                    if constexpr (HPRE) {
#pragma unroll
                        for (int kb = 0; kb < NKM; ++kb) load_qf(kb);
                    }
#pragma unroll
                    for (int kb = 0; kb < NKC; ++kb)
                        if (kb * KB < 16 * (TT + 1)) pf[kb] = P::template ld_pfrag<NKC>(sP, psP, TT, kb, lane);
                    const int tl = 16 * TT + l16;
#pragma unroll
                    for (int j = 0; j < DPW; ++j) {
                        floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kb = 0; kb < NKC; ++kb)
                            if (kb * KB < 16 * (TT + 1)) acc = P::mm_vd(va[j][kb], pf[kb], acc);
#pragma unroll
                        for (int kb = 0; kb < NKM; ++kb) {
                            if constexpr (HPRE) {
                                acc = P::mm_dd(hf[j][kb], qf[kb], acc);
                            } else {
                                if (j == 0) load_qf(kb);
                                acc = P::mm_dd(P::pack_perm(Hreg[j], kb), qf[kb], acc);
                            }
                        }
                        const int off =
                            tl < nvalid ? int((tl * rstride * Dv + 16 * Dj(j) + 4 * q4) * 4) : kOutRange + 16;
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint32x4, acc), orsrc, off, 0, 0);
                    }
                }
            });
        }
        static_for<NTM>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            dfrag kf[NKC];  // shared by the wave's column tiles
#pragma unroll
            for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
                for (int pl = 0; pl < NPL; ++pl)
                    kf[kb].p[pl] = P::template ld_col<true>(sQK, oK + pl * psQ + 16 * I, QP, kb, q4, l16);
            const float4 e4 = *reinterpret_cast<const float4*>(sE + (16 * I + 4 * q4));
            const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
            for (int j = 0; j < DPW; ++j) {
                floatx4 u = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) u = P::mm_dv(kf[kb], va[j][kb], u);
#pragma unroll
                for (int r = 0; r < 4; ++r)  // rows of slots untouched in the chunk (E = 1) keep their bits
                    Hreg[j][I][r] = ev[r] < 1.0f ? ev[r] * (Hreg[j][I][r] + u[r]) : Hreg[j][I][r];
            }
            // (M = 256: two slot tiles at a time, so the loads of the others are not hoisted
            // into the registers the state already fills)
            if constexpr (NTM > 8 && I % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- phase Y, exact path of a chunk whose decay product left the factored range:
    // token-by-token recurrence on the register state with the exact alphas.  Dense fp32
    // alpha [C][M] and q [C][M] go into one Qh/Kh buffer, k [C][M] into the other (neither
    // is in use: this chunk's Qh / Kh are invalid and chunk c+1 is prepared afterwards).
    auto exact = [&](auto cur, long c, int nvalid, auto dm, auto dp) __attribute__((always_inline)) {
        constexpr bool DM = decltype(dm)::value, DP = decltype(dp)::value;
        constexpr int CUR = decltype(cur)::value;
        float* xa = reinterpret_cast<float*>(CUR ? sQK1 : sQK0);
        float* xk = reinterpret_cast<float*>(CUR ? sQK0 : sQK1);
        float* sE = CUR ? sE1 : sE0;
        const T* rvc = CUR ? rv1 : rv0;
        if constexpr (DP) {
            float al[SPL], x[SPL];
            Seg qs2, ks2;
            if constexpr (DENSE) {
                load_qk(c, qs2, ks2);
                wait_vm<0>();
                gather_dense(ks2, nvalid, al);
            } else {
                gather(CUR ? rA1 : rA0, CUR ? rM1 : rM0, nvalid, al);
                load_qk(c, qs2, ks2);
            }
            if (LPT == 2 || C == 64 || lane < C) {
                Pol<float>::template put_row<SPL>(xa, 0, tl * M + s0, al);
                unpack(ks2, x);
                Pol<float>::template put_row<SPL>(xk, 0, tl * M + s0, x);
                if (!PASS_A) {
                    unpack(qs2, x);
                    Pol<float>::template put_row<SPL>(xa, 0, C * M + tl * M + s0, x);
                }
            }
#pragma unroll
            for (int j = 0; j < SPL; ++j) x[j] = al[j];
            wave_scan_mul_n<SPL, LPT == 1>(x);  // exact decay products
            if (tail_lane) Pol<float>::template put_row<SPL>(sE, 0, s0, x);
        }
        wg_barrier();
        if constexpr (DM) {
            for (int tt = 0; tt < nvalid; ++tt) {
#pragma unroll
                for (int j = 0; j < DPW; ++j) {
                    const float vd = Elem<T>::load(rvc, swz_elem<GV, 2, EPG>(tt, 16 * Dj(j) + l16));
                    float part = 0.0f;
#pragma unroll
                    for (int I = 0; I < NTM; ++I) {
                        const int i0 = tt * M + 16 * I + 4 * q4;
                        const float4 a4 = *reinterpret_cast<const float4*>(xa + i0);
                        const float4 k4 = *reinterpret_cast<const float4*>(xk + i0);
                        const float av[4] = {a4.x, a4.y, a4.z, a4.w}, kv[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
                        for (int r = 0; r < 4; ++r) {  // a select, not a conditional store: Hreg stays in registers
                            const float hn = fmaf(av[r], Hreg[j][I][r], (1.0f - av[r]) * kv[r] * vd);
                            Hreg[j][I][r] = av[r] != 1.0f ? hn : Hreg[j][I][r];
                        }
                        if (!PASS_A) {
                            const float4 x4 = *reinterpret_cast<const float4*>(xa + (C * M + i0));
                            part = fmaf(x4.x, Hreg[j][I][0], part);
                            part = fmaf(x4.y, Hreg[j][I][1], part);
                            part = fmaf(x4.z, Hreg[j][I][2], part);
                            part = fmaf(x4.w, Hreg[j][I][3], part);
                        }
                        // a slot tile at a time: the loads of the next are not hoisted above
                        // this one (the wave's registers are mostly state)
                        if constexpr (NTM > 4) __builtin_amdgcn_sched_barrier(0);
                    }
                    if (!PASS_A) {
                        part += __shfl_xor(part, 16);
                        part += __shfl_xor(part, 32);
                        if (g == 0 && q4 == 0)
                            o[((b * T_len + c * C + tt) * rstride + h) * Dv + d0 + 16 * Dj(j) + l16] = part;
                    }
                }
            }
        }
        wg_barrier();  // the dense copies are read; the exact sE is written
    };

    // ---- one chunk c with buffer CUR (CUR = chunk parity within the segment).  The q / k
    // pieces of chunk c+1 are in (qc, kc); those of chunk c+2 are loaded into the other pair
    // at the start of phase Y.
    Seg qA, kA, qB, kB;
    auto chunk = [&](auto cur, long c, auto dm, auto dp) __attribute__((always_inline)) {
        constexpr int CUR = decltype(cur)::value, NXT = CUR ^ 1;
        constexpr bool DM = decltype(dm)::value, DP = decltype(dp)::value;
        const int nvalid = valid_rows(c);
        Seg& qc = CUR ? qB : qA;
        Seg& kc = CUR ? kB : kA;
        Seg& qn = CUR ? qA : qB;
        Seg& kn = CUR ? kA : kB;
        // pass B: the decay-product waves' direct loads (v of chunk c, the route of c+1) have
        // landed before they read LDS; the q / k loads of chunk c+2, issued last, may still be
        // in flight.  (Pass A waits at the end of the previous chunk.)
        if constexpr (DP && !PASS_A) wait_vm<NQK>();
        const int* sF = CUR ? sF1 : sF0;
        int unsafe = 0;
#pragma unroll
        for (int i = PW0; i < NW; ++i) unsafe |= sF[i];
        unsafe = __builtin_amdgcn_readfirstlane(unsafe);
        if (!PASS_A) {
            // (the state waves: the decay-product waves' LDS reads here would wait for their
            // own q / k loads of chunk c+2)
            if constexpr (DM)
                if (!unsafe) s_phase(cur);
            wg_barrier();
        }
        // direct loads of v of chunk c+1 (its buffer was last read in the previous chunk) and
        // of the route of chunk c+2 (into the buffer chunk c's route was read from)
        auto issue_v_next = [&]() {
            if (c + 1 < c_end) issue_v(c + 1, NXT ? rv1 : rv0);
        };
        auto issue_route_next = [&]() {
            if (c + 2 < c_end) issue_route(c + 2, CUR ? rA1 : rA0, CUR ? rM1 : rM0);
        };
        float Ev[SPL];
        if (unsafe) {
            exact(cur, c, nvalid, dm, dp);
            if (MP > M || CP > C) {
                zero_qk();
                wg_barrier();
            }
        } else if constexpr (DM) {
            // output tiles, U and the state update
            if constexpr (GT == 1) {
                y_phase(cur, std::integral_constant<int, 0>{}, c, nvalid);
            } else {
                switch (g) {
                    case 0: y_phase(cur, std::integral_constant<int, 0>{}, c, nvalid); break;
                    case 1: y_phase(cur, std::integral_constant<int, 1>{}, c, nvalid); break;
                    case 2: if constexpr (GT > 2) y_phase(cur, std::integral_constant<int, 2>{}, c, nvalid); break;
                    case 3: if constexpr (GT > 3) y_phase(cur, std::integral_constant<int, 3>{}, c, nvalid); break;
                    case 4: if constexpr (GT > 4) y_phase(cur, std::integral_constant<int, 4>{}, c, nvalid); break;
                    case 5: if constexpr (GT > 5) y_phase(cur, std::integral_constant<int, 5>{}, c, nvalid); break;
                    case 6: if constexpr (GT > 6) y_phase(cur, std::integral_constant<int, 6>{}, c, nvalid); break;
                    case 7: if constexpr (GT > 7) y_phase(cur, std::integral_constant<int, 7>{}, c, nvalid); break;
                }
            }
        }
        // decay products and Qh / Kh of chunk c+1, then q / k of chunk c+2 into registers
        if constexpr (DP) {
            prep(std::integral_constant<int, NXT>{}, c + 1, qc, kc, Ev, issue_v_next, issue_route_next);
            load_qk(c + 2, qn, kn);
            prep_tail(std::integral_constant<int, NXT>{}, Ev);
        }
        if (PASS_A && tid < M) Eseg *= (CUR ? sE1 : sE0)[tid];
        if (PASS_A) wait_vm<NQK>();  // v of chunk c+1 and the route of c+2 have landed
        wg_barrier();
    };

    // ---- the whole walk for one role (or both): the two roles run the same sequence of
    // barriers; with separate copies of the loop each keeps only its own values live
    auto run = [&](auto dm, auto dp) __attribute__((always_inline)) {
        constexpr bool DM = decltype(dm)::value, DP = decltype(dp)::value;
        // ---- prologue: route, q, k and v of the first chunk in flight while the start state is
        // loaded and LDS is cleared; then the decay products and Qh / Kh of the first chunk
        if (DP && c_begin < c_end) {
            issue_route(c_begin, rA0, rM0);
            issue_v(c_begin, rv0);
            load_qk(c_begin, qB, kB);
            if (c_begin + 1 < c_end) issue_route(c_begin + 1, rA1, rM1);
            load_qk(c_begin + 1, qA, kA);
        }
        auto load_start = [&]() __attribute__((always_inline)) {
            // Segment 0 starts from H0 (or zero).  Segment s > 0 starts from the state the
            // segments before it leave: with more than kFoldMax + 1 segments it was folded in
            // place of dH_{s-1} between the two passes; otherwise it is folded here, every
            // segment's (E, dH) loaded at once.
            auto at = [&](int j, int I, int r) { return (16 * I + 4 * q4 + r) * Dv + d0 + 16 * Dj(j) + l16; };
            // (M = 256: always folded by the fold kernel; the in-kernel fold's loads would not
            // fit beside the state)
            constexpr bool kFoldHere = M <= 128;
            const bool folded = sg.S > kFoldMax + 1 || !kFoldHere;
            const float* hs = (seg > 0 && folded) ? sg.dH + (bh * (sg.S - 1) + seg - 1) * M * Dv
                                                  : H0 ? H0 + bh * M * Dv : nullptr;
            if (hs) {
#pragma unroll
                for (int j = 0; j < DPW; ++j)
#pragma unroll
                    for (int I = 0; I < NTM; ++I)
#pragma unroll
                        for (int r = 0; r < 4; ++r) Hreg[j][I][r] = hs[at(j, I, r)];
            }
            // segments per batch of loads: all of them if their (E, dH) values fit in about 144
            // registers, else one at a time
            constexpr int FB = NTM * (1 + DPW) * 4 * kFoldMax <= (NW > 8 ? 64 : 144) ? kFoldMax : 1;
            // (with one segment per batch, one slot tile at a time, the scheduler kept from
            // hoisting the loads of the next: a wave whose registers are mostly state)
            constexpr bool TILEWISE = FB == 1 && NTM > 4;
            for (int s0 = 0; kFoldHere && seg > 0 && !folded && s0 < seg; s0 += FB) {
                if constexpr (TILEWISE) {
                    const long sr = (bh * (sg.S - 1) + s0) * M;
                    static_for<NTM>([&](auto ic) {
                        constexpr int I = decltype(ic)::value;
                        float ev[4], xv[DPW][4];
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            ev[r] = sg.dE[sr + 16 * I + 4 * q4 + r];
#pragma unroll
                            for (int j = 0; j < DPW; ++j) xv[j][r] = sg.dH[sr * Dv + at(j, I, r)];
                        }
#pragma unroll
                        for (int j = 0; j < DPW; ++j)
#pragma unroll
                            for (int r = 0; r < 4; ++r)  // untouched rows keep their bits
                                Hreg[j][I][r] = ev[r] != 1.0f ? fmaf(ev[r], Hreg[j][I][r], xv[j][r]) : Hreg[j][I][r];
                        __builtin_amdgcn_sched_barrier(0);
                    });
                    continue;
                }
                float ev[FB][NTM][4], xv[FB][DPW][NTM][4];
#pragma unroll
                for (int sj = 0; sj < FB; ++sj) {
                    const long sr = (bh * (sg.S - 1) + (s0 + sj < seg ? s0 + sj : 0)) * M;  // a valid segment
#pragma unroll
                    for (int I = 0; I < NTM; ++I)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            ev[sj][I][r] = sg.dE[sr + 16 * I + 4 * q4 + r];
#pragma unroll
                            for (int j = 0; j < DPW; ++j) xv[sj][j][I][r] = sg.dH[sr * Dv + at(j, I, r)];
                        }
                }
#pragma unroll
                for (int sj = 0; sj < FB; ++sj)
#pragma unroll
                    for (int j = 0; j < DPW; ++j)
#pragma unroll
                        for (int I = 0; I < NTM; ++I)
#pragma unroll
                            for (int r = 0; r < 4; ++r) {  // untouched rows keep their bits
                                const float e = ev[sj][I][r];
                                const bool use = s0 + sj < seg && e != 1.0f;
                                Hreg[j][I][r] = use ? fmaf(e, Hreg[j][I][r], xv[sj][j][I][r]) : Hreg[j][I][r];
                            }
            }
        };
        // With split roles the state waves load and fold their start state while the
        // decay-product waves prepare the first chunk (its latency, a round trip per earlier
        // segment, then overlaps that work); otherwise it comes first.
        const bool late = SPLIT && c_begin < c_end;
        if (DM && !PASS_A && !late) load_start();
        if (MP > M || CP > C) zero_qk();
        if (!PASS_A) zero16(sP, int(sizeof(sP)));
        if (c_begin < c_end) {
            __builtin_amdgcn_s_waitcnt(0);
            wg_barrier();  // the loads and the zero fill are done
            if constexpr (DP) {
                float Ev[SPL];
                prep(std::integral_constant<int, 0>{}, c_begin, qB, kB, Ev, [] {}, [] {});
                prep_tail(std::integral_constant<int, 0>{}, Ev);
            }
            if (DM && !PASS_A && late) load_start();
            wg_barrier();
        }
        for (long c = c_begin; c < c_end; c += 2) {
            chunk(std::integral_constant<int, 0>{}, c, dm, dp);
            if (c + 1 < c_end) chunk(std::integral_constant<int, 1>{}, c + 1, dm, dp);
        }

        if (DM && g == 0 && (PASS_A || (H_out && seg == sg.S - 1))) {
            float* dst = PASS_A ? sg.dH + segrow * Dv : H_out + bh * M * Dv;
#pragma unroll
            for (int j = 0; j < DPW; ++j)
#pragma unroll
                for (int I = 0; I < NTM; ++I)
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[(16 * I + 4 * q4 + r) * Dv + d0 + 16 * Dj(j) + l16] = Hreg[j][I][r];
        }
    };
    if constexpr (FUSE) {
        // this segment's route, written before the walk's direct loads read it: each wave's
        // stores acknowledged (vmcnt 0), then the barrier.  Within one workgroup that is
        // enough: the vector L1 is write-through and holds none of these lines yet (an
        // agent-scope fence would also write back the L2, once per workgroup).
        route_segment(bh, seg);
        wait_vm<0>();
        __syncthreads();
    }
    if constexpr (SPLIT) {
        if (mwave) run(std::true_type{}, std::false_type{});
        else run(std::false_type{}, std::true_type{});
    } else {
        run(std::true_type{}, std::true_type{});
    }
    if (PASS_A && dtile == 0 && tid < M) sg.dE[segrow + tid] = Eseg;
}

}  // namespace rsm

#include "rsm_segstate.h"

namespace rsm {

template <typename T, int M, int C, int DT>
static int launch_scan(const T* q, const T* k, const T* v, const float* H0, long B, long T_len, long Hh, int Dv,
                       int K, const SegArgs& sg, const unsigned long long* rmask, const float* ralpha, float* o,
                       float* H_out, const void* zr, const float* f, int32_t* idx_out, bool fuse, bool dense,
                       hipStream_t s) {
    const long tiles = B * Hh * (Dv / DT);
    const T* z = static_cast<const T*>(zr);
    // every slot every token (K = M, default router; bf16 at M = 128, the dense case of the
    // router-limit sweep): both passes form the alphas from z and f, nothing routed
    if constexpr (M == 128 && std::is_same<T, bf16_t>::value) {
        if (dense) {
            if (sg.S > 1) {
                if (C >= 32 && Dv == DT)  // the segment-state pass, its alphas from z and f
                    hipLaunchKernelGGL((seg_state_kernel<M, C >= 32 ? C : 32, DT, false, true>),
                                       dim3(unsigned(B * Hh * (sg.S - 1))), dim3(512), 0, s, k, v, z, f, T_len,
                                       int(Hh), Dv, K, sg, const_cast<unsigned long long*>(rmask),
                                       const_cast<float*>(ralpha), idx_out);
                else
                    hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, true, false, true>),
                                       dim3(unsigned(tiles * (sg.S - 1))), dim3(64 * scan_waves<T, true, M>()), 0, s, q,
                                       k, v, H0, T_len, int(Hh), Dv, K, sg, rmask, ralpha, o, H_out, z, f, idx_out);
                if (hipGetLastError() != hipSuccess) return RSM_ERR_HIP;
                if (sg.S > kFoldMax + 1 || M > 128) {
                    const int st = seg_fold_launch(H0, sg, B * Hh, M, Dv, s);
                    if (st != RSM_OK) return st;
                }
            }
            hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, false, false, true>), dim3(unsigned(tiles * sg.S)),
                               dim3(64 * scan_waves<T, false, M>()), 0, s, q, k, v, H0, T_len, int(Hh), Dv, K, sg, rmask,
                               ralpha, o, H_out, z, f, idx_out);
            return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
        }
    }
    if (dense) return RSM_ERR_UNSUPPORTED;
    if (sg.S > 1) {
        bool routed = false;
        if constexpr (std::is_same<T, bf16_t>::value && M <= 128) {  // fp32 rows would spill in the pass
            if constexpr (C >= 32) {
                if (fuse) {  // segment states by the backward walk, which routes: one more workgroup
                             // per head routes the last segment
                    // M = 128, a segment that fits one routing round: the variant without mid-walk
                    // rounds (whose routing beside the walk's live registers spills there; at M <= 64
                    // it measured slower than the round-by-round kernel)
                    if (M >= 128 && long(sg.cps) * C <= seg_round_one<M, C, DT>())
                        hipLaunchKernelGGL((seg_state_kernel<M, C, DT, true>), dim3(unsigned(B * Hh * sg.S)), dim3(512),
                                           0, s, reinterpret_cast<const bf16_t*>(k), reinterpret_cast<const bf16_t*>(v),
                                           reinterpret_cast<const bf16_t*>(z), f, T_len, int(Hh), Dv, K, sg,
                                           const_cast<unsigned long long*>(rmask), const_cast<float*>(ralpha), idx_out);
                    else
                        hipLaunchKernelGGL((seg_state_kernel<M, C, DT, false>), dim3(unsigned(B * Hh * sg.S)),
                                           dim3(512), 0, s, reinterpret_cast<const bf16_t*>(k),
                                           reinterpret_cast<const bf16_t*>(v), reinterpret_cast<const bf16_t*>(z), f,
                                           T_len, int(Hh), Dv, K, sg, const_cast<unsigned long long*>(rmask),
                                           const_cast<float*>(ralpha), idx_out);
                    routed = true;
                }
            }
            if (fuse && !routed) {  // pass A routes: one more workgroup per head for the last segment
                hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, true, true>),
                                   dim3(unsigned(tiles * (sg.S - 1) + B * Hh)), dim3(64 * scan_waves<T, true, M>()), 0,
                                   s, q, k, v, H0, T_len, int(Hh), Dv, K, sg, rmask, ralpha, o, H_out, z, f, idx_out);
                routed = true;
            }
        }
        if (!routed)
            hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, true, false>), dim3(unsigned(tiles * (sg.S - 1))),
                               dim3(64 * scan_waves<T, true, M>()), 0, s,
                               q, k, v, H0, T_len, int(Hh), Dv, K, sg, rmask, ralpha, o, H_out, z, f, idx_out);
        if (hipGetLastError() != hipSuccess) return RSM_ERR_HIP;
        if (sg.S > kFoldMax + 1 || M > 128) {
            const int st = seg_fold_launch(H0, sg, B * Hh, M, Dv, s);
            if (st != RSM_OK) return st;
        }
    }
    hipLaunchKernelGGL((fwd_scan_kernel<T, M, C, DT, false, false>), dim3(unsigned(tiles * sg.S)),
                       dim3(64 * scan_waves<T, false, M>()), 0, s, q, k, v,
                       H0, T_len, int(Hh), Dv, K, sg, rmask, ralpha, o, H_out, z, f, idx_out);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}


template <typename T, int M, int C>
static int dispatch_dt(int DT, const ScanArgs& a) {
    const T *q = static_cast<const T*>(a.q), *k = static_cast<const T*>(a.k), *v = static_cast<const T*>(a.v);
#define RSM_SCAN(DTV) \
    return launch_scan<T, M, C, DTV>(q, k, v, a.H0, a.B, a.T_len, a.Hh, a.Dv, a.K, a.sg, a.rmask, a.ralpha, a.o, \
                                     a.H_out, a.z, a.f, a.idx_out, a.fuse_route, a.dense, a.s)
    constexpr int cap = (sizeof(T) == 4 ? 64 : 128) / (M >= 128 ? 2 : 1);  // (M = 256: 64, bf16 only)
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
    if constexpr (M == 256) {  // bf16, chunks of 32 only
        return C == 32 ? dispatch_dt<T, M, 32>(DT, a) : RSM_ERR_UNSUPPORTED;
    } else {
        switch (C) {
            case 16: return dispatch_dt<T, M, 16>(DT, a);
            case 32: return dispatch_dt<T, M, 32>(DT, a);
            case 64:
                if constexpr (M < 128) return dispatch_dt<T, M, 64>(DT, a);
                break;
        }
        return RSM_ERR_UNSUPPORTED;
    }
}

}  // namespace rsm
