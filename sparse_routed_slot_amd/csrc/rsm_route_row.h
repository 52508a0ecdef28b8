// rsm_route_row.h -- the per-row router (sigmoid scores, exact top-K with ties to the lower
// slot) as device code: used by the router kernels and by the chunked forward's first pass.
//
// RSM router of Raven (README page, "How Raven Works": TopK(sigmoid(r_proj(x))) and
// decay = exp(route_scores * f)), taking the projected logits z as input.
#pragma once

#include <type_traits>

#include "rsm_device.h"

namespace rsm {

// ------------------------------------------------------------------------------------
// Packed top-K for bf16 rows (K <= 16, M >= 32).  A row is held as M/2 registers of two
// logits (slots 2r, 2r+1).  Each logit gets a 16-bit order key, positive x -> x + 0x7FFF,
// negative x -> 0xFFFF - x: strictly increasing in the value, with -0 and +0 equal, so it
// ranks the slots exactly as the packed 32-bit keys of RowKey do, minus the slot index.
// The K-th largest key T (with multiplicity) comes from a bitonic network on packed 16-bit
// min / max, two groups of 16 keys (even and odd slots of 32) per register set; then slot
// i is selected iff key_i > T, or key_i == T and it is among the lowest-index slots with
// key T needed to make K (ties to the lower index).
// ------------------------------------------------------------------------------------
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 pair_keys(uint32_t raw) {
    const u16x2 x = __builtin_bit_cast(u16x2, raw);
    const u16x2 s = __builtin_bit_cast(u16x2, __builtin_bit_cast(i16x2, x) >> (i16x2){15, 15});
    return (x ^ s) + (~s & (u16x2){0x7FFF, 0x7FFF});
}

// descending bitonic sort of the 16 keys in each half of v[0..15]
__device__ __forceinline__ void pk_sort16_desc(u16x2 (&v)[16]) {
#pragma unroll
    for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const u16x2 hi = __builtin_elementwise_max(v[i], v[l]), lo = __builtin_elementwise_min(v[i], v[l]);
                    const bool desc = k == 16 || (i & k) == 0;
                    v[i] = desc ? hi : lo;
                    v[l] = desc ? lo : hi;
                }
            }
}

// descending bitonic merge of the bitonic 16-key sequence in each half of v[0..15]
__device__ __forceinline__ void pk_merge16_desc(u16x2 (&v)[16]) {
#pragma unroll
    for (int j = 8; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) {
                const u16x2 hi = __builtin_elementwise_max(v[i], v[l]), lo = __builtin_elementwise_min(v[i], v[l]);
                v[i] = hi;
                v[l] = lo;
            }
        }
}

// Two sorted 16-key lists per half (a: halves of x, b: halves of y) -> per half the sorted
// top 16 of the union of x's two lists (low half) and of y's two lists (high half): the
// element-wise maximum of one list and the other reversed is bitonic and holds the top 16.
__device__ __forceinline__ void pk_combine(const u16x2 (&x)[16], const u16x2 (&y)[16], u16x2 (&out)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
        out[i] = __builtin_elementwise_max(__builtin_shufflevector(x[i], y[i], 0, 2),
                                           __builtin_shufflevector(x[15 - i], y[15 - i], 1, 3));
    pk_merge16_desc(out);
}

// flags (key >= tv) of the M/2 key registers as selection bit masks (bit i of word i/64)
template <int M>
__device__ __forceinline__ void pk_mask_ge(const u16x2 (&key)[M / 2], unsigned short tv, unsigned long long (&mk)[(M + 63) / 64]) {
    uint32_t acc[M / 32];  // per 32 slots: bit k = slot 2k (low half), bit 16 + k = slot 2k + 1
#pragma unroll
    for (int b = 0; b < M / 32; ++b) acc[b] = 0u;
    if (tv == 0) {
#pragma unroll
        for (int b = 0; b < M / 32; ++b) acc[b] = 0xFFFFFFFFu;
    } else {
        const u16x2 t1 = {static_cast<unsigned short>(tv - 1), static_cast<unsigned short>(tv - 1)};
#pragma unroll
        for (int r = 0; r < M / 2; ++r) {
            // key > tv - 1: the saturated difference is >= 1, so adding 0x7FFF sets bit 15
            const u16x2 v = __builtin_elementwise_add_sat(__builtin_elementwise_sub_sat(key[r], t1),
                                                          (u16x2){0x7FFF, 0x7FFF});
            acc[r / 16] |= (__builtin_bit_cast(uint32_t, v) & 0x80008000u) >> (15 - r % 16);
        }
    }
    auto spread = [](uint32_t x) {  // bit k -> bit 2k, for k < 16
        x = (x | (x << 8)) & 0x00FF00FFu;
        x = (x | (x << 4)) & 0x0F0F0F0Fu;
        x = (x | (x << 2)) & 0x33333333u;
        return (x | (x << 1)) & 0x55555555u;
    };
#pragma unroll
    for (int w = 0; w < (M + 63) / 64; ++w) {
        unsigned long long m = 0ull;
#pragma unroll
        for (int h = 0; h < 2 && 64 * w + 32 * h < M; ++h) {
            const uint32_t a = acc[2 * w + h];
            m |= (unsigned long long)(spread(a & 0xFFFFu) | (spread(a >> 16) << 1)) << (32 * h);
        }
        mk[w] = m;
    }
}

// the selection masks of a bf16 row (M >= 32, K <= 16) from its raw registers
template <int M>
__device__ __forceinline__ void pk_select(const uint32_t (&raw)[M / 2], int K, unsigned long long (&mk)[(M + 63) / 64]) {
    constexpr int NB = M / 32;  // register sets of 16: the even and the odd slots of 32
    static_assert(NB == 1 || NB == 2 || NB == 4, "M");
    constexpr int MW = (M + 63) / 64;
    u16x2 key[M / 2];
#pragma unroll
    for (int r = 0; r < M / 2; ++r) key[r] = pair_keys(raw[r]);
    unsigned short th;
    if (K == 1) {  // the largest key: a running maximum, no network
        u16x2 mx = key[0];
#pragma unroll
        for (int r = 1; r < M / 2; ++r) mx = __builtin_elementwise_max(mx, key[r]);
        th = mx.x > mx.y ? mx.x : mx.y;
    } else {
        u16x2 e[16];
        {
            u16x2 w[NB][16];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
#pragma unroll
                for (int i = 0; i < 16; ++i) w[b][i] = key[16 * b + i];
                pk_sort16_desc(w[b]);
            }
            if constexpr (NB == 1) {
                pk_combine(w[0], w[0], e);
            } else if constexpr (NB == 2) {
                u16x2 q[16];
                pk_combine(w[0], w[1], q);
                pk_combine(q, q, e);
            } else {
                u16x2 q0[16], q1[16], r[16];
                pk_combine(w[0], w[1], q0);
                pk_combine(w[2], w[3], q1);
                pk_combine(q0, q1, r);
                pk_combine(r, r, e);
            }
        }
        th = e[0].x;
#pragma unroll
        for (int r = 1; r < 16; ++r) th = (r == K - 1) ? e[r].x : th;
    }
    pk_mask_ge<M>(key, th, mk);
    int cnt = 0;
#pragma unroll
    for (int w = 0; w < MW; ++w) cnt += __popcll(mk[w]);
    if (cnt > K) {  // keys equal to the threshold beyond the K-th: keep the lowest slots of them
        unsigned long long gt[MW];
        pk_mask_ge<M>(key, static_cast<unsigned short>(th + 1), gt);  // th < 0xFFFF here
        int need = K;
#pragma unroll
        for (int w = 0; w < MW; ++w) need -= __popcll(gt[w]);
#pragma unroll
        for (int w = 0; w < MW; ++w) {
            unsigned long long eq = mk[w] & ~gt[w], sel = 0ull;
            while (need > 0 && eq != 0ull) {
                const unsigned long long lb = eq & (~eq + 1ull);
                sel |= lb;
                eq ^= lb;
                --need;
            }
            mk[w] = gt[w] | sel;
        }
    }
}

// Raw row of M inputs held as 32-bit registers (two bf16 or one fp32 per register).
template <typename T, int M> struct RowRegs;
template <int M> struct RowRegs<bf16_t, M> {
    static constexpr int NR = M / 2;
    uint32_t r[NR];
    __device__ __forceinline__ void load(const bf16_t* p) {
#pragma unroll
        for (int v = 0; v < M / 8; ++v) {
            const uint4 x = reinterpret_cast<const uint4*>(p)[v];
            r[4 * v + 0] = x.x;
            r[4 * v + 1] = x.y;
            r[4 * v + 2] = x.z;
            r[4 * v + 3] = x.w;
        }
    }
    __device__ __forceinline__ float val(int i) const {
        return __uint_as_float((i & 1) ? (r[i >> 1] & 0xFFFF0000u) : (r[i >> 1] << 16));
    }
};
template <int M> struct RowRegs<float, M> {
    float r[M];
    __device__ __forceinline__ void load(const float* p) {
#pragma unroll
        for (int v = 0; v < M / 4; ++v) {
            const float4 x = reinterpret_cast<const float4*>(p)[v];
            r[4 * v + 0] = x.x;
            r[4 * v + 1] = x.y;
            r[4 * v + 2] = x.z;
            r[4 * v + 3] = x.w;
        }
    }
    __device__ __forceinline__ float val(int i) const { return r[i]; }
};

// kFwd = false: public router (idx int32 [row][K], score [row][K] or NULL).
// kFwd = true : forward router, rows in (b*Hh + h, t) order with T_pad tokens per head
//               (T_pad a multiple of the chunk length C): rmask uint64 [..][MW] (bit i%64 of
//               word i/64 set iff slot i is selected, MW = ceil(M/64)), and the alphas of the
//               selected slots in ascending slot order, stored per chunk as [n][C] (entry n
//               of token t of the chunk at n*C + t%C) so that the tokens of a chunk read one
//               entry each from consecutive words; idx int32 [row][K] or NULL.
// SMALLK: K <= 16, threshold by the partial top-16 network; otherwise a full sort.
// One row of the router, computed by the calling lane (the body of route_rows_kernel, also
// run by the chunked forward's first pass when it routes its own segment).  kFwd: row is
// the token-head row in (b, t, h) order, bh = b*Hh + h and t its token; outputs and layouts
// as described above.  Public router: row only.
// kCopy (forward router, K <= 16): also the token's mask words into cmask[0 .. MW-1] and its
// alpha list in ascending slot order into clist[0 .. K-1] (a token-major copy for the caller).
template <typename T, int M, bool kFwd, bool SMALLK, bool kCopy = false>
__device__ __forceinline__ void route_row(const T* __restrict__ z, const float* __restrict__ f, long row, long bh,
                                          long t, long T_pad, int K, int C, int32_t* __restrict__ idx,
                                          float* __restrict__ score, unsigned long long* __restrict__ rmask,
                                          float* __restrict__ ralpha, unsigned long long* cmask = nullptr,
                                          float* clist = nullptr) {
    static_assert(!kCopy || (kFwd && SMALLK), "the copy is a forward-router option for K <= 16");
    // the walk over the selection mask below visits word 0, then word MW-1: at most two words
    static_assert(M <= 128, "route_row covers at most 128 slots (the M = 256 router is route_wave_kernel)");
    typedef typename RowKey<T>::type U;
    RowRegs<T, M> x;
    x.load(z + row * M);
    const float ft = kFwd ? f[row] : 0.0f;  // issued with the row: its latency overlaps the top-K
    const bool all = (K == M);
    constexpr bool kPacked = std::is_same<T, bf16_t>::value && M >= 32 && SMALLK;
    constexpr bool kValKey = std::is_same<T, float>::value && SMALLK;  // fp32 rows: 32-bit value keys
    // selected slots as a bit mask (bit i%64 of word i/64)
    constexpr int MW = (M + 63) / 64;
    unsigned long long mk[MW];
#pragma unroll
    for (int wd = 0; wd < MW; ++wd) mk[wd] = 0ull;
    U th = 0;
    if (!all && !kPacked) {
        float v[M];
#pragma unroll
        for (int i = 0; i < M; ++i) v[i] = x.val(i);
        if constexpr (kValKey) select16_f32<M>(v, K, mk);
        else if constexpr (SMALLK) th = row_threshold16<T, M>(v, K);
        else th = row_threshold<T, M>(v, K);
    }
    if (!all && kPacked) {
        if constexpr (kPacked) pk_select<M>(x.r, K, mk);
    } else if (!all && !kValKey) {
#pragma unroll
        for (int i = 0; i < M; ++i)
            if (RowKey<T>::make(x.val(i), i) >= th) mk[i >> 6] |= 1ull << (i & 63);
    } else if (all) {
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) mk[wd] = (M - 64 * wd >= 64) ? ~0ull : ((1ull << (M - 64 * wd)) - 1ull);
    }
    const long dst = row * K;
    const T* zrow = z + row * M;
    if (kFwd) {
        const long orow = bh * T_pad + t;
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) rmask[orow * MW + wd] = mk[wd];
        if constexpr (kCopy) {
#pragma unroll
            for (int wd = 0; wd < MW; ++wd) cmask[wd] = mk[wd];
        }
    }
    float* alist = kFwd ? ralpha + (bh * T_pad + (t - t % C)) * K + t % C : nullptr;  // entry n at alist[n*C]
    // walk the selected slots in ascending order (lowest set bit first); the logit of a
    // selected slot is read again from the row just loaded (cached)
    unsigned long long m0 = mk[0], m1 = MW > 1 ? mk[MW - 1] : 0ull;
    if constexpr (SMALLK) {
        // K <= 16: all slot numbers first, then every logit load at once (one round trip)
        int sl[16];
        float zv[16];
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            int i = 0;
            if (MW == 1 || m0 != 0ull) {
                i = m0 != 0ull ? __builtin_ctzll(m0) : 0;
                m0 &= m0 - 1ull;
            } else {
                i = 64 + __builtin_ctzll(m1);
                m1 &= m1 - 1ull;
            }
            sl[n] = n < K ? i : 0;
        }
#pragma unroll
        for (int n = 0; n < 16; ++n) zv[n] = Elem<T>::load(zrow, sl[n]);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            if (n < K) {
                const float sc = sigmoidf_dev(zv[n]);
                if (kFwd) {
                    const float al = sc > 0.0f ? __expf(sc * ft) : 1.0f;
                    alist[long(n) * C] = al;
                    if constexpr (kCopy) clist[n] = al;
                    if (idx) idx[dst + n] = sl[n];
                } else {
                    idx[dst + n] = sl[n];
                    if (score) score[dst + n] = sc;
                }
            }
        }
        return;
    }
    if (all) {  // K = M: every slot, in order, its logit from the row in registers
#pragma unroll
        for (int i = 0; i < M; ++i) {
            const float s = sigmoidf_dev(x.val(i));
            if (kFwd) {
                alist[long(i) * C] = s > 0.0f ? __expf(s * ft) : 1.0f;
                if (idx) idx[dst + i] = i;
            } else {
                idx[dst + i] = i;
                if (score) score[dst + i] = s;
            }
        }
        return;
    }
    for (int n = 0; n < K; ++n) {
        int i;
        if (MW == 1 || m0 != 0ull) {
            i = __builtin_ctzll(m0);
            m0 &= m0 - 1ull;
        } else {
            i = 64 + __builtin_ctzll(m1);
            m1 &= m1 - 1ull;
        }
        const float s = sigmoidf_dev(Elem<T>::load(zrow, i));
        if (kFwd) {
            alist[long(n) * C] = s > 0.0f ? __expf(s * ft) : 1.0f;
            if (idx) idx[dst + n] = i;
        } else {
            idx[dst + n] = i;
            if (score) score[dst + n] = s;
        }
    }
}

}  // namespace rsm
