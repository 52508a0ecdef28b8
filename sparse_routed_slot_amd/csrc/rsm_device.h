// rsm_device.h -- device-side building blocks shared by the librsm kernels (gfx950).
//
// Element access for the two input types, the order-preserving integer key used by
// the router, the wave64 exact top-K, and the MFMA fragment types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rsm {

constexpr int kWave = 64;

// bfloat16 is carried as its 16 raw bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bfloat16, round to nearest even (finite inputs; infinities stay infinite).
__device__ __forceinline__ uint16_t float_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    static constexpr int kKeyBits = 32;
    __device__ static __forceinline__ float load(const float* p, long i) { return p[i]; }
};
template <> struct Elem<bf16_t> {
    static constexpr int kKeyBits = 16;
    __device__ static __forceinline__ float load(const bf16_t* p, long i) {
        return bf16_to_float(p[i].bits);
    }
};

// Order-preserving unsigned key of a float: a < b  <=>  key(a) < key(b), with -0 == +0.
// For bf16-representable values only the top 16 bits carry information.
template <int NB>
__device__ __forceinline__ uint32_t order_key(float x) {
    uint32_t u = __float_as_uint(x);
    if (u == 0x80000000u) u = 0u;
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return NB == 32 ? u : (u >> (32 - NB));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Block index permuted so that a grid whose blocks run head-major (nblk = heads x blocks per
// head) gives XCD x the heads [x*heads/8, (x+1)*heads/8), as the chunk scan does: workgroups
// are dealt to the 8 XCDs round-robin, so data a kernel writes for a head is then read by
// the scan through the same L2.  The identity unless the head count is a multiple of 8.
__device__ __forceinline__ long xcd_head_major(long bid, long nblk, long heads) {
    return heads % 8 == 0 ? (bid % 8) * (nblk / 8) + bid / 8 : bid;
}

__device__ __forceinline__ int popc64(unsigned long long m) { return __popcll(m); }

// Number of set bits of m in lanes below the calling lane.
__device__ __forceinline__ int mbcnt64(unsigned long long m) {
    return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0));
}

// Exact top-K of one row of M <= 64*SPL slots spread over a wave: slot r*64 + lane is held
// in key[r] (0 for lanes past M; every real value has a key >= 1).  A slot is selected iff
// fewer than K slots rank before it, ranking by key descending then slot index ascending.
//
// The K-th largest key is found by a bitwise search from the top bit: keep the candidate
// bit if at least K keys are >= the candidate.  The search stops early once exactly K keys
// are >= the candidate (that set is then the answer, with no tie across its boundary).
// Ties at the threshold are resolved by slot order with a prefix count over the wave.
template <int SPL, int NB>
__device__ __forceinline__ void wave_topk(const uint32_t (&key)[SPL], int K, bool (&sel)[SPL]) {
    uint32_t th = 0;
#pragma unroll 1
    for (int bit = NB - 1; bit >= 0; --bit) {
        const uint32_t cand = th | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int r = 0; r < SPL; ++r) cnt += popc64(__ballot(key[r] >= cand));
        if (cnt >= K) th = cand;
        if (cnt == K) break;
    }
    int gt = 0;
#pragma unroll
    for (int r = 0; r < SPL; ++r) gt += popc64(__ballot(key[r] > th));
    const int need = K - gt;
    int before = 0;
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
        const unsigned long long eq = __ballot(key[r] == th);
        const int rank = before + mbcnt64(eq);
        sel[r] = key[r] > th || (key[r] == th && rank < need);
        before += popc64(eq);
    }
}

// Position of each selected slot in the ascending list of selected slots.
template <int SPL>
__device__ __forceinline__ void wave_compact(const bool (&sel)[SPL], int (&pos)[SPL]) {
    int base = 0;
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
        const unsigned long long m = __ballot(sel[r]);
        pos[r] = base + mbcnt64(m);
        base += popc64(m);
    }
}

__device__ __forceinline__ float sigmoidf_dev(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }

// Sum and maximum over the 64 lanes of a wave (every lane gets the result).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x += __shfl_xor(x, m);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// ------------------------------------------------------------------------------------
// Lane-per-row exact top-K: one lane owns one row of M logits in registers.
//
// Each logit becomes a packed key (order key of the value, then the inverted slot index)
// so that all M packed keys of a row are distinct and ranking them descending ranks the
// slots by (value descending, slot ascending) -- the top-K rule with ties to the lower
// index.  A bitonic network sorts the packed keys descending; the K-th one is the
// threshold, and slot i is selected iff its packed key >= the threshold.
// bf16 inputs pack into 32 bits (16-bit key, 16-bit slot), fp32 inputs into 64 bits.
// ------------------------------------------------------------------------------------
template <typename T> struct RowKey;
template <> struct RowKey<bf16_t> {
    typedef uint32_t type;
    __device__ static __forceinline__ type make(float x, int slot) {
        return (order_key<16>(x) << 16) | uint32_t(0xFFFF - slot);
    }
};
template <> struct RowKey<float> {
    typedef unsigned long long type;
    __device__ static __forceinline__ type make(float x, int slot) {
        return ((unsigned long long)order_key<32>(x) << 32) | (unsigned long long)(0xFFFFFFFFu - uint32_t(slot));
    }
};

template <typename U, int N>
__device__ __forceinline__ void bitonic_sort_desc(U (&kv)[N]) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const U a = kv[i], b = kv[l];
                    const U hi = a > b ? a : b, lo = a > b ? b : a;
                    if ((i & k) == 0) {
                        kv[i] = hi;
                        kv[l] = lo;
                    } else {
                        kv[i] = lo;
                        kv[l] = hi;
                    }
                }
            }
}

// Descending bitonic merge of a bitonic sequence of 16 keys at kv[o .. o+15].
template <typename U, int N>
__device__ __forceinline__ void bitonic_merge_desc16(U (&kv)[N], const int o) {
#pragma unroll
    for (int j = 8; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) {
                const U a = kv[o + i], b = kv[o + l];
                kv[o + i] = a > b ? a : b;
                kv[o + l] = a > b ? b : a;
            }
        }
}

// K-th largest (K <= 16) of M keys, repeated keys counted (kv is overwritten).  Each group
// of 16 keys is sorted descending by a bitonic network; groups are then merged pairwise
// keeping only the top 16 (the elementwise maximum of one sorted list and the other reversed
// holds the top 16 of the union as a bitonic sequence, which a bitonic merge sorts).
template <typename U, int M>
__device__ __forceinline__ U topk16_threshold(U (&kv)[M], int K) {
    static_assert(M % 16 == 0, "groups of 16");
#pragma unroll
    for (int g = 0; g < M; g += 16) {
#pragma unroll
        for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
            for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int l = i ^ j;
                    if (l > i) {
                        const U a = kv[g + i], b = kv[g + l];
                        const U hi = a > b ? a : b, lo = a > b ? b : a;
                        const bool desc = k == 16 || (i & k) == 0;
                        kv[g + i] = desc ? hi : lo;
                        kv[g + l] = desc ? lo : hi;
                    }
                }
    }
#pragma unroll
    for (int span = 16; span < M; span <<= 1)
#pragma unroll
        for (int g = 0; g < M; g += 2 * span) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const U a = kv[g + i], b = kv[g + span + 15 - i];
                kv[g + i] = a > b ? a : b;
            }
            bitonic_merge_desc16<U, M>(kv, g);
        }
    U th = kv[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) th = (r == K - 1) ? kv[r] : th;
    return th;
}

// Threshold packed key of a row for K <= 16: the K-th largest of its M distinct packed keys.
template <typename T, int M>
__device__ __forceinline__ typename RowKey<T>::type row_threshold16(const float (&x)[M], int K) {
    typedef typename RowKey<T>::type U;
    U kv[M];
#pragma unroll
    for (int i = 0; i < M; ++i) kv[i] = RowKey<T>::make(x[i], i);
    return topk16_threshold<U, M>(kv, K);
}

// Selection mask of the K <= 16 largest fp32 values of a row, ties to the lower slot, with
// 32-bit keys of the values alone (half the width of value-and-slot keys): the K-th largest
// value key (repeats counted) is the threshold; every slot above it is selected, and of the
// slots equal to it the lowest ones up to K in all.  The same selection as ranking the
// packed (value, inverted slot) keys.
template <int M>
__device__ __forceinline__ void select16_f32(const float (&x)[M], int K, unsigned long long (&mk)[(M + 63) / 64]) {
    constexpr int MW = (M + 63) / 64;
    uint32_t key[M], kv[M];
#pragma unroll
    for (int i = 0; i < M; ++i) kv[i] = key[i] = order_key<32>(x[i]);
    const uint32_t th = topk16_threshold<uint32_t, M>(kv, K);
    int cnt = 0;
#pragma unroll
    for (int wd = 0; wd < MW; ++wd) mk[wd] = 0ull;
#pragma unroll
    for (int i = 0; i < M; ++i)
        if (key[i] >= th) mk[i >> 6] |= 1ull << (i & 63);
#pragma unroll
    for (int wd = 0; wd < MW; ++wd) cnt += __popcll(mk[wd]);
    if (cnt > K) {  // slots equal to the threshold beyond the K-th: keep the lowest of them
        unsigned long long gt[MW];
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) gt[wd] = 0ull;
#pragma unroll
        for (int i = 0; i < M; ++i)
            if (key[i] > th) gt[i >> 6] |= 1ull << (i & 63);
        int need = K;
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) need -= __popcll(gt[wd]);
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) {
            unsigned long long eq = mk[wd] & ~gt[wd], sel = 0ull;
            while (need > 0 && eq != 0ull) {
                const unsigned long long lb = eq & (~eq + 1ull);
                sel |= lb;
                eq ^= lb;
                --need;
            }
            mk[wd] = gt[wd] | sel;
        }
    }
}

// Threshold packed key of a row: the K-th largest of its M packed keys (K uniform).
template <typename T, int M>
__device__ __forceinline__ typename RowKey<T>::type row_threshold(const float (&x)[M], int K) {
    typedef typename RowKey<T>::type U;
    U kv[M];
#pragma unroll
    for (int i = 0; i < M; ++i) kv[i] = RowKey<T>::make(x[i], i);
    bitonic_sort_desc<U, M>(kv);
    U th = ~U(0);
#pragma unroll
    for (int r = 0; r < M; ++r) th = (r < K && kv[r] < th) ? kv[r] : th;
    return th;
}


// Workgroup barrier without a memory fence.  A workgroup-scope release fence would also
// wait for every global load still in flight (prefetches, direct global->LDS loads), which
// the kernels wait for only where they use them.  LDS is coherent inside the workgroup, so
// each wave's own LDS accesses having completed (lgkmcnt = 0) before s_barrier is what
// makes them visible.  The signal fences keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void wg_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// MFMA fragment types (16x16 output tiles).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

}  // namespace rsm
