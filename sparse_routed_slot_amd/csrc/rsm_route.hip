// rsm_route.hip -- router kernels: sigmoid scores and exact top-K per token-head row.
//
// RSM router of Raven (README page, "How Raven Works": TopK(sigmoid(r_proj(x))) and
// decay = exp(route_scores * f)), taking the projected logits z as input.
//
// One lane owns one row (M logits in registers).  The exact top-K with ties to the lower
// slot index compares distinct packed keys (order-preserving bits of z, then the inverted
// slot index) with the K-th largest key, found by a bitonic network (rsm_device.h).  The
// selected slots form a bit mask, walked in ascending slot order to score them:
//  * public router: idx (int32) and score = sigmoid(z) per selected slot;
//  * forward router: the per-token route the chunked forward consumes -- a selection bit
//    mask over the M slots and alpha = exp(s*f) of the selected slots in ascending slot
//    order (fp32, exact: 0 for f = -inf, 1 when s*f == 0) -- in (batch*head, token) order,
//    plus the optional int32 idx output in (b, t, h) order.
#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

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
template <typename T, int M, bool kFwd, bool SMALLK>
__global__ __launch_bounds__(64) void route_rows_kernel(const T* __restrict__ z, const float* __restrict__ f,
                                                        long n_rows, long T_len, int Hh, long T_pad, int K, int C,
                                                        int32_t* __restrict__ idx, float* __restrict__ score,
                                                        unsigned long long* __restrict__ rmask,
                                                        float* __restrict__ ralpha) {
    typedef typename RowKey<T>::type U;
    const int lane = threadIdx.x;
    // public router: lane = row.  Forward router: a workgroup takes 64 consecutive tokens of
    // one (b, h), so the route it writes (per token, and per chunk slot-major) is contiguous.
    long row, t = 0, bh = 0;
    if (kFwd) {
        const long nbt = (T_len + 63) / 64;
        bh = long(blockIdx.x) / nbt;
        t = (long(blockIdx.x) % nbt) * 64 + lane;
        if (t >= T_len) return;  // no cross-lane operations below
        row = ((bh / Hh) * T_len + t) * Hh + bh % Hh;
    } else {
        row = long(blockIdx.x) * 64 + lane;
        if (row >= n_rows) return;
    }

    RowRegs<T, M> x;
    x.load(z + row * M);
    const bool all = (K == M);
    U th = 0;
    if (!all) {
        float v[M];
#pragma unroll
        for (int i = 0; i < M; ++i) v[i] = x.val(i);
        if constexpr (SMALLK) th = row_threshold16<T, M>(v, K);
        else th = row_threshold<T, M>(v, K);
    }

    // selected slots as a bit mask (bit i%64 of word i/64)
    constexpr int MW = (M + 63) / 64;
    unsigned long long mk[MW];
#pragma unroll
    for (int wd = 0; wd < MW; ++wd) mk[wd] = 0ull;
    if (!all) {
#pragma unroll
        for (int i = 0; i < M; ++i)
            if (RowKey<T>::make(x.val(i), i) >= th) mk[i >> 6] |= 1ull << (i & 63);
    } else {
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) mk[wd] = (M - 64 * wd >= 64) ? ~0ull : ((1ull << (M - 64 * wd)) - 1ull);
    }
    const long dst = row * K;
    const T* zrow = z + row * M;
    if (kFwd) {
        const long orow = bh * T_pad + t;
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) rmask[orow * MW + wd] = mk[wd];
    }
    float* alist = kFwd ? ralpha + (bh * T_pad + (t - t % C)) * K + t % C : nullptr;  // entry n at alist[n*C]
    const float ft = kFwd ? f[row] : 0.0f;
    // walk the selected slots in ascending order (lowest set bit first); the logit of a
    // selected slot is read again from the row just loaded (cached)
    unsigned long long m0 = mk[0], m1 = MW > 1 ? mk[MW - 1] : 0ull;
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

template <typename T, bool kFwd>
static int launch_rows(const T* z, const float* f, long n_rows, long T_len, int Hh, long T_pad, int M, int K, int C,
                       int32_t* idx, float* score, unsigned long long* rmask, float* ralpha, hipStream_t stream) {
    if (n_rows == 0) return RSM_OK;
    const long nblk = kFwd ? (n_rows / T_len) * ((T_len + 63) / 64) : (n_rows + 63) / 64;
    const dim3 grid(static_cast<unsigned>(nblk)), block(64);
    const size_t lds = 0;
#define RSM_ROUTE_LAUNCH(MM)                                                                                   \
    if (K <= 16 && MM >= 16)                                                                                      \
        hipLaunchKernelGGL((route_rows_kernel<T, MM, kFwd, true>), grid, block, lds, stream, z, f, n_rows, T_len, Hh, \
                           T_pad, K, C, idx, score, rmask, ralpha);                                               \
    else                                                                                                          \
        hipLaunchKernelGGL((route_rows_kernel<T, MM, kFwd, false>), grid, block, lds, stream, z, f, n_rows, T_len, \
                           Hh, T_pad, K, C, idx, score, rmask, ralpha)
    switch (M) {
        case 16: RSM_ROUTE_LAUNCH(16); break;
        case 32: RSM_ROUTE_LAUNCH(32); break;
        case 64: RSM_ROUTE_LAUNCH(64); break;
        case 128: RSM_ROUTE_LAUNCH(128); break;
        default: return RSM_ERR_UNSUPPORTED;
    }
#undef RSM_ROUTE_LAUNCH
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

int route_topk_launch(const void* z, int dtype, long n_rows, int M, int K, int32_t* idx, float* score,
                      hipStream_t stream) {
    if (dtype == RSM_F32)
        return launch_rows<float, false>(static_cast<const float*>(z), nullptr, n_rows, 1, 1, 1, M, K, 1, idx, score,
                                         nullptr, nullptr, stream);
    return launch_rows<bf16_t, false>(static_cast<const bf16_t*>(z), nullptr, n_rows, 1, 1, 1, M, K, 1, idx, score,
                                      nullptr, nullptr, stream);
}

int route_fwd_launch(const void* z, int dtype, const float* f, long B, long T, long Hh, long T_pad, int M, int K,
                     int C, int32_t* idx_out, unsigned long long* rmask, float* ralpha, hipStream_t stream) {
    const long n_rows = B * T * Hh;
    if (dtype == RSM_F32)
        return launch_rows<float, true>(static_cast<const float*>(z), f, n_rows, T, int(Hh), T_pad, M, K, C, idx_out,
                                        nullptr, rmask, ralpha, stream);
    return launch_rows<bf16_t, true>(static_cast<const bf16_t*>(z), f, n_rows, T, int(Hh), T_pad, M, K, C, idx_out,
                                     nullptr, rmask, ralpha, stream);
}

}  // namespace rsm
