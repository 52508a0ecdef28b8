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
#include <type_traits>

#include "rsm_device.h"
#include "rsm_launch.h"
#include "rsm_route_row.h"
#include "rsm_scan_args.h"

namespace rsm {

// Router kernel: one lane per row (outputs and layouts at route_row, rsm_route_row.h).
template <typename T, int M, bool kFwd, bool SMALLK>
__global__ __launch_bounds__(64) void route_rows_kernel(const T* __restrict__ z, const float* __restrict__ f,
                                                        long n_rows, long T_len, int Hh, long T_pad, int K, int C,
                                                        int32_t* __restrict__ idx, float* __restrict__ score,
                                                        unsigned long long* __restrict__ rmask,
                                                        float* __restrict__ ralpha) {
    const int lane = threadIdx.x;
    // public router: lane = row.  Forward router: a workgroup takes 64 consecutive tokens of
    // one (b, h), so the route it writes (per token, and per chunk slot-major) is contiguous.
    long row, t = 0, bh = 0;
    if (kFwd) {
        const long nbt = (T_len + 63) / 64;
        const long id = xcd_head_major(blockIdx.x, gridDim.x, gridDim.x / nbt);
        bh = id / nbt;
        t = (id % nbt) * 64 + lane;
        if (t >= T_len) return;  // no cross-lane operations below
        row = ((bh / Hh) * T_len + t) * Hh + bh % Hh;
    } else {
        row = long(blockIdx.x) * 64 + lane;
        if (row >= n_rows) return;
    }

    route_row<T, M, kFwd, SMALLK>(z, f, row, bh, t, T_pad, K, C, idx, score, rmask, ralpha);
}

// Router variant (softmax scores, renormalised weights, per-slot decay rates, logit noise;
// the cases the pages name besides the default router).  Same outputs and row mapping as
// route_rows_kernel.  Without noise the selection is that of the default router (the
// scores are increasing in the logits), so it uses the same top-K; with noise the logits
// z + g (one fp32 add) are ranked by value with 32-bit keys, ties to the lower slot (K <= 16),
// or with packed 64-bit keys (value, then inverted slot) above that.
// The selected slots are walked in ascending order as in route_rows_kernel, their logits
// (and noise) read again from the rows just loaded; the softmax denominator is a sum over
// the whole row.
template <typename T, int M, bool kFwd, bool SMALLK, bool NOISY>
__global__ __launch_bounds__(64) void route_rows_ex_kernel(const T* __restrict__ z, const float* __restrict__ f,
                                                           long n_rows, long T_len, int Hh, long T_pad, int K, int C,
                                                           int32_t* __restrict__ idx, float* __restrict__ score,
                                                           unsigned long long* __restrict__ rmask,
                                                           float* __restrict__ ralpha, RouterOpts op) {
    typedef typename RowKey<T>::type U;
    const int lane = threadIdx.x;
    // row of the workgroup's l-th lane, and whether it exists
    const long nbt = (T_len + 63) / 64;
    const long bid = kFwd ? xcd_head_major(blockIdx.x, gridDim.x, gridDim.x / nbt) : long(blockIdx.x);
    const long bh = kFwd ? bid / nbt : 0;
    const long t0 = kFwd ? (bid % nbt) * 64 : 0;
    auto row_of = [&](int l, bool& ok) {
        if (kFwd) {
            ok = t0 + l < T_len;
            return ((bh / Hh) * T_len + (ok ? t0 + l : 0)) * Hh + bh % Hh;
        }
        ok = long(blockIdx.x) * 64 + l < n_rows;
        return ok ? long(blockIdx.x) * 64 + l : 0l;
    };
    bool valid;
    const long row = row_of(lane, valid);
    const long t = t0 + lane;
    // The noise rows (4*M contiguous bytes each) go through LDS: loaded row by row with
    // consecutive lanes on consecutive 16-byte pieces, then each lane reads its own row (read
    // directly, lane by lane, they made an uncoalesced stream).  One pad granule per LDS row.
    // The per-slot decay rates of the forward router (read at the K selected slots) likewise.
    // (not both: two 17 KB tiles per wave leave room for four waves per CU, measured slower)
    constexpr bool kStage = NOISY && M <= 64, kStageF = kFwd && M <= 64 && !NOISY;
    constexpr int GPR = M / 4, GP = GPR + 1;
    __shared__ float4 sg[kStage ? 64 * GP : 1];
    __shared__ float4 sf[kStageF ? 64 * GP : 1];
    auto stage = [&](float4* dst, const float* src) {
#pragma unroll
        for (int it = 0; it < GPR; ++it) {
            const int e = it * 64 + lane, rl = e / GPR, c = e % GPR;
            bool ok;
            const long r = row_of(rl, ok);
            if (ok) dst[rl * GP + c] = reinterpret_cast<const float4*>(src + r * M)[c];
        }
    };
    const bool stage_f = kStageF && op.f_per_slot;  // uniform
    if constexpr (kStage) stage(sg, op.noise);
    if (stage_f) stage(sf, f);
    if (kStage || stage_f) __syncthreads();
    if (!valid) return;  // no cross-lane operations below

    RowRegs<T, M> x;
    x.load(z + row * M);
    const float* grow = !NOISY ? nullptr : kStage ? reinterpret_cast<const float*>(sg + lane * GP) : op.noise + row * M;
    constexpr int MW = (M + 63) / 64;
    unsigned long long mk[MW];
#pragma unroll
    for (int wd = 0; wd < MW; ++wd) mk[wd] = (M - 64 * wd >= 64) ? ~0ull : ((1ull << (M - 64 * wd)) - 1ull);
    float zmax = 0.0f, rden = 1.0f;
    {
        float v[M];
#pragma unroll
        for (int i = 0; i < M; ++i) v[i] = x.val(i);
        if constexpr (NOISY) {
            const float4* g4 = reinterpret_cast<const float4*>(grow);
#pragma unroll
            for (int c = 0; c < M / 4; ++c) {
                const float4 g = g4[c];
                v[4 * c] += g.x;
                v[4 * c + 1] += g.y;
                v[4 * c + 2] += g.z;
                v[4 * c + 3] += g.w;
            }
        }
        if (K < M) {
#pragma unroll
            for (int wd = 0; wd < MW; ++wd) mk[wd] = 0ull;
            constexpr bool kPacked = std::is_same<T, bf16_t>::value && M >= 32 && SMALLK;
            if constexpr (kPacked && !NOISY) {
                pk_select<M>(x.r, K, mk);
            } else if constexpr (SMALLK && (NOISY || std::is_same<T, float>::value)) {
                select16_f32<M>(v, K, mk);  // fp32 values: the noisy logits, or fp32 rows
            } else if constexpr (!NOISY) {
                U th;
                if constexpr (SMALLK) th = row_threshold16<T, M>(v, K);
                else th = row_threshold<T, M>(v, K);
#pragma unroll
                for (int i = 0; i < M; ++i)
                    if (RowKey<T>::make(v[i], i) >= th) mk[i >> 6] |= 1ull << (i & 63);
            } else {
                typename RowKey<float>::type th = row_threshold<float, M>(v, K);
#pragma unroll
                for (int i = 0; i < M; ++i)
                    if (RowKey<float>::make(v[i], i) >= th) mk[i >> 6] |= 1ull << (i & 63);
            }
        }
        if (op.softmax) {
            zmax = v[0];
#pragma unroll
            for (int i = 1; i < M; ++i) zmax = fmaxf(zmax, v[i]);
            float den = 0.0f;
#pragma unroll
            for (int i = 0; i < M; ++i) den += __expf(v[i] - zmax);
            rden = 1.0f / den;
        }
    }
    const T* zrow = z + row * M;
    auto logit = [&](int i) { return NOISY ? Elem<T>::load(zrow, i) + grow[i] : Elem<T>::load(zrow, i); };
    auto weight = [&](float zi) { return op.softmax ? __expf(zi - zmax) * rden : sigmoidf_dev(zi); };
    const long dst = row * K;
    if (kFwd) {
        const long orow = bh * T_pad + t;
#pragma unroll
        for (int wd = 0; wd < MW; ++wd) rmask[orow * MW + wd] = mk[wd];
    }
    float* alist = kFwd ? ralpha + (bh * T_pad + (t - t % C)) * K + t % C : nullptr;  // entry n at alist[n*C]
    const float* frow = !kFwd ? nullptr
                        : stage_f ? reinterpret_cast<const float*>(sf + lane * GP)
                        : op.f_per_slot ? f + row * M : f + row;
    auto emit = [&](int n, int i, float s) {
        if (kFwd) {
            const float fi = frow[op.f_per_slot ? i : 0];
            alist[long(n) * C] = s > 0.0f ? __expf(s * fi) : 1.0f;
            if (idx) idx[dst + n] = i;
        } else {
            idx[dst + n] = i;
            if (score) score[dst + n] = s;
        }
    };
    auto next_slot = [&](unsigned long long& m0, unsigned long long& m1) {
        int i;
        if (MW == 1 || m0 != 0ull) {
            i = m0 != 0ull ? __builtin_ctzll(m0) : 0;
            m0 &= m0 - 1ull;
        } else {
            i = 64 + __builtin_ctzll(m1);
            m1 &= m1 - 1ull;
        }
        return i;
    };
    unsigned long long m0 = mk[0], m1 = MW > 1 ? mk[MW - 1] : 0ull;
    if constexpr (SMALLK) {
        int sl[16];
        float sc[16], tot = 0.0f;
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            const int i = next_slot(m0, m1);
            sl[n] = n < K ? i : 0;
        }
#pragma unroll
        for (int n = 0; n < 16; ++n) sc[n] = logit(sl[n]);
#pragma unroll
        for (int n = 0; n < 16; ++n) {
            sc[n] = n < K ? weight(sc[n]) : 0.0f;
            tot += sc[n];
        }
        const float rt = (op.normalize && tot > 0.0f) ? 1.0f / tot : 1.0f;
#pragma unroll
        for (int n = 0; n < 16; ++n)
            if (n < K) emit(n, sl[n], sc[n] * rt);
        return;
    }
    float rt = 1.0f;
    if (op.normalize) {
        unsigned long long a0 = m0, a1 = m1;
        float tot = 0.0f;
        for (int n = 0; n < K; ++n) tot += weight(logit(next_slot(a0, a1)));
        if (tot > 0.0f) rt = 1.0f / tot;
    }
    for (int n = 0; n < K; ++n) {
        const int i = next_slot(m0, m1);
        emit(n, i, weight(logit(i)) * rt);
    }
}

// Public router for wide rows (M = 256, the pages' default slot count): one wave per row,
// lane l holding slots r*64 + l, the exact top-K by the wave-wide bitwise threshold search
// (rsm_device.h), then the scores (sigmoid, or softmax over the row) of the selected slots,
// renormalised over them if asked, and each selected slot's position in the ascending list.
template <typename T, int M, bool EX>
__global__ __launch_bounds__(256) void route_wave_kernel(const T* __restrict__ z, long n_rows, int K,
                                                         int32_t* __restrict__ idx, float* __restrict__ score,
                                                         RouterOpts op) {
    constexpr int SPL = M / kWave;
    constexpr int NB = EX ? 32 : Elem<T>::kKeyBits;
    const int lane = threadIdx.x & 63;
    const long row = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;  // the whole wave
    float zv[SPL];
    uint32_t key[SPL];
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
        zv[r] = Elem<T>::load(z + row * M, r * kWave + lane);
        if (EX && op.noise) zv[r] += op.noise[row * M + r * kWave + lane];
        key[r] = order_key<NB>(zv[r]);
    }
    bool sel[SPL];
    wave_topk<SPL, NB>(key, K, sel);
    float sc[SPL];
    if constexpr (EX) {
        float zmax = -INFINITY, rden = 1.0f, tot = 0.0f;
        if (op.softmax) {
#pragma unroll
            for (int r = 0; r < SPL; ++r) zmax = fmaxf(zmax, zv[r]);
            zmax = wave_max(zmax);
            float den = 0.0f;
#pragma unroll
            for (int r = 0; r < SPL; ++r) den += __expf(zv[r] - zmax);
            rden = 1.0f / wave_sum(den);
        }
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            sc[r] = sel[r] ? (op.softmax ? __expf(zv[r] - zmax) * rden : sigmoidf_dev(zv[r])) : 0.0f;
            tot += sc[r];
        }
        if (op.normalize) {
            tot = wave_sum(tot);
            if (tot > 0.0f) {
                const float rt = 1.0f / tot;
#pragma unroll
                for (int r = 0; r < SPL; ++r) sc[r] *= rt;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < SPL; ++r) sc[r] = sel[r] ? sigmoidf_dev(zv[r]) : 0.0f;
    }
    int pos[SPL];
    wave_compact<SPL>(sel, pos);
#pragma unroll
    for (int r = 0; r < SPL; ++r)
        if (sel[r]) {
            idx[row * K + pos[r]] = r * kWave + lane;
            if (score) score[row * K + pos[r]] = sc[r];
        }
}

// Forward router at M = 256 (default router), for the chunked forward: one workgroup of 8
// waves per (b*Hh + h, chunk of C tokens).  Wave w routes tokens w, w + 8, ... of the chunk,
// a token per wave (lane l holds slots r*64 + l, the exact top-K by the bitwise threshold
// search of wave_topk), alpha = exp(s*f) of each selected slot going to its list position.
// The chunk's alpha lists (slot-major: entry n of token t at n*C + t) and selection masks
// (token-major, 4 words per token) are assembled in LDS and written out contiguously, so
// every store is coalesced; entries of tokens past the sequence end are never read.
template <typename T>
__global__ __launch_bounds__(512) void route_chunk_wave_kernel(const T* __restrict__ z, const float* __restrict__ f,
                                                               long T_len, int Hh, long T_pad, int K, int C,
                                                               int32_t* __restrict__ idx,
                                                               unsigned long long* __restrict__ rmask,
                                                               float* __restrict__ ralpha) {
    constexpr int M = 256, SPL = M / kWave, MW = M / 64, NWV = 8;
    constexpr int NB = Elem<T>::kKeyBits;
    __shared__ float sA[kRouteKCap256 * 64];          // [n][C], C <= 64
    __shared__ unsigned long long sM[64 * MW];         // [t][MW]
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long nch = T_pad / C;
    const long bid = xcd_head_major(blockIdx.x, gridDim.x, gridDim.x / nch);
    const long bh = bid / nch, c = bid % nch;
    const long hb = bh / Hh, hh = bh % Hh;
    for (int tt = w; tt < C; tt += NWV) {
        const long t = c * C + tt;
        if (t >= T_len) break;  // the whole wave
        const long row = (hb * T_len + t) * Hh + hh;
        float zv[SPL];
        uint32_t key[SPL];
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            zv[r] = Elem<T>::load(z + row * M, r * kWave + lane);
            key[r] = order_key<NB>(zv[r]);
        }
        const float ft = f[row];
        bool sel[SPL];
        wave_topk<SPL, NB>(key, K, sel);
        int pos[SPL];
        wave_compact<SPL>(sel, pos);
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            const unsigned long long m = __ballot(sel[r]);
            if (lane == 0) sM[tt * MW + r] = m;
            if (sel[r]) {
                const float sc = sigmoidf_dev(zv[r]);
                sA[pos[r] * C + tt] = sc > 0.0f ? __expf(sc * ft) : 1.0f;
                if (idx) idx[row * K + pos[r]] = r * kWave + lane;
            }
        }
    }
    __syncthreads();
    const long tok0 = bh * T_pad + c * C;
    for (int i = threadIdx.x; i < K * C; i += NWV * kWave) ralpha[tok0 * K + i] = sA[i];
    for (int i = threadIdx.x; i < C * MW; i += NWV * kWave) rmask[tok0 * MW + i] = sM[i];
}

template <typename T, bool kFwd>
static int launch_rows(const T* z, const float* f, long n_rows, long T_len, int Hh, long T_pad, int M, int K, int C,
                       int32_t* idx, float* score, unsigned long long* rmask, float* ralpha, const RouterOpts& op,
                       hipStream_t stream) {
    if (n_rows == 0) return RSM_OK;
    const long nblk = kFwd ? (n_rows / T_len) * ((T_len + 63) / 64) : (n_rows + 63) / 64;
    const dim3 grid(static_cast<unsigned>(nblk)), block(64);
    const size_t lds = 0;
    const bool ex = !op.is_default();
    if (M == 256) {
        if (kFwd) {  // the chunked forward's route (default router, K <= 32, chunks of at most 64)
            if (ex || K > kRouteKCap256 || C > 64 || T_pad % C != 0) return RSM_ERR_UNSUPPORTED;
            const long nblk_c = (n_rows / T_len) * (T_pad / C);
            hipLaunchKernelGGL((route_chunk_wave_kernel<T>), dim3(static_cast<unsigned>(nblk_c)), dim3(512), 0,
                               stream, z, f, T_len, Hh, T_pad, K, C, idx, rmask, ralpha);
            return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
        }
        const dim3 g4(static_cast<unsigned>((n_rows + 3) / 4)), b4(256);
        if (ex)
            hipLaunchKernelGGL((route_wave_kernel<T, 256, true>), g4, b4, 0, stream, z, n_rows, K, idx, score, op);
        else
            hipLaunchKernelGGL((route_wave_kernel<T, 256, false>), g4, b4, 0, stream, z, n_rows, K, idx, score, op);
        return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
    }
#define RSM_ROUTE_EX(MM, SK, NZ)                                                                               \
    hipLaunchKernelGGL((route_rows_ex_kernel<T, MM, kFwd, SK, NZ>), grid, block, lds, stream, z, f, n_rows, T_len,  \
                       Hh, T_pad, K, C, idx, score, rmask, ralpha, op)
#define RSM_ROUTE_LAUNCH(MM)                                                                                   \
    if (ex && K <= 16 && op.noise)                                                                                \
        RSM_ROUTE_EX(MM, true, true);                                                                             \
    else if (ex && K <= 16)                                                                                       \
        RSM_ROUTE_EX(MM, true, false);                                                                            \
    else if (ex && op.noise)                                                                                      \
        RSM_ROUTE_EX(MM, false, true);                                                                            \
    else if (ex)                                                                                                  \
        RSM_ROUTE_EX(MM, false, false);                                                                           \
    else if (K <= 16 && MM >= 16)                                                                                 \
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
#undef RSM_ROUTE_EX
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

int route_topk_launch(const void* z, int dtype, long n_rows, int M, int K, int32_t* idx, float* score,
                      const RouterOpts& op, hipStream_t stream) {
    if (dtype == RSM_F32)
        return launch_rows<float, false>(static_cast<const float*>(z), nullptr, n_rows, 1, 1, 1, M, K, 1, idx, score,
                                         nullptr, nullptr, op, stream);
    return launch_rows<bf16_t, false>(static_cast<const bf16_t*>(z), nullptr, n_rows, 1, 1, 1, M, K, 1, idx, score,
                                      nullptr, nullptr, op, stream);
}

int route_fwd_launch(const void* z, int dtype, const float* f, long B, long T, long Hh, long T_pad, int M, int K,
                     int C, int32_t* idx_out, unsigned long long* rmask, float* ralpha, const RouterOpts& op,
                     hipStream_t stream) {
    const long n_rows = B * T * Hh;
    if (dtype == RSM_F32)
        return launch_rows<float, true>(static_cast<const float*>(z), f, n_rows, T, int(Hh), T_pad, M, K, C, idx_out,
                                        nullptr, rmask, ralpha, op, stream);
    return launch_rows<bf16_t, true>(static_cast<const bf16_t*>(z), f, n_rows, T, int(Hh), T_pad, M, K, C, idx_out,
                                     nullptr, rmask, ralpha, op, stream);
}

}  // namespace rsm
