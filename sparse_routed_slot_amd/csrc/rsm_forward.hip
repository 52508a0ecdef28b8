// rsm_forward.hip -- host side of the chunked forward: workspace layout, segment split, and the
// launch sequence (route, then passes A and B of the chunk scan).  The kernels are in
// rsm_scan.h (method, layout and precision notes there) and rsm_route.hip.
#include "rsm_device.h"
#include "rsm_launch.h"
#include "rsm_scan_args.h"

namespace rsm {

// H_out = H0 (or zeros) for empty sequences.
__global__ void copy_state_kernel(const float* __restrict__ H0, float* __restrict__ H_out, long n) {
    const long i = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) H_out[i] = H0 ? H0[i] : 0.0f;
}

// Segment fold (see seg_fold_launch): one thread per W consecutive columns of a state row
// (W = 4, or 1 when there are too few float4 of state to fill the chip); the segments are
// walked in order, their (E, dH) read a batch at a time ahead of use.
// keep: a row whose product E is 1 (untouched in the segment, so its dH is zero) keeps its
// bits; otherwise every row is folded.
template <int W>
__global__ void seg_fold_kernel(const float* __restrict__ H0, float* __restrict__ dH, const float* __restrict__ dE,
                                long nw, int S, int M, int Dv, int keep) {
    constexpr int NB = 8;
    typedef float vec __attribute__((ext_vector_type(W)));
    for (long idx = long(blockIdx.x) * blockDim.x + threadIdx.x; idx < nw; idx += long(gridDim.x) * blockDim.x) {
        const long e0 = idx * W;
        const int d = int(e0 % Dv);
        const long row = e0 / Dv;  // bh * M + i
        const long bh = row / M;
        const int i = int(row % M);
        vec hv = H0 ? *reinterpret_cast<const vec*>(H0 + e0) : vec(0.0f);
        for (int s0 = 0; s0 < S - 1; s0 += NB) {
            float e[NB];
            vec x[NB];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (s0 + j < S - 1) {
                    const long r = (bh * (S - 1) + s0 + j) * M + i;
                    e[j] = dE[r];
                    x[j] = *reinterpret_cast<const vec*>(dH + r * Dv + d);
                }
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if (s0 + j < S - 1) {
                    const long r = (bh * (S - 1) + s0 + j) * M + i;
                    if (!keep || e[j] != 1.0f) {  // rows untouched in the segment keep their bits
#pragma unroll
                        for (int c = 0; c < W; ++c) hv[c] = fmaf(e[j], hv[c], x[j][c]);
                    }
                    *reinterpret_cast<vec*>(dH + r * Dv + d) = hv;
                }
            }
        }
    }
}

// idx of a dense route (K = M): slot i in entry i of every token-head row
__global__ void idx_iota_kernel(int32_t* __restrict__ idx, long n, int M) {
    const long e = long(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e < n) idx[e] = int32_t(e % M);
}

int seg_fold_launch(const float* H0, const SegArgs& sg, long BH, int M, int Dv, hipStream_t stream, bool keep) {
    const long n = BH * M * Dv;
    if (n / 4 >= 65536) {  // enough float4 of state for 256 blocks of 256 threads
        const long blocks = (n / 4 + 255) / 256;
        hipLaunchKernelGGL(seg_fold_kernel<4>, dim3(unsigned(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, H0,
                           sg.dH, sg.dE, n / 4, sg.S, M, Dv, keep ? 1 : 0);
    } else {
        const long blocks = (n + 255) / 256;
        hipLaunchKernelGGL(seg_fold_kernel<1>, dim3(unsigned(blocks < 4096 ? blocks : 4096)), dim3(256), 0, stream, H0,
                           sg.dH, sg.dE, n, sg.S, M, Dv, keep ? 1 : 0);
    }
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

// ------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Chunk length the kernels run: the requested C, except M = 128, whose C = 64 tiles do not
// fit in LDS and run as chunks of 32, and M = 256, which always runs chunks of 32 (same
// result up to rounding).
static int scan_chunk(int M, int C) { return M == 256 ? 32 : (M == 128 && C > 32) ? 32 : C; }

// Dv tile of a workgroup: the whole head up to 128 columns (bf16) / 64 (fp32), half that
// for M >= 128 (the fp32 state tile is at most 32 KB, 64 KB at M = 256).
static int pick_dt(int dtype, int M, int Dv) {
    int cap = dtype == RSM_F32 ? 64 : 128;
    if (M >= 128) cap /= 2;
    return Dv < cap ? Dv : cap;
}

// M = 256 runs chunked for bf16 inputs with the default router and K <= 32 (the alpha lists
// in LDS are sized for that), else in the recurrent form.
bool chunked_m256(int dtype, int K, const RouterOpts& op) {
    return dtype == RSM_BF16 && op.is_default() && K <= kRouteKCap256;
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
    // with segments, a copy of H0 for an in-place call (H_out == H0): the last segment writes
    // H_out while workgroups of earlier segments may still read H0
    L.h0c_off = off;
    if (L.S > 1) off += align256(size_t(B) * size_t(Hh) * size_t(M) * size_t(Dv) * 4);
    L.total = off;
    return L;
}

static int dispatch_m(int dtype, int M, int C, int DT, const ScanArgs& a) {
    const bool f = dtype == RSM_F32;
    switch (M) {
        case 16: return f ? scan_f32_m16(C, DT, a) : scan_bf16_m16(C, DT, a);
        case 32: return f ? scan_f32_m32(C, DT, a) : scan_bf16_m32(C, DT, a);
        case 64: return f ? scan_f32_m64(C, DT, a) : scan_bf16_m64(C, DT, a);
        case 128: return f ? scan_f32_m128(C, DT, a) : scan_bf16_m128(C, DT, a);
        case 256: return f ? RSM_ERR_UNSUPPORTED : scan_bf16_m256(C, DT, a);
    }
    return RSM_ERR_UNSUPPORTED;
}

int forward_chunked_launch(const void* q, const void* k, const void* z, const void* v, int dtype,
                           const float* f, const float* H0, long B, long T, long Hh, int M, int Dv, int K,
                           int C, float* o, float* H_out, int32_t* idx_out, void* workspace,
                           const RouterOpts& op, hipStream_t stream) {
    const long BH = B * Hh;
    if (BH == 0) return RSM_OK;
    if (T == 0) {
        if (!H_out || H_out == H0) return RSM_OK;
        const long n = BH * M * Dv;
        hipLaunchKernelGGL(copy_state_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, H0, H_out, n);
        return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
    }
    if (M == 256 && !chunked_m256(dtype, K, op))  // the recurrent form
        return forward_recurrent_launch(q, k, z, v, dtype, f, H0, B, T, Hh, M, Dv, K, o, H_out, idx_out, workspace, op,
                                        stream);
    const FwdLayout L = forward_layout(dtype, B, T, Hh, M, Dv, C, K);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    if (H0 && H_out == H0 && L.S > 1) {  // in place: the passes read a copy of H0
        float* h0c = reinterpret_cast<float*>(ws + L.h0c_off);
        if (hipMemcpyAsync(h0c, H0, size_t(BH) * size_t(M) * size_t(Dv) * 4, hipMemcpyDeviceToDevice, stream) !=
            hipSuccess)
            return RSM_ERR_HIP;
        H0 = h0c;
    }
    auto* rmask = reinterpret_cast<unsigned long long*>(ws + L.rmask_off);
    auto* ralpha = reinterpret_cast<float*>(ws + L.ralpha_off);
    const SegArgs sg{L.n_chunks, L.S, L.cps, reinterpret_cast<float*>(ws + L.dh_off),
                     reinterpret_cast<float*>(ws + L.de_off)};
    // With more than one segment and one Dv tile per head the first pass routes its own
    // segments (bf16 inputs, default router, K <= 16); otherwise the router kernel runs first.
    const bool fuse = dtype == RSM_BF16 && op.is_default() && K <= 16 && L.S > 1 && L.dt == Dv && M <= 128;
    const bool dense = dtype == RSM_BF16 && op.is_default() && K == M && M == 128;
    if (dense) {
        if (idx_out) {
            const long n = B * T * Hh * long(M);
            hipLaunchKernelGGL(idx_iota_kernel, dim3(unsigned((n + 255) / 256)), dim3(256), 0, stream, idx_out, n, M);
            if (hipGetLastError() != hipSuccess) return RSM_ERR_HIP;
        }
    } else if (!fuse) {
        const int st = route_fwd_launch(z, dtype, f, B, T, Hh, L.n_chunks * L.chunk, M, K, L.chunk, idx_out, rmask,
                                        ralpha, op, stream);
        if (st != RSM_OK) return st;
    }
    const ScanArgs a{q, k, v, H0, B, T, Hh, Dv, K, sg, rmask, ralpha, o, H_out, stream, z, f, idx_out, fuse, dense};
    return dispatch_m(dtype, M, L.chunk, L.dt, a);
}

}  // namespace rsm
