// rsm_decode.hip -- fused recurrent decode step (route + sparse update + read) for one
// token of every head.
//
// Raven README page, "How Raven Works": per token, the top-K slots by sigmoid score are
// decayed by alpha = exp(s*f) and written with (1-alpha)*k_i*v; o = q . H is read after
// the update; the README names "fused recurrent kernels for generation" for this case.
//
// Router variants (softmax scores, renormalised weights, per-slot decay rates, logit noise)
// run in the same kernel (EX), the router wave doing the extra reductions.
//
// One workgroup (256 threads) per head.  The fp32 state H [M, Dv] is streamed once as
// float4 rows (Dv/4 threads per row); the loads are issued before the router runs so
// the HBM latency overlaps with the top-K (the router's own inputs are issued first).  Wave 0 routes the M logits (lane = slot) and
// publishes alpha, (1-alpha)*k and q per slot in LDS.  Every thread then updates the
// selected rows it holds in registers, writes back only those rows, and accumulates its
// partial read q_i*H[i,:]; a reduction over row groups in LDS finishes o.
#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

// EX: router variant (op): logits z + noise ranked as fp32 values (32-bit keys), softmax or
// sigmoid scores, optional renormalisation over the selected slots, per-slot decay rates.
// DTC: state columns per workgroup: at most 64 for M <= 64 (measured: 2 tiles of 64 at
// M = 64, d_v = 128 are 1% faster than whole rows, 4 tiles of 32 slower), else the whole row
// unless M * DV is large.  Each column tile's workgroup routes the token again, which is
// cheap, and only tile 0 writes idx_out.
template <int M, int DV>
constexpr int decode_cols() {
    return M <= 64 ? (DV < 64 ? DV : 64) : (DV < 16384 / M ? DV : 16384 / M);
}

template <typename T, int M, int DV, bool EX>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ z, const T* __restrict__ v,
    const float* __restrict__ f, float* __restrict__ H, int K, float* __restrict__ o,
    int32_t* __restrict__ idx_out, RouterOpts op) {
    constexpr int SPL = M > kWave ? M / kWave : 1;
    constexpr int NB = EX ? 32 : Elem<T>::kKeyBits;
    constexpr int DTC = decode_cols<M, DV>(), NTL = DV / DTC;
    constexpr int TPR = DTC / 4;              // threads per state row, one float4 each
    constexpr int RPP = 256 / TPR;            // rows covered per pass of the workgroup
    constexpr int RPT = (M + RPP - 1) / RPP;  // rows held per thread
    __shared__ float s_a[M], s_wk[M], s_q[M];
    __shared__ int s_upd[M];
    __shared__ float4 s_red[RPP][TPR];

    const long bh = blockIdx.x / NTL;
    const int tile = int(blockIdx.x % NTL), c0 = tile * DTC;
    const int tid = threadIdx.x;
    const int cg = tid % TPR, rg = tid / TPR;
    float* Hb = H + bh * long(M) * DV + c0;

    // The router wave's inputs (z, q, k of every slot, noise, f) are loaded ahead of the
    // state rows: they do not queue behind them, and no second round trip follows the top-K.
    float zv[SPL], qv[SPL], kv[SPL], nv[SPL];
    float ft0 = 0.0f;
    if (tid < kWave) {
        const long hb = bh * M;
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            const int slot = r * kWave + tid;
            zv[r] = slot < M ? Elem<T>::load(z + hb, slot) : 0.0f;
            qv[r] = slot < M ? Elem<T>::load(q + hb, slot) : 0.0f;
            kv[r] = slot < M ? Elem<T>::load(k + hb, slot) : 0.0f;
            nv[r] = (EX && op.noise && slot < M) ? op.noise[hb + slot] : 0.0f;
        }
        if (!(EX && op.f_per_slot)) ft0 = f[bh];
    }

    float4 hv[RPT];
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = rg + j * RPP;
        if (row < M) hv[j] = *reinterpret_cast<const float4*>(Hb + row * DV + 4 * cg);
    }
    const T* vb = v + bh * DV + c0 + 4 * cg;
    const float4 vv = make_float4(Elem<T>::load(vb, 0), Elem<T>::load(vb, 1), Elem<T>::load(vb, 2),
                                  Elem<T>::load(vb, 3));

    if (tid < kWave) {
        const int lane = tid;
        uint32_t key[SPL];
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            const int slot = r * kWave + lane;
            if (EX && op.noise) zv[r] += nv[r];
            key[r] = slot < M ? order_key<NB>(zv[r]) : 0u;
        }
        bool sel[SPL];
        wave_topk<SPL, NB>(key, K, sel);
        float sc[SPL];
        if constexpr (EX) {
            float zmax = -INFINITY, rden = 1.0f, tot = 0.0f;
            if (op.softmax) {
#pragma unroll
                for (int r = 0; r < SPL; ++r)
                    if (r * kWave + lane < M) zmax = fmaxf(zmax, zv[r]);
                zmax = wave_max(zmax);
                float den = 0.0f;
#pragma unroll
                for (int r = 0; r < SPL; ++r)
                    if (r * kWave + lane < M) den += __expf(zv[r] - zmax);
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
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            const int slot = r * kWave + lane;
            if (slot < M) {
                float a = 1.0f, wk = 0.0f;
                int upd = 0;
                if (sel[r]) {
                    const float s = sc[r];
                    const float ft = (EX && op.f_per_slot) ? f[bh * M + slot] : ft0;
                    if (s > 0.0f) a = __expf(s * ft);
                    if (a != 1.0f) {
                        upd = 1;
                        wk = (1.0f - a) * kv[r];
                    }
                }
                s_a[slot] = a;
                s_wk[slot] = wk;
                s_upd[slot] = upd;
                s_q[slot] = qv[r];
            }
        }
        if (idx_out && tile == 0) {
            int pos[SPL];
            wave_compact<SPL>(sel, pos);
#pragma unroll
            for (int r = 0; r < SPL; ++r)
                if (sel[r]) idx_out[bh * K + pos[r]] = r * kWave + lane;
        }
    }
    __syncthreads();

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
        const int row = rg + j * RPP;
        if (row < M) {
            float4 h = hv[j];
            if (s_upd[row]) {
                const float a = s_a[row], wk = s_wk[row];
                h.x = fmaf(a, h.x, wk * vv.x);
                h.y = fmaf(a, h.y, wk * vv.y);
                h.z = fmaf(a, h.z, wk * vv.z);
                h.w = fmaf(a, h.w, wk * vv.w);
                *reinterpret_cast<float4*>(Hb + row * DV + 4 * cg) = h;
            }
            const float qi = s_q[row];
            acc.x = fmaf(qi, h.x, acc.x);
            acc.y = fmaf(qi, h.y, acc.y);
            acc.z = fmaf(qi, h.z, acc.z);
            acc.w = fmaf(qi, h.w, acc.w);
        }
    }
    s_red[rg][cg] = acc;
    __syncthreads();
    if (rg == 0) {
        float4 sum = s_red[0][cg];
        for (int g = 1; g < RPP; ++g) {
            const float4 p = s_red[g][cg];
            sum.x += p.x;
            sum.y += p.y;
            sum.z += p.z;
            sum.w += p.w;
        }
        *reinterpret_cast<float4*>(o + bh * DV + c0 + 4 * cg) = sum;
    }
}

template <typename T, int M, int DV>
static int launch_decode_mdv(const T* q, const T* k, const T* z, const T* v, const float* f, float* H,
                             long n_heads, int K, float* o, int32_t* idx_out, const RouterOpts& op,
                             hipStream_t stream) {
    const dim3 grid(unsigned(n_heads * (DV / decode_cols<M, DV>())));
    if (op.is_default())
        hipLaunchKernelGGL((decode_step_kernel<T, M, DV, false>), grid, dim3(256), 0, stream, q, k, z, v, f, H, K, o,
                           idx_out, op);
    else
        hipLaunchKernelGGL((decode_step_kernel<T, M, DV, true>), grid, dim3(256), 0, stream, q, k, z, v, f, H, K, o,
                           idx_out, op);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

template <typename T, int M>
static int launch_decode_m(const T* q, const T* k, const T* z, const T* v, const float* f, float* H,
                           long n_heads, int Dv, int K, float* o, int32_t* idx_out, const RouterOpts& op,
                           hipStream_t s) {
    switch (Dv) {
        case 16: return launch_decode_mdv<T, M, 16>(q, k, z, v, f, H, n_heads, K, o, idx_out, op, s);
        case 32: return launch_decode_mdv<T, M, 32>(q, k, z, v, f, H, n_heads, K, o, idx_out, op, s);
        case 64: return launch_decode_mdv<T, M, 64>(q, k, z, v, f, H, n_heads, K, o, idx_out, op, s);
        case 128: return launch_decode_mdv<T, M, 128>(q, k, z, v, f, H, n_heads, K, o, idx_out, op, s);
        case 256: return launch_decode_mdv<T, M, 256>(q, k, z, v, f, H, n_heads, K, o, idx_out, op, s);
    }
    return RSM_ERR_UNSUPPORTED;
}

template <typename T>
static int launch_decode(const void* q, const void* k, const void* z, const void* v, const float* f,
                         float* H, long n_heads, int M, int Dv, int K, float* o, int32_t* idx_out,
                         const RouterOpts& op, hipStream_t s) {
    const T *qq = static_cast<const T*>(q), *kk = static_cast<const T*>(k), *zz = static_cast<const T*>(z),
            *vv = static_cast<const T*>(v);
    switch (M) {
        case 16: return launch_decode_m<T, 16>(qq, kk, zz, vv, f, H, n_heads, Dv, K, o, idx_out, op, s);
        case 32: return launch_decode_m<T, 32>(qq, kk, zz, vv, f, H, n_heads, Dv, K, o, idx_out, op, s);
        case 64: return launch_decode_m<T, 64>(qq, kk, zz, vv, f, H, n_heads, Dv, K, o, idx_out, op, s);
        case 128: return launch_decode_m<T, 128>(qq, kk, zz, vv, f, H, n_heads, Dv, K, o, idx_out, op, s);
        case 256: return launch_decode_m<T, 256>(qq, kk, zz, vv, f, H, n_heads, Dv, K, o, idx_out, op, s);
    }
    return RSM_ERR_UNSUPPORTED;
}

int decode_step_launch(const void* q, const void* k, const void* z, const void* v, int dtype,
                       const float* f, float* H, long n_heads, int M, int Dv, int K, float* o,
                       int32_t* idx_out, const RouterOpts& op, hipStream_t stream) {
    if (n_heads == 0) return RSM_OK;
    if (dtype == RSM_F32) return launch_decode<float>(q, k, z, v, f, H, n_heads, M, Dv, K, o, idx_out, op, stream);
    return launch_decode<bf16_t>(q, k, z, v, f, H, n_heads, M, Dv, K, o, idx_out, op, stream);
}

}  // namespace rsm
