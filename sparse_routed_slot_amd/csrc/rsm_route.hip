// rsm_route.hip -- standalone router: sigmoid scores and exact top-K per token-head row.
//
// RSM router of Raven (README page, "How Raven Works": TopK(sigmoid(r_proj(x)))), taking
// the projected logits z as input.  One wave64 per row; slot r*64 + lane lives in lane
// `lane`, register r.  The selection is computed on the order-preserving key of z, so
// it equals ranking the exact sigmoid with ties to the lower slot index.
#include "rsm_device.h"
#include "rsm_launch.h"

namespace rsm {

template <typename T, int SPL>
__global__ __launch_bounds__(256) void route_topk_kernel(const T* __restrict__ z, long n_rows, int M,
                                                         int K, int32_t* __restrict__ idx,
                                                         float* __restrict__ score) {
    constexpr int NB = Elem<T>::kKeyBits;
    const int lane = lane_id();
    const long row = long(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (row >= n_rows) return;  // whole wave leaves together
    const T* zr = z + row * M;
    uint32_t key[SPL];
    float zv[SPL];
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
        const int slot = r * kWave + lane;
        zv[r] = slot < M ? Elem<T>::load(zr, slot) : 0.0f;
        key[r] = slot < M ? order_key<NB>(zv[r]) : 0u;
    }
    bool sel[SPL];
    wave_topk<SPL, NB>(key, K, sel);
    int pos[SPL];
    wave_compact<SPL>(sel, pos);
#pragma unroll
    for (int r = 0; r < SPL; ++r) {
        if (sel[r]) {
            idx[row * K + pos[r]] = r * kWave + lane;
            if (score) score[row * K + pos[r]] = 1.0f / (1.0f + expf(-zv[r]));
        }
    }
}

template <typename T>
static int launch_route(const T* z, long n_rows, int M, int K, int32_t* idx, float* score,
                        hipStream_t stream) {
    if (n_rows == 0) return RSM_OK;
    const dim3 grid(unsigned((n_rows + 3) / 4)), block(256);
    if (M <= 64)
        hipLaunchKernelGGL((route_topk_kernel<T, 1>), grid, block, 0, stream, z, n_rows, M, K, idx, score);
    else
        hipLaunchKernelGGL((route_topk_kernel<T, 2>), grid, block, 0, stream, z, n_rows, M, K, idx, score);
    return hipGetLastError() == hipSuccess ? RSM_OK : RSM_ERR_HIP;
}

int route_topk_launch(const void* z, int dtype, long n_rows, int M, int K, int32_t* idx, float* score,
                      hipStream_t stream) {
    if (dtype == RSM_F32) return launch_route(static_cast<const float*>(z), n_rows, M, K, idx, score, stream);
    return launch_route(static_cast<const bf16_t*>(z), n_rows, M, K, idx, score, stream);
}

}  // namespace rsm
