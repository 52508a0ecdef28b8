// rsm_launch.h -- host-side launchers implemented by the kernel sources and called by the
// C ABI layer (rsm_api.hip).  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/rsm.h"

namespace rsm {

// Router / decay variant as the kernels take it (validated copy of rsm_router_opts).
struct RouterOpts {
    int softmax;        // scores: 0 sigmoid, 1 softmax over all M logits
    int normalize;      // selected scores divided by their sum
    int f_per_slot;     // f [.., M] instead of [..]
    const float* noise; // fp32 [.., M] added to z, or nullptr
    bool is_default() const { return !softmax && !normalize && !f_per_slot && !noise; }
};

int route_topk_launch(const void* z, int dtype, long n_rows, int M, int K, int32_t* idx,
                      float* score, const RouterOpts& op, hipStream_t stream);

int decode_step_launch(const void* q, const void* k, const void* z, const void* v, int dtype,
                       const float* f, float* H, long n_heads, int M, int Dv, int K, float* o,
                       int32_t* idx_out, const RouterOpts& op, hipStream_t stream);

// Workspace of the chunked forward: the route of every token-head in (batch*head, padded
// token) order -- a selection bit mask (uint64 words) and the alphas of the selected slots
// (fp32, ascending slot order, slot-major within each chunk) -- then the state and decay
// product of every sequence segment but the last, and room for a copy of H0 (in-place calls
// with segments); byte offsets and total.
struct FwdLayout {
    size_t rmask_off, ralpha_off;  // route
    size_t dh_off, de_off;         // per-segment states and decay products (S > 1)
    size_t h0c_off;                // copy of H0 for an in-place call (S > 1)
    size_t total;
    long n_chunks;
    int chunk;  // chunk length the kernels run
    int dt;     // Dv columns per workgroup
    int S;      // sequence segments per head
    int cps;    // chunks per segment
};
FwdLayout forward_layout(int dtype, long B, long T, long Hh, int M, int Dv, int C, int K);
// whether the forward at M = 256 runs chunked (else in the recurrent form)
bool chunked_m256(int dtype, int K, const RouterOpts& op);

int route_fwd_launch(const void* z, int dtype, const float* f, long B, long T, long Hh, long T_pad, int M, int K,
                     int C, int32_t* idx_out, unsigned long long* rmask, float* ralpha, const RouterOpts& op,
                     hipStream_t stream);

// Forward in the recurrent form (M = 256): the router over all rows into the workspace (or
// idx_out), then one workgroup per (head, column tile) walks the tokens in order.
size_t forward_recurrent_workspace(long B, long T, long Hh, int K);
int forward_recurrent_launch(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                             const float* H0, long B, long T, long Hh, int M, int Dv, int K, float* o, float* H_out,
                             int32_t* idx_out, void* workspace, const RouterOpts& op, hipStream_t stream);

// Backward pass (default router): gradients of q, k, z, v, f and H0 for upstream gradients
// dO and dH_T (nullable); workspace of backward_workspace() bytes.
size_t backward_workspace(long B, long T, long Hh, int M, int Dv, int K);
int backward_launch(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                    const float* H0, const float* dO, const float* dHT, long B, long T, long Hh, int M, int Dv, int K,
                    float* dq, float* dk, float* dz, float* dv, float* df, float* dH0, void* workspace,
                    hipStream_t s);

int forward_chunked_launch(const void* q, const void* k, const void* z, const void* v, int dtype,
                           const float* f, const float* H0, long B, long T, long Hh, int M,
                           int Dv, int K, int C, float* o, float* H_out, int32_t* idx_out,
                           void* workspace, const RouterOpts& op, hipStream_t stream);

}  // namespace rsm
