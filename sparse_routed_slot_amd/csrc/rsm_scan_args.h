// rsm_scan_args.h -- launch arguments of the chunk scan (shared by the host launcher and the
// per-type kernel instantiation units).
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/rsm.h"

namespace rsm {

// Largest K of the chunked forward at M = 256 (the alpha lists in LDS are sized for it).
constexpr int kRouteKCap256 = 32;

struct SegArgs {
    long nC;    // chunks in the sequence
    int S;      // segments
    int cps;    // chunks per segment
    float* dH;  // [B*Hh][S-1][M][Dv]
    float* dE;  // [B*Hh][S-1][M]
};

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
    // the router's inputs and optional idx output, used when the first pass routes
    // (fuse_route: bf16 inputs, default router, K <= 16, one Dv tile per head, more than one
    // segment)
    const void* z;
    const float* f;
    int32_t* idx_out;
    bool fuse_route;
    // every slot every token (K = M, default router): no route, the passes form the alphas
    // from z and f (bf16, M = 128)
    bool dense;
};

// Between the two passes: dH_s <- H_start(s+1) = diag(E_s) H_start(s) + dH_s for s = 0 .. S-2,
// H_start(0) = H0 (or zero), so that each segment of pass B reads its start state directly.
// keep: rows with E_s = 1 keep their bits (their dH_s is zero); false for a fold whose
// untouched rows still carry a contribution (the backward's gradient carries).
int seg_fold_launch(const float* H0, const SegArgs& sg, long BH, int M, int Dv, hipStream_t stream, bool keep = true);

// Launch passes A (if S > 1) and B of the chunk scan for one input type and slot count M;
// C and DT are the chunk length and Dv tile the layout chose.  Each is defined in its own
// compilation unit (rsm_scan_<type>_m<M>.hip).
#define RSM_SCAN_DECL(TY, MV) int scan_##TY##_m##MV(int C, int DT, const ScanArgs& a);
RSM_SCAN_DECL(f32, 16)
RSM_SCAN_DECL(f32, 32)
RSM_SCAN_DECL(f32, 64)
RSM_SCAN_DECL(f32, 128)
RSM_SCAN_DECL(bf16, 16)
RSM_SCAN_DECL(bf16, 32)
RSM_SCAN_DECL(bf16, 64)
RSM_SCAN_DECL(bf16, 128)
RSM_SCAN_DECL(bf16, 256)
#undef RSM_SCAN_DECL

}  // namespace rsm
