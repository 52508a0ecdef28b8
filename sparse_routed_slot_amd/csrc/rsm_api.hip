// rsm_api.hip -- extern "C" entry points of librsm.so (declared in include/rsm.h):
// argument validation, aliasing checks, and dispatch to the kernel launchers.
// No argument error ever reaches the GPU: everything is checked before a launch.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "rsm_launch.h"
#include "rsm_scan_args.h"

namespace {

bool dtype_ok(int dtype) { return dtype == RSM_F32 || dtype == RSM_BF16; }
bool m_ok(int64_t M) { return M == 16 || M == 32 || M == 64 || M == 128; }
// the router and the decode step also take the pages' default slot count
bool m_ok_rd(int64_t M) { return m_ok(M) || M == 256; }
bool dv_ok(int64_t Dv) { return Dv == 16 || Dv == 32 || Dv == 64 || Dv == 128 || Dv == 256; }
bool c_ok(int64_t C) { return C == 16 || C == 32 || C == 64; }
size_t esize(int dtype) { return dtype == RSM_F32 ? 4 : 2; }

// Product of non-negative sizes, or -1 past 2^62.
int64_t mul_ck(std::initializer_list<int64_t> xs) {
    int64_t p = 1;
    for (int64_t x : xs) {
        if (x < 0) return -1;
        if (x != 0 && p > (int64_t(1) << 62) / x) return -1;
        p *= x;
    }
    return p;
}

struct Range {
    const void* p;
    size_t n;
};
bool overlap(Range a, Range b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

// Validated kernel-side copy of a router variant (nullptr = the default router).
bool router_opts(const rsm_router_opts* in, rsm::RouterOpts& out) {
    out = rsm::RouterOpts{0, 0, 0, nullptr};
    if (!in) return true;
    if ((in->score != RSM_SCORE_SIGMOID && in->score != RSM_SCORE_SOFTMAX) || (in->normalize & ~1) ||
        (in->f_per_slot & ~1))
        return false;
    if (reinterpret_cast<uintptr_t>(in->noise) % 16 != 0) return false;  // read as float4 rows
    out = rsm::RouterOpts{in->score, in->normalize, in->f_per_slot, in->noise};
    return true;
}

}  // namespace

extern "C" {

const char* rsm_status_string(int status) {
    switch (status) {
        case RSM_OK: return "ok";
        case RSM_ERR_NULL: return "a required pointer is NULL";
        case RSM_ERR_SHAPE: return "a size is negative or outside the supported set";
        case RSM_ERR_K: return "K must satisfy 1 <= K <= M";
        case RSM_ERR_DTYPE: return "dtype must be RSM_F32 or RSM_BF16";
        case RSM_ERR_UNSUPPORTED: return "combination not built into this library";
        case RSM_ERR_WORKSPACE: return "workspace is NULL or smaller than rsm_forward_workspace_bytes()";
        case RSM_ERR_HIP: return "the HIP runtime reported an error at launch";
        case RSM_ERR_ALIAS: return "an output buffer overlaps an input it must not overlap";
        case RSM_ERR_TOO_LARGE:
            return "the call needs more workspace than the fixed scratch array of the no-allocation entry point";
    }
    return "unknown status";
}

int rsm_abi_version(void) { return 10300; }

int rsm_route_topk(const void* z, int dtype, int64_t B, int64_t T, int64_t Hh, int64_t M, int64_t K,
                   int32_t* idx, float* score, void* stream) {
    return rsm_route_topk_ex(z, dtype, nullptr, B, T, Hh, M, K, idx, score, stream);
}

int rsm_route_topk_ex(const void* z, int dtype, const rsm_router_opts* opts, int64_t B, int64_t T, int64_t Hh,
                      int64_t M, int64_t K, int32_t* idx, float* score, void* stream) {
    rsm::RouterOpts op;
    if (!router_opts(opts, op)) return RSM_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return RSM_ERR_DTYPE;
    if (B < 0 || T < 0 || Hh < 0 || !m_ok_rd(M)) return RSM_ERR_SHAPE;
    if (K < 1 || K > M) return RSM_ERR_K;
    const int64_t rows = mul_ck({B, T, Hh});
    if (rows < 0 || rows / 4 >= (int64_t(1) << 31)) return RSM_ERR_SHAPE;
    if (rows == 0) return RSM_OK;
    if (!z || !idx) return RSM_ERR_NULL;
    const Range rz{z, size_t(rows * M) * esize(dtype)}, ri{idx, size_t(rows * K) * 4},
        rs{score, size_t(rows * K) * 4}, rn{op.noise, size_t(rows * M) * 4};
    if (overlap(ri, rz) || overlap(rs, rz) || overlap(ri, rs) || overlap(ri, rn) || overlap(rs, rn))
        return RSM_ERR_ALIAS;
    return rsm::route_topk_launch(z, dtype, long(rows), int(M), int(K), idx, score, op,
                                  static_cast<hipStream_t>(stream));
}

size_t rsm_forward_workspace_bytes(int dtype, int64_t B, int64_t T, int64_t Hh, int64_t M, int64_t Dv,
                                   int64_t C, int64_t K) {
    if (!dtype_ok(dtype) || B < 0 || T < 0 || Hh < 0 || !m_ok_rd(M) || !dv_ok(Dv) || !c_ok(C)) return 0;
    if (K < 1 || K > M) return 0;
    if (mul_ck({B, T + C, Hh, M, 5}) < 0 || mul_ck({B, Hh, T / C + 2, M, Dv, 4}) < 0) return 0;
    const size_t chunked = rsm::forward_layout(dtype, long(B), long(T), long(Hh), int(M), int(Dv), int(C), int(K)).total;
    if (M != 256) return chunked;
    // M = 256: the recurrent form's workspace, or the chunked one (bf16, K <= 32: the default
    // router runs chunked, a variant recurrent), whichever is larger
    const size_t rec = rsm::forward_recurrent_workspace(long(B), long(T), long(Hh), int(K));
    return (dtype == RSM_BF16 && K <= rsm::kRouteKCap256 && chunked > rec) ? chunked : rec;
}

int rsm_forward_chunked(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                        const float* H0, int64_t B, int64_t T, int64_t Hh, int64_t M, int64_t Dv, int64_t K,
                        int64_t C, float* o, float* H_out, int32_t* idx_out, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return rsm_forward_chunked_ex(q, k, z, v, dtype, f, H0, B, T, Hh, M, Dv, K, C, o, H_out, idx_out, workspace,
                                  workspace_bytes, nullptr, stream);
}

int rsm_forward_chunked_ex(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                           const float* H0, int64_t B, int64_t T, int64_t Hh, int64_t M, int64_t Dv, int64_t K,
                           int64_t C, float* o, float* H_out, int32_t* idx_out, void* workspace,
                           size_t workspace_bytes, const rsm_router_opts* opts, void* stream) {
    rsm::RouterOpts op;
    if (!router_opts(opts, op)) return RSM_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return RSM_ERR_DTYPE;
    if (B < 0 || T < 0 || Hh < 0 || !m_ok_rd(M) || !dv_ok(Dv) || !c_ok(C)) return RSM_ERR_SHAPE;
    if (K < 1 || K > M) return RSM_ERR_K;
    const int64_t rows = mul_ck({B, T, Hh});
    const int64_t heads = mul_ck({B, Hh});
    if (rows < 0 || heads < 0 || mul_ck({rows, M > Dv ? M : Dv}) < 0) return RSM_ERR_SHAPE;
    // recurrent form (M = 256): token indices mark slots as int, the router grid is rows / 4
    if (M == 256 && (T >= (int64_t(1) << 31) || rows / 4 >= (int64_t(1) << 31))) return RSM_ERR_SHAPE;
    const int64_t nbhc = heads * ((T + C - 1) / C);
    if (nbhc >= (int64_t(1) << 31) || heads * (Dv / 16) >= (int64_t(1) << 31)) return RSM_ERR_SHAPE;
    if (heads == 0) return RSM_OK;
    if (T > 0 && (!q || !k || !z || !v || !f || !o)) return RSM_ERR_NULL;
    const size_t es = esize(dtype);
    const size_t need = rsm_forward_workspace_bytes(dtype, B, T, Hh, M, Dv, C, K);
    if (need > 0 && (!workspace || workspace_bytes < need)) return RSM_ERR_WORKSPACE;
    const Range rq{q, size_t(rows * M) * es}, rk{k, size_t(rows * M) * es}, rz{z, size_t(rows * M) * es},
        rv{v, size_t(rows * Dv) * es}, rf{f, size_t(rows) * (op.f_per_slot ? size_t(M) : 1) * 4},
        rh0{H0, size_t(heads * M * Dv) * 4}, ro{o, size_t(rows * Dv) * 4}, rh{H_out, size_t(heads * M * Dv) * 4},
        ri{idx_out, size_t(rows * K) * 4}, rw{workspace, need}, rn{op.noise, size_t(rows * M) * 4};
    const Range ins[] = {rq, rk, rz, rv, rf, rn, rh0};
    const Range outs[] = {ro, ri, rw};
    for (const Range& a : outs) {
        for (const Range& b : ins)
            if (overlap(a, b)) return RSM_ERR_ALIAS;
        if (overlap(a, rh)) return RSM_ERR_ALIAS;
    }
    if (overlap(ro, ri) || overlap(ro, rw) || overlap(ri, rw)) return RSM_ERR_ALIAS;
    for (int j = 0; j < 6; ++j)
        if (overlap(rh, ins[j])) return RSM_ERR_ALIAS;
    if (overlap(rh, rh0) && H_out != H0) return RSM_ERR_ALIAS;
    return rsm::forward_chunked_launch(q, k, z, v, dtype, f, H0, long(B), long(T), long(Hh), int(M), int(Dv),
                                       int(K), int(C), o, H_out, idx_out, workspace, op,
                                       static_cast<hipStream_t>(stream));
}

size_t rsm_backward_workspace_bytes(int dtype, int64_t B, int64_t T, int64_t Hh, int64_t M, int64_t Dv, int64_t K) {
    if (!dtype_ok(dtype) || B < 0 || T < 0 || Hh < 0 || !m_ok_rd(M) || !dv_ok(Dv) || K < 1 || K > M) return 0;
    const int64_t rows = mul_ck({B, T, Hh});
    if (rows < 0 || mul_ck({rows, M, 16}) < 0) return 0;
    return rsm::backward_workspace(long(B), long(T), long(Hh), int(M), int(Dv), int(K));
}

int rsm_backward(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                 const float* H0, const float* dO, const float* dH_T, int64_t B, int64_t T, int64_t Hh, int64_t M,
                 int64_t Dv, int64_t K, float* dq, float* dk, float* dz, float* dv, float* df, float* dH0,
                 void* workspace, size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype)) return RSM_ERR_DTYPE;
    if (B < 0 || T < 0 || Hh < 0 || !m_ok_rd(M) || !dv_ok(Dv)) return RSM_ERR_SHAPE;
    if (K < 1 || K > M) return RSM_ERR_K;
    const int64_t rows = mul_ck({B, T, Hh});
    const int64_t heads = mul_ck({B, Hh});
    if (rows < 0 || heads < 0 || mul_ck({rows, M > Dv ? M : Dv, 16}) < 0) return RSM_ERR_SHAPE;
    if (rows / 4 >= (int64_t(1) << 31) || heads * 16 >= (int64_t(1) << 31)) return RSM_ERR_SHAPE;
    if (heads == 0) return RSM_OK;
    if (T > 0 && (!q || !k || !z || !v || !f || !dO || !dq || !dk || !dz || !dv || !df)) return RSM_ERR_NULL;
    const size_t need = rsm_backward_workspace_bytes(dtype, B, T, Hh, M, Dv, K);
    if (need > 0 && (!workspace || workspace_bytes < need)) return RSM_ERR_WORKSPACE;
    const size_t es = esize(dtype);
    const Range rq{q, size_t(rows * M) * es}, rk{k, size_t(rows * M) * es}, rz{z, size_t(rows * M) * es},
        rv{v, size_t(rows * Dv) * es}, rf{f, size_t(rows) * 4}, rh0{H0, size_t(heads * M * Dv) * 4},
        rdo{dO, size_t(rows * Dv) * 4}, rdh{dH_T, size_t(heads * M * Dv) * 4}, odq{dq, size_t(rows * M) * 4},
        odk{dk, size_t(rows * M) * 4}, odz{dz, size_t(rows * M) * 4}, odv{dv, size_t(rows * Dv) * 4},
        odf{df, size_t(rows) * 4}, odh{dH0, size_t(heads * M * Dv) * 4}, rw{workspace, need};
    const Range ins[] = {rq, rk, rz, rv, rf, rh0, rdo, rdh};
    const Range outs[] = {odq, odk, odz, odv, odf, odh, rw};
    for (int a = 0; a < 7; ++a) {
        for (const Range& b : ins)
            if (overlap(outs[a], b)) return RSM_ERR_ALIAS;
        for (int c = a + 1; c < 7; ++c)
            if (overlap(outs[a], outs[c])) return RSM_ERR_ALIAS;
    }
    return rsm::backward_launch(q, k, z, v, dtype, f, H0, dO, dH_T, long(B), long(T), long(Hh), int(M), int(Dv),
                                int(K), dq, dk, dz, dv, df, dH0, workspace, static_cast<hipStream_t>(stream));
}

int rsm_decode_step(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                    float* H, int64_t B, int64_t Hh, int64_t M, int64_t Dv, int64_t K, float* o,
                    int32_t* idx_out, void* stream) {
    return rsm_decode_step_ex(q, k, z, v, dtype, f, H, B, Hh, M, Dv, K, o, idx_out, nullptr, stream);
}

int rsm_decode_step_ex(const void* q, const void* k, const void* z, const void* v, int dtype, const float* f,
                       float* H, int64_t B, int64_t Hh, int64_t M, int64_t Dv, int64_t K, float* o,
                       int32_t* idx_out, const rsm_router_opts* opts, void* stream) {
    rsm::RouterOpts op;
    if (!router_opts(opts, op)) return RSM_ERR_UNSUPPORTED;
    if (!dtype_ok(dtype)) return RSM_ERR_DTYPE;
    if (B < 0 || Hh < 0 || !m_ok_rd(M) || !dv_ok(Dv)) return RSM_ERR_SHAPE;
    if (K < 1 || K > M) return RSM_ERR_K;
    const int64_t heads = mul_ck({B, Hh});
    if (heads < 0 || heads >= (int64_t(1) << 29) || mul_ck({heads, M, Dv}) < 0) return RSM_ERR_SHAPE;
    if (heads == 0) return RSM_OK;
    if (!q || !k || !z || !v || !f || !H || !o) return RSM_ERR_NULL;
    const size_t es = esize(dtype);
    const Range rq{q, size_t(heads * M) * es}, rk{k, size_t(heads * M) * es}, rz{z, size_t(heads * M) * es},
        rv{v, size_t(heads * Dv) * es}, rf{f, size_t(heads) * (op.f_per_slot ? size_t(M) : 1) * 4},
        rh{H, size_t(heads * M * Dv) * 4}, ro{o, size_t(heads * Dv) * 4}, ri{idx_out, size_t(heads * K) * 4},
        rn{op.noise, size_t(heads * M) * 4};
    const Range ins[] = {rq, rk, rz, rv, rf, rn};
    for (const Range& b : ins)
        if (overlap(rh, b) || overlap(ro, b) || overlap(ri, b)) return RSM_ERR_ALIAS;
    if (overlap(ro, rh) || overlap(ri, rh) || overlap(ro, ri)) return RSM_ERR_ALIAS;
    return rsm::decode_step_launch(q, k, z, v, dtype, f, H, long(heads), int(M), int(Dv), int(K), o, idx_out, op,
                                   static_cast<hipStream_t>(stream));
}

}  // extern "C"
