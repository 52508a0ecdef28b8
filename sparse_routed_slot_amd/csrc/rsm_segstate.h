#pragma once
// rsm_segstate.h -- first pass of the segmented chunked forward: the state every sequence
// segment but the last reaches from a zero state, and its decay product.
//
// The recurrence (Raven README page, "How Raven Works") is linear in the state, so segment s
// of a head contributes
//     dH_s = sum_{t in s} diag(R_t) ((1 - alpha_t) o k_t) v_t^T,   R_t = prod_{tau in s, tau > t} alpha_tau,
//     E_s  = prod_{t in s} alpha_t,
// and the next segment starts from diag(E_s) H_start(s) + dH_s.  Unselected slots have
// alpha = 1 and contribute nothing.  R is a suffix product: it only shrinks, so it can
// underflow to 0 (its exact limit) but never needs a division, a clamp or an exact path,
// and f = -inf (alpha = 0) is exact.
//
// One workgroup of 8 waves per (head, segment).  The segment is routed in rounds of 512
// tokens (one per thread; the route also goes to the workspace for the second pass), then
// its chunks are walked from the last to the first.  Lane = slot: for the chunk's tokens a
// wave takes 8 consecutive ones, gathers each token's alphas through its selection mask
// (the position of a selected slot in the alpha list is the number of selected slots below
// it, one mbcnt for the whole wave), and forms the exclusive suffix product within its 8
// tokens.  The products of the later waves' blocks and of the later chunks (one running
// product per slot) complete R.  W = (1 - alpha) k R goes to LDS as hi / lo bf16 rows, and
// U += W^T V runs on MFMA with the v tile loaded directly into LDS; the accumulators stay in
// registers for the whole segment, so the per-chunk work carries no dependency but the
// running product.
namespace rsm {

// LDS of seg_state_kernel besides the route of a round, and the largest round (a multiple of
// the 512 threads) that fits beside it in 160 KB: a segment no longer than that is routed in
// one round before its walk (no routing while the walk's registers are live).
template <int M, int C, int DT>
constexpr int seg_lds_base() {
    constexpr int MP = M > 32 ? M : 32, QP = MP + 8, psW = C * QP + 8;
    constexpr int SPL = M > 64 ? M / 64 : 1;
    return 2 * 2 * psW * 2 + 4 * ((C * DT * 2 + 1023) / 1024 * 1024) + 2 * 8 * 64 * SPL * 4;
}
template <int M, int C, int DT>
constexpr int seg_round_one() {
    constexpr int per_tok = ((M + 63) / 64) * 8 + 16 * 4;  // mask words and 16 alpha-list entries
    constexpr int r = (160 * 1024 - seg_lds_base<M, C, DT>()) / per_tok / 512 * 512;
    return r > 512 ? r : 512;
}

// DENSE (K = M, default router): no routing; each wave forms its tokens' alphas from z and f
// (loaded two steps ahead like k), and the grid has no route-only workgroups.
template <int M, int C, int DT, bool ONE, bool DENSE = false>
__global__ __launch_bounds__(512) void seg_state_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                        const bf16_t* __restrict__ z, const float* __restrict__ f,
                                                        long T_len, int Hh, int Dv, int K, SegArgs sg,
                                                        unsigned long long* __restrict__ rmask,
                                                        float* __restrict__ ralpha, int32_t* __restrict__ idx_out) {
    typedef Pol<bf16_t> P;
    typedef P::frag frag;
    typedef P::dfrag dfrag;
    static_assert(C == 32 || C == 64, "chunk length");
    constexpr int NW = 8, NT = 64 * NW;
    constexpr int KB = P::KB, NPL = P::NPL;
    constexpr int MP = M > KB ? M : KB;       // padded slot dimension of a W row
    constexpr int QP = MP + 8;                // W row pitch (elements)
    constexpr int psW = C * QP + 8;           // W plane stride
    constexpr int SPL = M > 64 ? M / 64 : 1;  // slots per lane
    constexpr int MW = (M + 63) / 64;         // mask words per token
    constexpr int TPW = C / NW;               // tokens per wave in a chunk
    constexpr int R = ONE ? seg_round_one<M, C, DT>() : NT;  // tokens per routing round
    constexpr int NTM = M / 16, NTD = DT / 16, NKC = C / KB;
    constexpr int NOT = NTM * NTD;             // 16x16 output tiles of U
    constexpr int NPT = (NOT + NW - 1) / NW;   // output tiles per wave, at most
    constexpr int GV = DT * 2 / 16;            // 16-byte granules per v row
    static_assert(R % C == 0 && M <= 128 && DT <= 128, "shape");

    __shared__ __align__(16) unsigned long long sMask[R * MW];  // token-major route of a round
    __shared__ __align__(16) float sList[R * 16];
    __shared__ __align__(16) bf16_t sW0[NPL * psW];  // W hi / lo planes, even steps
    __shared__ __align__(16) bf16_t sW1[NPL * psW];  // odd steps
    __shared__ __align__(16) bf16_t rv0[pad1k(C * DT * 2) / 2];  // v tiles: a ring of four
    __shared__ __align__(16) bf16_t rv1[pad1k(C * DT * 2) / 2];
    __shared__ __align__(16) bf16_t rv2[pad1k(C * DT * 2) / 2];
    __shared__ __align__(16) bf16_t rv3[pad1k(C * DT * 2) / 2];
    __shared__ __align__(16) float sB0[NW * 64 * SPL];  // block products, [wave][slot], even steps
    __shared__ __align__(16) float sB1[NW * 64 * SPL];  // odd steps

    const int nseg = sg.S - 1;
    // nseg segment workgroups per head, + 1 routing one (not in dense mode)
    const long heads = long(gridDim.x) / (DENSE ? nseg : sg.S);
    const long nblk = heads * nseg;
    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q4 = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const long T_pad = sg.nC * C;
    const long seglen = long(sg.cps) * C;

    // heads on XCDs as in the second pass: workgroups are dealt to the 8 XCDs round-robin, and
    // the second pass gives XCD x the heads [x*heads/8, (x+1)*heads/8), so the route and the
    // segment states it reads were written through the same L2
    const bool xmap = nblk % 8 == 0 && heads % 8 == 0;
    if (!DENSE && long(blockIdx.x) >= nblk) {  // route the last segment of one head (read by the second pass only)
        const long r = long(blockIdx.x) - nblk;
        const long bh = xmap ? (r % 8) * (heads / 8) + r / 8 : r;
        const long hb = bh / Hh, hh = bh % Hh;
        for (long t = long(nseg) * seglen + tid; t < T_len; t += NT)
            route_row<bf16_t, M, true, true>(z, f, (hb * T_len + t) * Hh + hh, bh, t, T_pad, K, C, idx_out, nullptr,
                                             rmask, ralpha);
        return;
    }
    const long id = xmap ? (long(blockIdx.x) % 8) * (nblk / 8) + long(blockIdx.x) / 8 : long(blockIdx.x);
    const long bh = id / nseg;
    const int seg = int(id % nseg);
    const long hb = bh / Hh, hh = bh % Hh;
    const long t_lo = long(seg) * seglen, t_hi = t_lo + seglen;  // segments but the last are full
    const long rstride = long(Hh);
    const long rowbase = hb * T_len * rstride + hh;  // token-head row of token 0 is rowbase + t * rstride

    // ---- direct loads of a v chunk tile, rows in token order
    const long v_pitch = rstride * Dv * 2;
    TileDma<int(sizeof(rv0)), DT * 2, NW, 2> dv;
    dv.init(w, lane, v_pitch);
    const bf16_t* vbase = v + rowbase * Dv;
    auto issue_v = [&](long c, bf16_t* dst) __attribute__((always_inline)) {
        dv.issue(dst, reinterpret_cast<const char*>(vbase + c * C * rstride * Dv), w, lane, C, v_pitch);
    };
    // ---- k of this wave's tokens of chunk c, lane = slot (0 for lanes past M)
    const uint16_t* kb16 = reinterpret_cast<const uint16_t*>(k) + rowbase * M;
    auto load_k = [&](long c, float (&kx)[TPW][SPL]) __attribute__((always_inline)) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
#pragma unroll
        for (int e = 0; e < TPW; ++e) {
            const long t = c * C + w * TPW + e;
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = lane + 64 * r;
                const uint16_t x = kb16[t * rstride * M + (slot < M ? slot : M - 1)];
                kx[e][r] = slot < M ? __uint_as_float(uint32_t(x) << 16) : 0.0f;
            }
        }
    };

    floatx4 acc[NPT];
#pragma unroll
    for (int p = 0; p < NPT; ++p) acc[p] = floatx4{0.f, 0.f, 0.f, 0.f};
    float carry[SPL];  // product of alpha over the chunks after the current one (within the segment)
#pragma unroll
    for (int r = 0; r < SPL; ++r) carry[r] = 1.0f;
    float al[2][TPW][SPL], rl[2][TPW][SPL];  // this wave's alphas and in-block exclusive suffix products
    float kx[4][TPW][SPL];                    // k of this wave's tokens, one set per step modulo 4
    // dense mode: z of this wave's tokens and f (lane e % TPW holds token e's), per step modulo 4
    float zx[DENSE ? 4 : 1][TPW][SPL], fx[DENSE ? 4 : 1];
    const uint16_t* zb16 = reinterpret_cast<const uint16_t*>(z) + rowbase * M;
    auto load_zf = [&](long c, float (&zc)[TPW][SPL], float& fc) __attribute__((always_inline)) {
#pragma unroll
        for (int e = 0; e < TPW; ++e) {
            const long t = c * C + w * TPW + e;
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = lane + 64 * r;
                const uint16_t x = zb16[t * rstride * M + (slot < M ? slot : M - 1)];
                zc[e][r] = __uint_as_float(uint32_t(x) << 16);
            }
        }
        fc = f[rowbase + (c * C + w * TPW + (lane % TPW)) * rstride];
    };

    // W rows past the slot count stay zero (never read); clear once
    for (int i = tid; i < int(sizeof(sW0)) / 16; i += NT) {
        reinterpret_cast<uint4*>(sW0)[i] = make_uint4(0u, 0u, 0u, 0u);
        reinterpret_cast<uint4*>(sW1)[i] = make_uint4(0u, 0u, 0u, 0u);
    }

    // ---- route the round of tokens [rl0, rl0 + rn): global route for the second pass and a
    // token-major copy in LDS
    long rl0 = 0;
    auto route_round = [&](long lo, long n) __attribute__((always_inline)) {
        rl0 = lo;
        for (int tr = tid; tr < n; tr += NT) {
            const long t = lo + tr;
            route_row<bf16_t, M, true, true, true>(z, f, rowbase + t * rstride, bh, t, T_pad, K, C, idx_out, nullptr,
                                                   rmask, ralpha, sMask + tr * MW, sList + tr * K);
        }
        wait_vm<0>();
        __syncthreads();
    };

    // ---- phase 1 of chunk c: alphas of this wave's tokens and their in-block suffix products;
    // the block product goes to sB
    auto phase1 = [&](auto nb, long c, const float (&zc)[TPW][SPL], float fc) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb)::value;
        float* sB = NB ? sB1 : sB0;
        float a[TPW][SPL];
        bool sel[TPW][SPL];
        if constexpr (DENSE) {  // every slot: alpha = exp(sigmoid(z) f), as the router forms it
#pragma unroll
            for (int e = 0; e < TPW; ++e) {
                const float fe = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fc), e));  // token e's f
#pragma unroll
                for (int r = 0; r < SPL; ++r) {
                    const float sc = sigmoidf_dev(zc[e][r]);
                    sel[e][r] = true;
                    a[e][r] = sc > 0.0f ? __expf(sc * fe) : 1.0f;
                }
            }
        } else {
        const int tl0 = int(c * C - rl0) + w * TPW;  // round-local index of this wave's first token
        // every LDS read first (masks, then the list entries), then the arithmetic
        unsigned long long m[TPW][MW];
#pragma unroll
        for (int e = 0; e < TPW; ++e)
#pragma unroll
            for (int wd = 0; wd < MW; ++wd) m[e][wd] = sMask[(tl0 + e) * MW + wd];
#pragma unroll
        for (int e = 0; e < TPW; ++e)
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const unsigned long long mw = m[e][MW > 1 ? r : 0];
                const int below = (r == 1 ? __popcll(m[e][0]) : 0) + mbcnt64(mw);
                sel[e][r] = (mw >> lane) & 1ull;
                a[e][r] = sList[(tl0 + e) * K + (below < K ? below : K - 1)];
            }
        }
        float run[SPL];
#pragma unroll
        for (int r = 0; r < SPL; ++r) run[r] = 1.0f;
#pragma unroll
        for (int e = TPW - 1; e >= 0; --e)
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                al[NB][e][r] = sel[e][r] ? a[e][r] : 1.0f;
                rl[NB][e][r] = run[r];
                run[r] *= al[NB][e][r];
            }
#pragma unroll
        for (int r = 0; r < SPL; ++r) sB[w * 64 * SPL + 64 * r + lane] = run[r];
    };

    // ---- phase 2 of chunk c into W buffer NB: W = (1 - alpha) k R as hi / lo bf16 rows
    auto phase2 = [&](auto nb, const float (&kc)[TPW][SPL]) __attribute__((always_inline)) {
        constexpr int NB = decltype(nb)::value;
        bf16_t* sW = NB ? sW1 : sW0;
        const float* sB = NB ? sB1 : sB0;
        // fw: product over the later blocks of this chunk and the later chunks; the new carry
        // (every wave forms it in the same order, so the copies agree bit for bit)
        float fw[SPL], all[SPL];
#pragma unroll
        for (int r = 0; r < SPL; ++r) {
            float after = 1.0f, whole = 1.0f;
#pragma unroll
            for (int u = 0; u < NW; ++u) {
                const float b = sB[u * 64 * SPL + 64 * r + lane];
                whole *= b;
                if (u > w) after *= b;
            }
            fw[r] = carry[r] * after;
            all[r] = carry[r] * whole;
        }
        uint16_t* hi = reinterpret_cast<uint16_t*>(sW);
#pragma unroll
        for (int e = 0; e < TPW; e += 2) {
#pragma unroll
            for (int r = 0; r < SPL; ++r) {
                const int slot = lane + 64 * r;
                const float x0 = (1.0f - al[NB][e][r]) * kc[e][r] * (rl[NB][e][r] * fw[r]);
                const float x1 = (1.0f - al[NB][e + 1][r]) * kc[e + 1][r] * (rl[NB][e + 1][r] * fw[r]);
                uint32_t lo;
                const uint32_t h = P::split2(x0, x1, lo);
                if (slot < M) {
                    const int off = (w * TPW + e) * QP + slot;
                    hi[off] = uint16_t(h);
                    hi[psW + off] = uint16_t(lo);
                    hi[off + QP] = uint16_t(h >> 16);
                    hi[psW + off + QP] = uint16_t(lo >> 16);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < SPL; ++r) carry[r] = all[r];
    };

    // ---- U += W^T V of the chunk in buffer NB: wave w takes output tiles w, w + 8, ...
    auto mfma = [&](auto ph) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph)::value;  // step modulo 4: W buffer PH % 2, v buffer PH
        const bf16_t* sW = (PH & 1) ? sW1 : sW0;
        const bf16_t* rvc = PH == 0 ? rv0 : PH == 1 ? rv1 : PH == 2 ? rv2 : rv3;
        // all fragments first, then the MFMAs (independent accumulators interleaved)
        constexpr bool SAME_D = NTD % NW == 0;  // every tile of a wave has column tile w % NTD
        dfrag wf[NPT][NKC];
        frag va[SAME_D ? 1 : NPT][NKC];
#pragma unroll
        for (int p = 0; p < NPT; ++p) {
            const int pt = w + NW * p;
            if (NOT % NW == 0 || pt < NOT) {
                const int I = pt / NTD, D = pt % NTD;
#pragma unroll
                for (int kb = 0; kb < NKC; ++kb) {
#pragma unroll
                    for (int pl = 0; pl < NPL; ++pl)
                        wf[p][kb].p[pl] = P::template ld_col<true>(sW, pl * psW + 16 * I, QP, kb, q4, l16);
                    if (!SAME_D || p == 0) va[SAME_D ? 0 : p][kb] = P::template ld_col_swz<true, GV, 2>(rvc, 0, 16 * D, kb, q4, l16);
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < NKC; ++kb)
#pragma unroll
            for (int pl = NPL - 1; pl >= 0; --pl)
#pragma unroll
                for (int p = 0; p < NPT; ++p) {
                    const int pt = w + NW * p;
                    if (NOT % NW == 0 || pt < NOT)
                        acc[p] = P::mma(wf[p][kb].p[pl], va[SAME_D ? 0 : p][kb], acc[p]);
                }
    };

    // ---- the walk, one barrier per step.  Step s runs, for c = c_last - s, the MFMAs of chunk
    // c+2, phase 2 of chunk c+1 and phase 1 of chunk c, and issues the loads two steps ahead:
    // v of chunk c (read at step s+2, ring buffer (s+2) % 4) and k of chunk c-1 (read at step
    // s+2, register set (s+2) % 4).  The loads are unconditional (indices clamped to the
    // segment), so no branch splits the count of loads in flight.
    const long c_first = t_lo / C, c_last = t_hi / C - 1;
    const long nsteps = c_last - c_first + 1;
    constexpr int NI = (int(sizeof(rv0)) / 1024 + NW - 1) / NW;  // direct-load instructions of a v tile, at most
    constexpr bool EVEN = int(sizeof(rv0)) % (1024 * NW) == 0;    // every wave issues exactly NI of them
    // start of the round holding chunk c (rounds are cut from the segment end)
    auto round_lo = [&](long c) __attribute__((always_inline)) {
        const long back = (t_hi - c * C - 1) / R;  // rounds after the one holding chunk c
        const long lo = t_hi - (back + 1) * R;
        return lo > t_lo ? lo : t_lo;
    };
    auto step = [&](auto ph, long s) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph)::value;  // s % 4
        const long c = c_last - s;
        if constexpr (!ONE && !DENSE)
            if (s > 0 && s < nsteps && c * C + C == rl0) route_round(round_lo(c), rl0 - round_lo(c));  // next round
        const long cv = c > c_first ? c : c_first, ck = c - 1 > c_first ? c - 1 : c_first;
        constexpr int PV = (PH + 2) & 3;
        issue_v(cv, PV == 0 ? rv0 : PV == 1 ? rv1 : PV == 2 ? rv2 : rv3);
        load_k(ck, kx[PV]);
        if constexpr (DENSE) {  // z and f of chunk c-2, read by its phase 1 at step s+2
            const long cz = c - 2 > c_first ? c - 2 : c_first;
            load_zf(cz, zx[PV], fx[PV]);
        }
        if (s >= 2 && s <= nsteps + 1) mfma(ph);
        if (s >= 1 && s <= nsteps) phase2(std::integral_constant<int, (PH + 1) & 1>{}, kx[PH]);
        if (s < nsteps) phase1(std::integral_constant<int, PH & 1>{}, c, zx[DENSE ? PH : 0], fx[DENSE ? PH : 0]);
        // what this step issued may stay in flight; everything before it has landed
        constexpr int NV = NI + TPW * SPL + (DENSE ? TPW * SPL + 1 : 0);  // vector loads issued this step
        if constexpr (EVEN) wait_vm<NV>();
        else wait_vm<0>();
        wg_barrier();
    };

    if constexpr (DENSE) {
        load_zf(c_last, zx[0], fx[0]);                                      // read at step 0
        load_zf(c_last - 1 > c_first ? c_last - 1 : c_first, zx[1], fx[1]);  // read at step 1
    } else {
        route_round(round_lo(c_last), t_hi - round_lo(c_last));
    }
    load_k(c_last, kx[1]);  // read at step 1
    for (long s = 0; s < nsteps + 2; s += 4) {
        step(std::integral_constant<int, 0>{}, s);
        step(std::integral_constant<int, 1>{}, s + 1);
        step(std::integral_constant<int, 2>{}, s + 2);
        step(std::integral_constant<int, 3>{}, s + 3);
    }
    wait_vm<0>();  // no direct load may land after the workgroup has left

    // ---- outputs: dH_s and E_s
    const long segrow = (bh * nseg + seg) * M;
    float* dst = sg.dH + segrow * Dv;
#pragma unroll
    for (int p = 0; p < NPT; ++p) {
        const int pt = w + NW * p;
        if (NOT % NW == 0 || pt < NOT) {
            const int I = pt / NTD, D = pt % NTD;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[long(16 * I + 4 * q4 + r) * Dv + 16 * D + l16] = acc[p][r];
        }
    }
    if (w == 0) {
#pragma unroll
        for (int r = 0; r < SPL; ++r)
            if (lane + 64 * r < M) sg.dE[segrow + lane + 64 * r] = carry[r];
    }
}

}  // namespace rsm
