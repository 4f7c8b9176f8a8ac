// gdr2_bwd.hip -- gate-aware backward of the chunked Gated Delta Rule-2 layer (gfx950).
//
// The ainews.random.gg article on Gated DeltaNet-2, section "Chunkwise training and gate-aware
// backward", notes that KDA's scalar shortcut no longer applies: the erase and write gates are
// different diagonal gates on the key and value channels, so they appear inside the dot products
// that accumulate gradients.  Written out for one chunk (forward: Delta = U - Y S,
// O = Qbar S + P Delta, S' = Diag(gamma) S + Ktilde^T Delta; see gdr2_fwd.hip), with dS' the
// gradient of the state leaving the chunk:
//     dDelta = Ktilde dS' + P^T dO
//     dS     = Diag(gamma) dS' + Qbar^T dO - Y^T dDelta          (passed to the previous chunk)
//     dX     = T^T dDelta,  X = Z - Ebar S = T^-1 Delta            (dZ = dX: dv = dX . w, dw = dX . v)
//     dA     = strict_lower(-dX Delta^T),   dP = lower(dO Delta^T)
//     dQbar  = dO S^T + dP Kbar,  dEbar = -dX S^T + dA Kbar,  dKbar = dP^T Qbar + dA^T Ebar,
//     dKtilde = Delta dS'^T,  dgamma_i = sum_j dS'_ij S_ij
// and the chain rule through Qbar = q e^G, Ebar = (b . k) e^G, Kbar = k e^-G,
// Ktilde = k e^{G_C - G}, gamma = e^{G_C}, G = in-chunk cumsum of log alpha.
//
// Kernels:
//   gdr2_dstate_kernel  sequential over chunks in reverse, one workgroup per (chain, value slice):
//                       the dS carry; writes the gradient of every chunk's exit state and dS0.
//   gdr2_bgrad_kernel   one workgroup per (chain, chunk), all chunks in parallel: every input
//                       gradient of the chunk (see the comment above the kernel).
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"
#include "gdr2_wy.hpp"

namespace gdr2 {

template <typename OT, int DK, int DVS>
struct DsCfg {
    static constexpr int C = kChunk;
    static constexpr int KS = Mfma<OT>::KS;
    static constexpr int ES = (int)sizeof(OT);
    static constexpr int PAD = 16 / ES;
    static constexpr int PK = DK + PAD, PC = C + PAD, PO = DVS + PAD;
    static constexpr int NKS = DK / KS, NCK = C / KS;
    static constexpr int NJB = DVS / 16, NIB = DK / 16;
    static constexpr int BPW = NIB * NJB / kWaves;
    static constexpr int VEC = 16 / ES;
    static constexpr int KVEC = C * DK * ES / 16 / kThreads;   // [C][DK] tile, vectors per thread
    static constexpr int PVEC = (C * C * ES / 16 + kThreads - 1) / kThreads;
    static constexpr int NOV = C * DVS * ES / 16;                // [C][DVS] slice, vectors
    static constexpr int OVEC = (NOV + kThreads - 1) / kThreads;
    static_assert(BPW >= 1 && BPW * kWaves == NIB * NJB, "state block mapping");
};

template <typename OT, int DK, int DVS>
struct alignas(16) DsSmem {
    using Cf = DsCfg<OT, DK, DVS>;
    OT Qt[kChunk * Cf::PK];   // Qbar                      [r][i]
    OT Yt[kChunk * Cf::PK];   // -Y                        [r][i]
    OT Pt[kChunk * Cf::PC];   // P                         [r][s]
    OT dOt[kChunk * Cf::PO];  // dO slice                  [r][j]
    OT dST[DVS * Cf::PK];     // dS^T operand copy         [j][i]
    OT dDT[DVS * Cf::PC];     // dDelta^T                  [j][r]
    float gam[DK];
};

template <typename OT, int DK, int DVS>
__global__ __launch_bounds__(kThreads, 1) void gdr2_dstate_kernel(BwdParams p) {
    using Cf = DsCfg<OT, DK, DVS>;
    using MM = Mfma<OT>;
    using FR = Frag<OT>;
    constexpr int C = kChunk, KS = Cf::KS, PK = Cf::PK, PC = Cf::PC, PO = Cf::PO;
    constexpr int NKS = Cf::NKS, NCK = Cf::NCK, NJB = Cf::NJB, BPW = Cf::BPW;
    constexpr int VEC = Cf::VEC, KVEC = Cf::KVEC, PVEC = Cf::PVEC, NOV = Cf::NOV, OVEC = Cf::OVEC;
    __shared__ DsSmem<OT, DK, DVS> sm;

    const int tid = threadIdx.x, R = wave_id(), l = lane_id();
    const int work = xcd_swizzle(blockIdx.x, gridDim.x);
    const int chain = work / p.NS, slice = work % p.NS;
    const int bb = chain / p.H, h = chain % p.H;
    const int j0 = slice * DVS;
    const long T = p.T, H = p.H, DV = p.DV;
    const int NC = p.NC;
    const OT* dO = (const OT*)p.dO + ((long)bb * T * H + h) * DV + j0;

    f32x4 dS[BPW];
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
        const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v = 0.f;
            if (p.dST) v = p.dST[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()];
            dS[u][e] = v;
        }
        store_acc_T(sm.dST, PK, 16 * jb, 16 * ib, dS[u]);
    }

    struct Buf {
        typename FR::t K[NKS];
        i32x4 Q[KVEC], Y[KVEC], P[PVEC], O[OVEC];
        f32x4 g;
    };
    auto fetch = [&](Buf& b, int cc) __attribute__((always_inline)) {
        const long cix = (long)chain * NC + cc;
        const OT* Kc = (const OT*)p.wy.Kt + cix * C * DK;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) b.K[ks] = FFrag<OT>::fkc(Kc, DK, 16 * R, ks * KS);
        const OT* Qc = (const OT*)p.wy.Qg + cix * C * DK;
        const OT* Yc = (const OT*)p.wy.Yh + cix * C * DK;
#pragma unroll
        for (int m = 0; m < KVEC; ++m) {
            b.Q[m] = *(const i32x4*)(Qc + (long)(tid + m * kThreads) * VEC);
            b.Y[m] = *(const i32x4*)(Yc + (long)(tid + m * kThreads) * VEC);
        }
        const OT* Pc = (const OT*)p.wy.P + cix * C * C;
#pragma unroll
        for (int m = 0; m < PVEC; ++m) {
            const int x = tid + m * kThreads;
            if (x < C * C / VEC) b.P[m] = *(const i32x4*)(Pc + (long)x * VEC);
        }
#pragma unroll
        for (int m = 0; m < OVEC; ++m) {
            const int x = tid + m * kThreads;
            const int rr = (x * VEC) / DVS, jj = (x * VEC) % DVS;
            const long t = (long)cc * C + rr;
            i32x4 z = {0, 0, 0, 0};
            if (x < NOV && t < T) z = *(const i32x4*)(dO + t * H * DV + jj);
            b.O[m] = z;
        }
        if (tid < DK / 4) b.g = *(const f32x4*)(p.wy.gam + cix * DK + 4 * tid);
    };
    auto chunk = [&](const Buf& cur, Buf& nxt, int c) __attribute__((always_inline)) {
        // ---- stage the chunk's factors and dO slice, checkpoint dS' of this chunk
#pragma unroll
        for (int m = 0; m < KVEC; ++m) {  // fragment order -> row-major
            const int x = tid + m * kThreads;
            const int o = FLay<OT>::unit_row(x, DK) * PK + FLay<OT>::unit_col(x, DK);
            *(i32x4*)(sm.Qt + o) = cur.Q[m];
            *(i32x4*)(sm.Yt + o) = cur.Y[m];
        }
#pragma unroll
        for (int m = 0; m < PVEC; ++m) {
            const int x = tid + m * kThreads;
            if (x < C * C / VEC)
                *(i32x4*)(sm.Pt + FLay<OT>::unit_row(x, C) * PC + FLay<OT>::unit_col(x, C)) = cur.P[m];
        }
#pragma unroll
        for (int m = 0; m < OVEC; ++m) {
            const int x = tid + m * kThreads;
            if (x < NOV) *(i32x4*)(sm.dOt + ((x * VEC) / DVS) * PO + (x * VEC) % DVS) = cur.O[m];
        }
        if (tid < DK / 4) *(f32x4*)(sm.gam + 4 * tid) = cur.g;
        if (c > 0) fetch(nxt, c - 1);
        {
            OT* dst = (OT*)p.dSx + (((long)chain * NC + c) * DV + j0) * DK;
            constexpr int NSV = DVS * DK / VEC;
#pragma unroll
            for (int x0 = 0; x0 < NSV; x0 += kThreads) {
                const int x = x0 + tid;
                if (NSV % kThreads == 0 || x < NSV) {
                    const int j = (x * VEC) / DK, i = (x * VEC) % DK;
                    *(i32x4*)(dst + (long)j * DK + i) = *(const i32x4*)(sm.dST + j * PK + i);
                }
            }
        }
        lds_barrier();
        // ---- dDelta = Ktilde dS' + P^T dO   (wave R: token block R)
        {
            f32x4 aD[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) aD[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) MM::mma(aD[jb], cur.K[ks], FR::kc(sm.dST, PK, 16 * jb, ks * KS));
#pragma unroll
            for (int kk = 0; kk < NCK; ++kk) {
                if (kk * KS + KS > 16 * R) {  // P^T is upper triangular: s >= r
                    typename FR::t a = FR::tr(sm.Pt, PC, kk * KS, 16 * R);
#pragma unroll
                    for (int jb = 0; jb < NJB; ++jb) MM::mma(aD[jb], a, FR::tr(sm.dOt, PO, kk * KS, 16 * jb));
                }
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) store_acc_T(sm.dDT, PC, 16 * jb, 16 * R, aD[jb]);
        }
        lds_barrier();
        // ---- dS <- Diag(gamma) dS' + Qbar^T dO + (-Y)^T dDelta
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[u][e] *= sm.gam[16 * ib + acc_row(e)];
#pragma unroll
            for (int kk = 0; kk < NCK; ++kk) {
                MM::mma(dS[u], FR::tr(sm.Qt, PK, kk * KS, 16 * ib), FR::tr(sm.dOt, PO, kk * KS, 16 * jb));
                MM::mma(dS[u], FR::tr(sm.Yt, PK, kk * KS, 16 * ib), FR::kc(sm.dDT, PC, 16 * jb, kk * KS));
            }
            store_acc_T(sm.dST, PK, 16 * jb, 16 * ib, dS[u]);
        }
        lds_barrier();
    };

    Buf bA, bB;
    if (NC > 0) fetch(bA, NC - 1);
    lds_barrier();
    for (int c = NC - 1; c >= 0; c -= 2) {
        chunk(bA, bB, c);
        if (c - 1 >= 0) chunk(bB, bA, c - 1);
    }
    if (p.dS0) {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.dS0[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()] = dS[u][e];
        }
    }
}

// --------------------------------------------------------------------------------------------
// State-gradient carry with loader waves (16-bit operands), the backward twin of
// gdr2_carry_lds_kernel: waves 0-3 compute (wave R owns token block R) and write the dS'
// checkpoints, waves 4-7 stream the factors and the dO slice of chunk c - 1 into the other LDS
// slot (loaded two steps ahead into their registers) while chunk c computes.
template <int DK, int DVS>
struct DsLCfg {
    static constexpr int C = kChunk, KS = 32;
    static constexpr int PK = DK + 8, PC = C + 8, PO = DVS + 8;
    static constexpr int NKS = DK / KS, NCK = C / KS, NJB = DVS / 16, NIB = DK / 16;
    static constexpr int BPW = NIB * NJB / kWaves;
    // slot layout (bf16 elements): Q, Y, K [C][DK] and P [C][C] in fragment order, then the dO
    // slice [C][PO] (row-major, padded)
    static constexpr int OQ = 0, OY = C * DK, OK = 2 * C * DK, OP = 3 * C * DK, OO = OP + C * C;
    static constexpr int SLOT = OO + C * PO;
    // 16-byte units of one chunk: Q, Y, K, P (contiguous in the slot), dO rows, gamma
    static constexpr int UM = C * DK / 8, UP = C * C / 8, UO = C * DVS / 8, UG = DK / 4;
    static constexpr int NUNIT = 3 * UM + UP + UO + UG;
    static constexpr int LPT = (NUNIT + kThreads - 1) / kThreads;
    static_assert(BPW >= 1 && BPW * kWaves == NIB * NJB, "state block mapping");
};

template <int DK, int DVS>
struct alignas(16) DsLSmem {
    using Cf = DsLCfg<DK, DVS>;
    bf16 slot[2][Cf::SLOT];
    float gam[2][DK];
    bf16 dST[DVS * Cf::PK];   // dS^T operand copy   [j][i]
    bf16 dDT[DVS * Cf::PC];   // dDelta^T            [j][r]
};

template <int DK, int DVS>
__global__ __launch_bounds__(2 * kThreads, 1) void gdr2_dstate_lds_kernel(BwdParams p) {
    using Cf = DsLCfg<DK, DVS>;
    using MM = Mfma<bf16>;
    using FR = Frag<bf16>;
    using FF = FFrag<bf16>;
    constexpr int C = kChunk, KS = Cf::KS, PK = Cf::PK, PC = Cf::PC, PO = Cf::PO;
    constexpr int NKS = Cf::NKS, NCK = Cf::NCK, NJB = Cf::NJB, BPW = Cf::BPW, LPT = Cf::LPT;
    __shared__ DsLSmem<DK, DVS> sm;

    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const bool loader = w >= kWaves;
    const int R = w & 3, lt = tid & (kThreads - 1);
    const int work = xcd_swizzle(blockIdx.x, gridDim.x);
    const int chain = work / p.NS, slice = work % p.NS;
    const int bb = chain / p.H, h = chain % p.H;
    const int j0 = slice * DVS;
    const long T = p.T, H = p.H, DV = p.DV;
    const int NC = p.NC, c0 = p.c0, NR = p.ncr;  // chunks [c0, c0 + NR) of NC, walked backwards
    const int cl = c0 + NR - 1;                   // from the range's last chunk
    const bf16* dO = (const bf16*)p.dO + ((long)bb * T * H + h) * DV + j0;

    // ---- loader units of chunk cc (the region of unit lt + kThreads * m depends on m only)
    auto src_unit = [&](int cc, int m) __attribute__((always_inline)) -> const i32x4* {
        const long cix = (long)chain * NC + cc;
        int x = lt + kThreads * m;
        if (x >= Cf::NUNIT) x = Cf::NUNIT - 1;
        if (x < 3 * Cf::UM) {
            const int mat = x / Cf::UM, u = x % Cf::UM;
            const bf16* base = mat == 0 ? (const bf16*)p.wy.Qg : mat == 1 ? (const bf16*)p.wy.Yh : (const bf16*)p.wy.Kt;
            return (const i32x4*)(base + cix * C * DK + u * 8);
        }
        x -= 3 * Cf::UM;
        if (x < Cf::UP) return (const i32x4*)((const bf16*)p.wy.P + cix * C * C + x * 8);
        x -= Cf::UP;
        if (x < Cf::UO) {
            const int rr = x / (DVS / 8), c8 = x % (DVS / 8);
            const long t = (long)cc * C + rr < T ? (long)cc * C + rr : T - 1;  // zeroed when put
            return (const i32x4*)(dO + t * H * DV + 8 * c8);
        }
        x -= Cf::UO;
        return (const i32x4*)(p.wy.gam + cix * DK + 4 * x);
    };
    auto put_unit = [&](int sl, int cc, int m, const i32x4& v) __attribute__((always_inline)) {
        int x = lt + kThreads * m;
        if (x >= Cf::NUNIT) return;
        if (x < 3 * Cf::UM + Cf::UP) {
            *(i32x4*)(sm.slot[sl] + x * 8) = v;
            return;
        }
        x -= 3 * Cf::UM + Cf::UP;
        if (x < Cf::UO) {
            const int rr = x / (DVS / 8), c8 = x % (DVS / 8);
            const i32x4 z = {0, 0, 0, 0};
            *(i32x4*)(sm.slot[sl] + Cf::OO + rr * PO + 8 * c8) = (long)cc * C + rr < T ? v : z;
            return;
        }
        x -= Cf::UO;
        *(i32x4*)(sm.gam[sl] + 4 * x) = v;
    };
    i32x4 lbA[LPT], lbB[LPT];  // loader registers; step s handles chunk cl - s

    f32x4 dS[BPW];
    if (!loader) {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float v = 0.f;
                if (p.dST) v = p.dST[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()];
                dS[u][e] = v;
            }
            store_acc_T(sm.dST, PK, 16 * jb, 16 * ib, dS[u]);
        }
    } else if (NR > 0) {
        const int a1 = NR > 1 ? cl - 1 : c0, a2 = NR > 2 ? cl - 2 : c0;
#pragma unroll
        for (int m = 0; m < LPT; ++m) lbB[m] = *src_unit(cl, m);
#pragma unroll
        for (int m = 0; m < LPT; ++m) put_unit(0, cl, m, lbB[m]);
#pragma unroll
        for (int m = 0; m < LPT; ++m) lbA[m] = *src_unit(a1, m);
#pragma unroll
        for (int m = 0; m < LPT; ++m) lbB[m] = *src_unit(a2, m);
    }
    lds_barrier();

    // loader step st: the chunk of step st + 1 (registers `cur`) into slot (st + 1) & 1, then the
    // loads of the chunk of step st + 3 (clamped to the range) into the same registers
    auto loader_step = [&](int st, i32x4* cur) __attribute__((always_inline)) {
        if (st + 1 < NR) {
#pragma unroll
            for (int m = 0; m < LPT; ++m) put_unit((st + 1) & 1, cl - 1 - st, m, cur[m]);
        }
        const int c3 = st + 3 < NR ? cl - 3 - st : c0;
#pragma unroll
        for (int m = 0; m < LPT / 2; ++m) cur[m] = *src_unit(c3, m);
        lds_barrier();
#pragma unroll
        for (int m = LPT / 2; m < LPT; ++m) cur[m] = *src_unit(c3, m);
        lds_barrier();
    };
    auto compute_step = [&](int c, int sl) __attribute__((always_inline)) {
        {   // checkpoint: gradient of the state leaving chunk c
            bf16* dst = (bf16*)p.dSx + (((long)chain * NC + c) * DV + j0) * DK;
            constexpr int NSV = DVS * DK / 8;
#pragma unroll
            for (int x0 = 0; x0 < NSV; x0 += kThreads) {
                const int x = x0 + tid;
                if (NSV % kThreads == 0 || x < NSV) {
                    const int j = (x * 8) / DK, i = (x * 8) % DK;
                    store_stream((i32x4*)(dst + (long)j * DK + i), *(const i32x4*)(sm.dST + j * PK + i));
                }
            }
        }
        const bf16* Qs = sm.slot[sl] + Cf::OQ;
        const bf16* Ys = sm.slot[sl] + Cf::OY;
        const bf16* Ks = sm.slot[sl] + Cf::OK;
        const bf16* Ps = sm.slot[sl] + Cf::OP;
        const bf16* Os = sm.slot[sl] + Cf::OO;
        // dO as a B operand (k = tokens) per (k-step, value block): read once, used by both phases
        bf16x8 ob[NCK][NJB];
#pragma unroll
        for (int kk = 0; kk < NCK; ++kk)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) ob[kk][jb] = FR::tr(Os, PO, kk * KS, 16 * jb);
        // ---- dDelta = Ktilde dS' + P^T dO   (wave R: token block R)
        {
            f32x4 aD[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) aD[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const bf16x8 ak = FF::fkc(Ks, DK, 16 * R, ks * KS);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) MM::mma(aD[jb], ak, FR::kc(sm.dST, PK, 16 * jb, ks * KS));
            }
#pragma unroll
            for (int kk = 0; kk < NCK; ++kk) {
                if (kk * KS + KS > 16 * R) {  // P^T is upper triangular: s >= r
                    const bf16x8 a = FF::ftr(Ps, C, kk * KS, 16 * R);
#pragma unroll
                    for (int jb = 0; jb < NJB; ++jb) MM::mma(aD[jb], a, ob[kk][jb]);
                }
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) store_acc_T(sm.dDT, PC, 16 * jb, 16 * R, aD[jb]);
        }
        lds_barrier();
        // ---- dS <- Diag(gamma) dS' + Qbar^T dO + (-Y)^T dDelta: dDelta^T fragments per (k-step,
        // value block) and Qbar^T, -Y^T per (key block, k-step) read once (this wave's state blocks
        // come in groups of NJB sharing one key block)
        bf16x8 ddf[NCK][NJB];
#pragma unroll
        for (int kk = 0; kk < NCK; ++kk)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) ddf[kk][jb] = FR::kc(sm.dDT, PC, 16 * jb, kk * KS);
#pragma unroll
        for (int v = 0; v < BPW / NJB; ++v) {
            const int ib = R * BPW / NJB + v;
            const f32x4 gm = *(const f32x4*)(sm.gam[sl] + 16 * ib + 4 * (l >> 4));
            bf16x8 qf[NCK], yf[NCK];
#pragma unroll
            for (int kk = 0; kk < NCK; ++kk) {
                qf[kk] = FF::ftr(Qs, DK, kk * KS, 16 * ib);
                yf[kk] = FF::ftr(Ys, DK, kk * KS, 16 * ib);
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                f32x4& acc = dS[v * NJB + jb];
                acc *= gm;
#pragma unroll
                for (int kk = 0; kk < NCK; ++kk) {
                    MM::mma(acc, qf[kk], ob[kk][jb]);
                    MM::mma(acc, yf[kk], ddf[kk][jb]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
            store_acc_T(sm.dST, PK, 16 * jb, 16 * ib, dS[u]);
        }
        lds_barrier();
    };

    const int NCR = (NR + 1) / 2 * 2;
    if (loader) {
        for (int st = 0; st < NCR; st += 2) {
            loader_step(st, lbA);
            loader_step(st + 1, lbB);
        }
    } else {
        for (int st = 0; st < NCR; st += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (st + u < NR) {
                    compute_step(cl - st - u, (st + u) & 1);
                } else {
                    lds_barrier();
                    lds_barrier();
                }
            }
        }
        if (p.dS0) {
#pragma unroll
            for (int u = 0; u < BPW; ++u) {
                const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.dS0[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()] = dS[u][e];
            }
        }
    }
}

template <int DK, int DVS>
static hipError_t launch_dstate_lds(const BwdParams& p, hipStream_t s) {
    const long nblk = (long)p.B * p.H * p.NS;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((gdr2_dstate_lds_kernel<DK, DVS>), dim3(nblk), dim3(2 * kThreads), 0, s, p);
    return hipGetLastError();
}

template <typename OT, int DK, int DVS>
static hipError_t launch_dstate(const BwdParams& p, hipStream_t s) {
    const long nblk = (long)p.B * p.H * p.NS;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((gdr2_dstate_kernel<OT, DK, DVS>), dim3(nblk), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t dstate_dispatch(int bf, int dk, int dvs, const BwdParams& p, hipStream_t s) {
    if (bf) {
        if (dk == 128 && dvs == 32) return launch_dstate_lds<128, 32>(p, s);
        if (dk == 128 && dvs == 16) return launch_dstate_lds<128, 16>(p, s);
        if (dk == 64 && dvs == 64) return launch_dstate_lds<64, 64>(p, s);
        if (dk == 64 && dvs == 32) return launch_dstate_lds<64, 32>(p, s);
        if (dk == 64 && dvs == 16) return launch_dstate_lds<64, 16>(p, s);
    } else {
        if (dk == 128 && dvs == 32) return launch_dstate<float, 128, 32>(p, s);
        if (dk == 128 && dvs == 16) return launch_dstate<float, 128, 16>(p, s);
        if (dk == 64 && dvs == 32) return launch_dstate<float, 64, 32>(p, s);
        if (dk == 64 && dvs == 16) return launch_dstate<float, 64, 16>(p, s);
    }
    return hipErrorInvalidValue;
}

// --------------------------------------------------------------------------------------------
// Chunk gradients: one workgroup (8 waves) per (chain, chunk), all chunks in parallel.  Given the
// state S entering the chunk (forward checkpoint), the gradient dS' of the state leaving it (the
// state-carry kernel above) and dO, it recomputes Delta, dDelta and dX for DVH value columns at a
// time and reduces over the value columns in MFMA accumulators (held transposed, channel x token):
//     R1 = S dO^T,  R2 = S dX^T,  R3 = dS' Delta^T,   R4 = dO Delta^T,  R5 = dX Delta^T,
//     R6_i = sum_j dS'_ij S_ij.
// dP = lower(R4) and dA = -strict_lower(R5) then meet the decay-absorbed key factors in the
// blocked Gram gradients (same per-16-token-block references as the forward):
//     G1 = dP Kbar,  G2 = dA Kbar,  G3 = dP^T Qbar + dA^T Ebar.
// Wave w = (R, half): token block R = w % 4, key-channel half = w / 4.  Lane = token row
// r = 16R + l%16 with key channels 16 ib + 4 (l/16) + e for the half's ib: the DPP row scans
// over the 16 tokens of a block give G and the in-chunk reverse cumsum of dG (dlog alpha).
constexpr int kBgThreads = 512;

template <typename OT, int DK, int DV, int DVH>
struct BgCfg {
    static constexpr int C = kChunk;
    static constexpr int KS = Mfma<OT>::KS, KPL = Mfma<OT>::KPL;
    static constexpr int ES = (int)sizeof(OT);
    static constexpr int PAD = 16 / ES;
    // key-indexed tiles (-Y, Ktilde, S, dS' and the Gram-phase tiles) padded by 32 bytes per row in
    // the 16-bit path: their transposed 8-byte reads conflict less in the LDS banks than with 16
    // bytes (bgrad 436 -> 426 us at B=4 T=4096 H=16 d=128; 48 or more bytes were slower again)
    static constexpr int PK = DK + (ES == 2 ? 2 : 1) * PAD, PC = C + PAD, PH = DVH + PAD;
    static constexpr int NKS = DK / KS, NIB = DK / 16, NIBH = NIB / 2, NJH = DVH / 16;
    static constexpr int VEC = 16 / ES;
    static constexpr int NSV = DVH * DK / VEC;   // [DVH][DK] tile, 16-byte vectors
    static constexpr int SVEC = (NSV + kBgThreads - 1) / kBgThreads;
    static constexpr int NOV = C * DVH / VEC;    // [C][DVH] tile, 16-byte vectors
    static constexpr int OVEC = (NOV + kBgThreads - 1) / kBgThreads;
    static constexpr int NTV = C * C / VEC;      // [C][C] tile
    static constexpr int TVEC = (NTV + kBgThreads - 1) / kBgThreads;
    static_assert((C * DK / VEC) % kBgThreads == 0, "Y / Ktilde staging");
    static constexpr bool YK_LDS = ES == 2;
    static constexpr int NBUF = ES == 2 ? 2 : 1;  // value-column block buffers (fp32: LDS-bound)
    // The gradients leave through LDS as whole token rows (dv, dw and dlog alpha on the 16-bit
    // path, dq, dk and db on every path), written with streaming stores: whole cache lines per
    // instruction go past the L2, so the kernels that follow do not write back this kernel's
    // dirty lines (at B=4 T=4096 H=16 d=128 the next factor kernel runs 4-7 us faster; this
    // kernel is unchanged).  The lanes' own 8-byte pieces could not be streamed: the L2 has to
    // combine them into lines.
    static constexpr bool STG = ES == 2;
    // 16-bit path: v and w of a value-column block arrive like dO (16-byte pieces of token rows by
    // consecutive threads) and are staged beside it; each lane then reads its own four columns
    // from LDS (the lanes' own 8-byte pieces of 16 token rows cost the kernel about 19 us at
    // B=4 T=4096 H=16 d=128)
    static constexpr bool VW_LDS = ES == 2;
    // 16-bit path: q, k and b of the chunk are loaded the same way with the last value-column
    // block and put into the Gram tiles' places after the loop, where each lane reads back the
    // elements it later overwrites with the decay-absorbed tiles (the lanes' own 8-byte pieces
    // cost about 15 us)
    static constexpr bool QKB_LDS = ES == 2;
    static constexpr int QVEC = C * DK / VEC / kBgThreads;
    static constexpr int PV = DV + PAD, PL = DK + 4;
    static_assert(NJH == 2, "one 16-column block per wave half");
};

template <typename OT, int DK, int DV, int DVH>
struct alignas(16) BgSmem {
    using Cf = BgCfg<OT, DK, DV, DVH>;
    struct alignas(16) Gram {  // Gram-gradient phase
        OT Kb[kChunk * Cf::PK];    // k . exp(ref_S - G)  [s][i]
        OT Qb[kChunk * Cf::PK];    // q . exp(G - ref_R)  [r][i]
        OT Eb[kChunk * Cf::PK];    // e . exp(G - ref_R)  [r][i]
        OT dPT[kChunk * Cf::PC];   // dP^T                [s][r]
        OT dAT[kChunk * Cf::PC];   // dA^T                [s][r]
    };
    union {
        struct {  // value-column phase
            OT Yt[Cf::YK_LDS ? kChunk * Cf::PK : 1];  // -Y      [r][i] (16-bit operands)
            OT Kt[Cf::YK_LDS ? kChunk * Cf::PK : 1];  // Ktilde  [r][i]
            OT Tt[kChunk * Cf::PC];    // T                   [r][s]
            OT Pt[kChunk * Cf::PC];    // P                   [r][s]
            OT St[Cf::NBUF][DVH * Cf::PK];      // S^T block   [j][i]  (16-bit: two buffers, the
            OT dSt[Cf::NBUF][DVH * Cf::PK];     // dS'^T block [j][i]   next block is staged
            OT dOt[Cf::NBUF][kChunk * Cf::PH];  // dO block    [r][j]   while this one is reduced)
            OT vt[Cf::NBUF][Cf::VW_LDS ? kChunk * Cf::PH : 1];  // v block [r][j]
            OT wt[Cf::NBUF][Cf::VW_LDS ? kChunk * Cf::PH : 1];  // w block [r][j]
            OT DlT[DVH * Cf::PC];      // Delta^T             [j][r]
            OT dDT[DVH * Cf::PC];      // dDelta^T            [j][r]
            OT dXt[kChunk * Cf::PH];   // dX block            [r][j]
        } j;
        Gram g;
        struct {  // token-row staging of the gradients behind the Gram tiles, which are still
                  // read while dv and dw leave and hold dq, dk, db at the end
            Gram keep;
            union {
                struct {
                    OT dV[Cf::STG ? kChunk * Cf::PV : 1];  // dv  [r][j]
                    OT dW[Cf::STG ? kChunk * Cf::PV : 1];  // dw  [r][j]
                } vw;
                float dL[Cf::STG ? kChunk * Cf::PL : 1];  // dlog alpha [r][i]
            } x;
        } s;
    } u;
    float tot[4][DK];
    float ctab[6][DK];
    float gRt[4][DK];
    float hRt[4][DK];
    float hRl[4][DK];   // G_C - ref_R (deep-decay path)
    int deep[8];        // per wave: its block decays by more than exp(-kDeepDecay) on a channel
    float r6[DK];
    float r6x[4][DK];  // R6 partials: [lane group l / 16][channel]
    float btot[4][DK];
    float ktot[4][DK];
    float gred[2][kChunk][3];  // per-token partial sums of db, dw, dlog alpha (scalar gates)
    float nrm[2][kChunk][4];   // fused prologue: per-token |q|^2, |k|^2, qhat.dq, khat.dk partials
};

template <typename OT, int DK, int DV, int DVH, int MODE>
__global__ __launch_bounds__(kBgThreads, 1) void gdr2_bgrad_kernel(BwdParams p) {
    using Cf = BgCfg<OT, DK, DV, DVH>;
    using MM = Mfma<OT>;
    using FR = Frag<OT>;
    using RW = Raw4<OT>;
    constexpr int C = kChunk, KS = Cf::KS, KPL = Cf::KPL, PK = Cf::PK, PC = Cf::PC, PH = Cf::PH;
    constexpr int NKS = Cf::NKS, NIBH = Cf::NIBH, VEC = Cf::VEC;
    constexpr int NSV = Cf::NSV, SVEC = Cf::SVEC, NOV = Cf::NOV, OVEC = Cf::OVEC;
    constexpr int NTV = Cf::NTV, TVEC = Cf::TVEC, NT = kBgThreads;
    constexpr bool STG = Cf::STG;
    constexpr int PV = Cf::PV, PL = Cf::PL;
    __shared__ BgSmem<OT, DK, DV, DVH> sm;

    // wave index made wave-uniform, so that branches on R and half are scalar branches
    const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(wave_id()), R = w & 3, half = w >> 2;
    const int l = lane_id(), rl = l & 15, g = l >> 4;
    const int NC = p.NC;
    // heads fastest: workgroups that run at the same time read neighbouring 256-byte pieces of the
    // same token rows of q, k, v, dO, ... ([B, T, H, D] layout) rather than rows 4 KB apart
    // (chunks [c0, c0 + ncr) of the sequence: one launch may cover a part of it)
    const int h = blockIdx.x % p.H, c = p.c0 + (blockIdx.x / p.H) % p.ncr, bb = blockIdx.x / (p.H * p.ncr);
    const int chain = bb * p.H + h;
    const long T = p.T, H = p.H;
    const long cix = (long)chain * NC + c;
    const int r = 16 * R + rl;
    const long t = (long)c * C + r;
    const bool valid = t < T;
    const long row = ((long)bb * T + (valid ? t : T - 1)) * H + h;
    const long tok0 = ((long)bb * T + (long)c * C) * H + h;  // token row of the chunk's first token
    const int ibase = NIBH * half;                            // this wave's first key-channel block
    const int kbeg = (16 * R / KS) * KS;                      // first k-step touching tokens >= 16R

    // ---- this lane's log alpha (token r, channels 16 (ibase+ib) + 4g + e); q, k, b come later
    typename RW::t qr[NIBH], kr[NIBH], br[NIBH];
    // (a fixed scalar b or w leaves too little of q, k, b or v, w to move for the staging to pay)
    constexpr int FGM = MODE >= kModeFixedGates ? MODE - kModeFixedGates : 0;
    constexpr bool QKB_LDS = Cf::QKB_LDS && !(FGM & kEraseScalar);
    constexpr int QVEC = QKB_LDS ? Cf::QVEC : 1;
    i32x4 rQ[QVEC], rK[QVEC], rB[QVEC];  // raw q, k, b rows (16-byte pieces) on their way to LDS
    // scalar gates and the fused prologue (the plain instance carries no gate branches)
    constexpr bool GS = MODE != kModePlain, PRO = mode_prologue(MODE);
    const int gm = gate_bits<MODE>(p.gates);
    const bool b_sc = GS && (gm & kEraseScalar), w_sc = GS && (gm & kWriteScalar);
    const bool a_sc = GS && (gm & kDecayScalar);
    // log alpha, then G_r - ref_R (loaded ahead of the value-column blocks or with the last one,
    // see scan_la)
    f32x4 sc[NIBH];
    auto load_la = [&]() __attribute__((always_inline)) {
        if (a_sc) {
            const float x = p.la[row];
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib) sc[ib] = f32x4{x, x, x, x};
        } else {
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib) sc[ib] = *(const f32x4*)(p.la + row * DK + 16 * (ibase + ib) + 4 * g);
        }
    };
    // in-block cumsum of log alpha (DPP over the 16 tokens), the block totals and the deep-decay
    // ballot; then the per-channel tables exp(ref_R), exp(G_C - ref_R), exp(ref_R - ref_S) from
    // the totals.  Without the fused prologue this runs at the start, while the first value-column
    // blocks are in flight (log alpha is loaded ahead of them; its registers then stay live across
    // the value-column loop); with it, after the loop, where the prologue's q, k arrive.
    // fused prologue: log alpha = -decay_scale * softplus(a); the chain-rule factor
    // -decay_scale * sigmoid(a) of dlog alpha comes from the same exponential
    constexpr bool EARLY = !PRO;
    f32x4 dsa[PRO ? NIBH : 1];
    auto scan_la = [&]() __attribute__((always_inline)) {
        if (PRO) {
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = sc[ib][e], ex = __expf(x);
                    const float sp = x > 20.f ? x : 0.69314718f * __builtin_amdgcn_logf(1.f + ex);
                    dsa[PRO ? ib : 0][e] = -p.pro.decay_scale * (x > 20.f ? 1.f : ex * __builtin_amdgcn_rcpf(1.f + ex));
                    sc[ib][e] = -p.pro.decay_scale * sp;
                }
        }
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib)
#pragma unroll
            for (int e = 0; e < 4; ++e) sc[ib][e] = row_scan16(valid ? sc[ib][e] : 0.f);
        {   // does this block decay past the fast path's range on one of this wave's channels?
            float mn = 0.f;
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib)
#pragma unroll
                for (int e = 0; e < 4; ++e) mn = fminf(mn, sc[ib][e]);
            const unsigned long long dp = __ballot(rl == 15 && mn < -kDeepDecay);
            if (l == 0) sm.deep[w] = dp != 0ull;
        }
        if (rl == 15) {
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib) *(f32x4*)(&sm.tot[R][16 * (ibase + ib) + 4 * g]) = sc[ib];
        }
    };
    auto decay_tables = [&]() __attribute__((always_inline)) {
        for (int chn = tid; chn < DK; chn += NT) {
            float refs[4], run = 0.f;
#pragma unroll
            for (int Rp = 0; Rp < 4; ++Rp) {
                refs[Rp] = run;
                run += sm.tot[Rp][chn];
            }
#pragma unroll
            for (int Rp = 0; Rp < 4; ++Rp) {
                sm.gRt[Rp][chn] = __expf(refs[Rp]);
                sm.hRt[Rp][chn] = __expf(run - refs[Rp]);
                sm.hRl[Rp][chn] = run - refs[Rp];
#pragma unroll
                for (int S = 0; S < Rp; ++S) sm.ctab[Rp * (Rp - 1) / 2 + S][chn] = __expf(refs[Rp] - refs[S]);
            }
        }
    };
    // ---- the chunk's -Y and Ktilde: staged into LDS with T and P below (16-bit operands), or
    //      this wave's token block kept as fragments (fp32)
    constexpr bool YK_LDS = Cf::YK_LDS;
    constexpr int YVEC = YK_LDS ? C * DK / VEC / NT : 1;
    constexpr int NKF = YK_LDS ? 1 : NKS;
    i32x4 pY[YVEC], pK[YVEC];
    typename FR::t Yf[NKF], Kf[NKF];
    {
        const OT* Yc = (const OT*)p.wy.Yh + cix * C * DK;
        const OT* Kc = (const OT*)p.wy.Kt + cix * C * DK;
        if constexpr (YK_LDS) {
#pragma unroll
            for (int m = 0; m < YVEC; ++m) {
                pY[m] = *(const i32x4*)(Yc + (long)(tid + m * NT) * VEC);
                pK[m] = *(const i32x4*)(Kc + (long)(tid + m * NT) * VEC);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKF; ++ks) {
                Yf[ks] = FFrag<OT>::fkc(Yc, DK, 16 * R, ks * KS, l);
                Kf[ks] = FFrag<OT>::fkc(Kc, DK, 16 * R, ks * KS, l);
            }
        }
    }
    // ---- value-column block prefetch registers
    const OT* Sx = (const OT*)p.states + cix * DV * DK;
    const OT* dSxp = (const OT*)p.dSx + cix * DV * DK;
    // NS register sets: 16-bit operands fetch two blocks ahead (the loads take longer than one
    // block's work), fp32 one
    constexpr int NS = Cf::NBUF;
    i32x4 pS[NS][SVEC], pdS[NS][SVEC], pO[NS][OVEC];
    constexpr bool VW_LDS = Cf::VW_LDS && !(FGM & kWriteScalar);
    typename RW::t pv[NS], pw[NS], pU[NS];
    i32x4 pV[NS][VW_LDS ? OVEC : 1], pW[NS][VW_LDS ? OVEC : 1];
    const OT* Uc = (const OT*)p.wy.U + cix * C * DV;
    auto fetch_block = [&](int jq, int st) __attribute__((always_inline)) {
        const int jb0 = jq * DVH;
#pragma unroll
        for (int m = 0; m < SVEC; ++m) {
            const int x = tid + m * NT;
            if (NSV % NT == 0 || x < NSV) {
                const int jj = (x * VEC) / DK, i = (x * VEC) % DK;
                pS[st][m] = *(const i32x4*)(Sx + (long)(jb0 + jj) * DK + i);
                pdS[st][m] = *(const i32x4*)(dSxp + (long)(jb0 + jj) * DK + i);
            }
        }
#pragma unroll
        for (int m = 0; m < OVEC; ++m) {
            const int x = tid + m * NT;
            const int rr = (x * VEC) / DVH, jj = (x * VEC) % DVH;
            i32x4 z = {0, 0, 0, 0}, zv = z, zw = z;
            if ((NOV % NT == 0 || x < NOV) && (long)c * C + rr < T) {
                const long o = (tok0 + (long)rr * H) * DV + jb0 + jj;
                z = *(const i32x4*)((const OT*)p.dO + o);
                if constexpr (VW_LDS) {
                    zv = *(const i32x4*)((const OT*)p.v + o);
                    if (!w_sc) zw = *(const i32x4*)((const OT*)p.w + o);
                }
            }
            pO[st][m] = z;
            if constexpr (VW_LDS) {
                pV[st][m] = zv;
                pW[st][m] = zw;
            }
        }
        // v, w of (token r, columns jb0 + 16 half + 4g .. +3) for dv, dw
        const long trow = valid ? (tok0 + (long)r * H) : row;
        const long o = trow * DV + jb0 + 16 * half + 4 * g;
        if constexpr (!VW_LDS) pv[st] = *(const typename RW::t*)((const OT*)p.v + o);
        if (w_sc) {
            const OT x = ((const OT*)p.w)[trow];
            pw[st] = typename RW::t{x, x, x, x};
        } else if constexpr (!VW_LDS) {
            pw[st] = *(const typename RW::t*)((const OT*)p.w + o);
        }
        pU[st] = *(const typename RW::t*)(Uc + ((long)(R * (DV / 16) + jb0 / 16 + half) * 64 + l) * 4);
    };
    i32x4 pT[TVEC], pP[TVEC];
    {
        const OT* Tc = (const OT*)p.wy.Tm + cix * C * C;
        const OT* Pc = (const OT*)p.wy.P + cix * C * C;
#pragma unroll
        for (int m = 0; m < TVEC; ++m) {
            const int x = tid + m * NT;
            if (NTV % NT == 0 || x < NTV) {
                pT[m] = *(const i32x4*)(Tc + (long)x * VEC);
                pP[m] = *(const i32x4*)(Pc + (long)x * VEC);
            }
        }
    }
    if constexpr (EARLY) load_la();
    fetch_block(0, 0);
    if (NS == 2 && DV / DVH > 1) fetch_block(1, 1);
#pragma unroll
    for (int m = 0; m < TVEC; ++m) {
        const int x = tid + m * NT;
        if (NTV % NT == 0 || x < NTV) {  // fragment order -> row-major
            const int o = FLay<OT>::unit_row(x, C) * PC + FLay<OT>::unit_col(x, C);
            *(i32x4*)(sm.u.j.Tt + o) = pT[m];
            *(i32x4*)(sm.u.j.Pt + o) = pP[m];
        }
    }
    if constexpr (YK_LDS) {
#pragma unroll
        for (int m = 0; m < YVEC; ++m) {  // fragment order -> row-major
            const int x = tid + m * NT;
            const int o = FLay<OT>::unit_row(x, DK) * PK + FLay<OT>::unit_col(x, DK);
            *(i32x4*)(sm.u.j.Yt + o) = pY[m];
            *(i32x4*)(sm.u.j.Kt + o) = pK[m];
        }
    }
    if (tid < DK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) sm.r6x[q][tid] = 0.f;
    }

    float dw_acc = 0.f;                   // sum_j dX_j v_j of this lane's columns (scalar w)
    f32x4 A1[NIBH], A2[NIBH], A3[NIBH];  // R1, R2, R3 (channel x token)
    f32x4 R4[2], R5[2];                   // dO Delta^T, dX Delta^T for s-blocks 2half+{0,1}
#pragma unroll
    for (int ib = 0; ib < NIBH; ++ib) A1[ib] = A2[ib] = A3[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
    R4[0] = R4[1] = R5[0] = R5[1] = f32x4{0.f, 0.f, 0.f, 0.f};

    // staging of a fetched value-column block into LDS buffer b, and the next fetch (block jn, or
    // after the last block the raw key inputs for the Gram phase and the epilogue)
    constexpr int NJ = DV / DVH;
    typename RW::t cv, cw, cU;
    auto stage = [&](int b, int st) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < SVEC; ++m) {
            const int x = tid + m * NT;
            if (NSV % NT == 0 || x < NSV) {
                const int jj = (x * VEC) / DK, i = (x * VEC) % DK;
                *(i32x4*)(sm.u.j.St[b] + jj * PK + i) = pS[st][m];
                *(i32x4*)(sm.u.j.dSt[b] + jj * PK + i) = pdS[st][m];
            }
        }
#pragma unroll
        for (int m = 0; m < OVEC; ++m) {
            const int x = tid + m * NT;
            if (NOV % NT == 0 || x < NOV) {
                const int o = ((x * VEC) / DVH) * PH + (x * VEC) % DVH;
                *(i32x4*)(sm.u.j.dOt[b] + o) = pO[st][m];
                if constexpr (VW_LDS) {
                    *(i32x4*)(sm.u.j.vt[b] + o) = pV[st][m];
                    if (!w_sc) *(i32x4*)(sm.u.j.wt[b] + o) = pW[st][m];
                }
            }
        }
        if constexpr (!VW_LDS) cv = pv[st];
        if (!VW_LDS || w_sc) cw = pw[st];
        cU = pU[st];
    };
    auto fetch_next = [&](int jn, int st) __attribute__((always_inline)) {
        if (jn < NJ) {
            fetch_block(jn, st);
        } else if (jn == NJ) {
            if constexpr (!EARLY) load_la();
            if constexpr (QKB_LDS) {  // rows past T read row T - 1: finite values, zeroed later
#pragma unroll
                for (int m = 0; m < QVEC; ++m) {
                    const int x = tid + m * NT, rr = x / (DK / VEC), i = (x % (DK / VEC)) * VEC;
                    const long tc = (long)c * C + rr < T ? (long)c * C + rr : T - 1;
                    const long o = (((long)bb * T + tc) * H + h) * DK + i;
                    rQ[m] = *(const i32x4*)((const OT*)p.q + o);
                    rK[m] = *(const i32x4*)((const OT*)p.k + o);
                    if (!b_sc) rB[m] = *(const i32x4*)((const OT*)p.b + o);
                }
            }
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib) {
                const int i0 = 16 * (ibase + ib) + 4 * g;
                if constexpr (!QKB_LDS) {
                    qr[ib] = *(const typename RW::t*)((const OT*)p.q + row * DK + i0);
                    kr[ib] = *(const typename RW::t*)((const OT*)p.k + row * DK + i0);
                }
                if (b_sc) {
                    const OT x = ((const OT*)p.b)[row];
                    br[ib] = typename RW::t{x, x, x, x};
                } else if constexpr (!QKB_LDS) {
                    br[ib] = *(const typename RW::t*)((const OT*)p.b + row * DK + i0);
                }
            }
        }
    };
    if constexpr (EARLY) scan_la();
    stage(0, 0);
    fetch_next(NS, 0);
    lds_barrier();
    if constexpr (EARLY) decay_tables();  // read from the Gram phase on, after several barriers

    constexpr int JUNROLL = NS == 2 ? NJ : 1;  // two register sets: unrolled, set indices static
    typename RW::t dvk[NS == 2 ? NJ : 1], dwk[NS == 2 ? NJ : 1];  // dv, dw of every block
#pragma unroll JUNROLL
    for (int jq = 0; jq < NJ; ++jq) {
        constexpr int NBUF = Cf::NBUF;
        const int jb0 = jq * DVH, bq = NBUF == 1 ? 0 : (jq & 1);
        const OT* St = sm.u.j.St[bq];
        const OT* dSt = sm.u.j.dSt[bq];
        const OT* dOt = sm.u.j.dOt[bq];
        // Delta = U - Y S, dDelta = Ktilde dS' + P^T dO: block (token R, columns 16 half)
        {
            const int jb = half;
            f32x4 aD = RW::widen(cU);
            f32x4 adD = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                typename FR::t ay, ak;
                if constexpr (YK_LDS) {
                    ay = FR::kc(sm.u.j.Yt, PK, 16 * R, ks * KS, l);
                    ak = FR::kc(sm.u.j.Kt, PK, 16 * R, ks * KS, l);
                } else {
                    ay = Yf[ks < NKF ? ks : 0];
                    ak = Kf[ks < NKF ? ks : 0];
                }
                MM::mma(aD, ay, FR::kc(St, PK, 16 * jb, ks * KS, l));
                MM::mma(adD, ak, FR::kc(dSt, PK, 16 * jb, ks * KS, l));
            }
            for (int k0 = kbeg; k0 < C; k0 += KS)
                MM::mma(adD, FR::tr(sm.u.j.Pt, PC, k0, 16 * R, l), FR::tr(dOt, PH, k0, 16 * jb, l));
            store_acc_T(sm.u.j.DlT, PC, 16 * jb, 16 * R, aD, l);
            store_acc_T(sm.u.j.dDT, PC, 16 * jb, 16 * R, adD, l);
        }
        lds_barrier();
        // dX^T = dDelta^T T (lane: token r, columns 16 half + 4g .. +3); dv = dX . w, dw = dX . v
        {
            const int jb = half;
            f32x4 ax = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = kbeg; k0 < C; k0 += KS)
                MM::mma(ax, FR::kc(sm.u.j.dDT, PC, 16 * jb, k0, l), FR::tr(sm.u.j.Tt, PC, k0, 16 * R, l));
            const int jc = 16 * jb + 4 * g;
            store4(sm.u.j.dXt + r * PH + jc, ax);
            if constexpr (VW_LDS) {  // this lane's columns of the staged v, w block
                cv = *(const typename RW::t*)(sm.u.j.vt[bq] + r * PH + jc);
                if (!w_sc) cw = *(const typename RW::t*)(sm.u.j.wt[bq] + r * PH + jc);
            }
            f32x4 wg = RW::widen(cw), dwv = ax * RW::widen(cv);
            if (PRO) {  // w = sigmoid(w pre-activation): dw_pre = dw . w (1 - w)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wg[e] = sigmoid_f(wg[e]);
                    dwv[e] *= wg[e] * (1.f - wg[e]);
                }
            }
            if (w_sc) dw_acc += (dwv[0] + dwv[1]) + (dwv[2] + dwv[3]);
            if constexpr (NS == 2) {  // held until the loop ends: no stores between the fetches
                dvk[jq] = RW::narrow(ax * wg);
                dwk[jq] = RW::narrow(dwv);
            } else if (valid) {
                const long o = (tok0 + (long)r * H) * DV + jb0 + jc;
                store4((OT*)p.dv + o, ax * wg);
                if (!w_sc) store4((OT*)p.dw + o, dwv);
            }
        }
        lds_barrier();
        // reductions over this block of value columns
#pragma unroll
        for (int k0 = 0; k0 < DVH; k0 += KS) {
            const typename FR::t bO = FR::kc(dOt, PH, 16 * R, k0, l);          // dO    (col r, k = j)
            const typename FR::t bX = FR::kc(sm.u.j.dXt, PH, 16 * R, k0, l);   // dX    (col r, k = j)
            const typename FR::t bD = FR::tr(sm.u.j.DlT, PC, k0, 16 * R, l);   // Delta (col r, k = j)
#pragma unroll
            for (int ib = 0; ib < NIBH; ++ib) {
                const int i0 = 16 * (ibase + ib);
                const typename FR::t aS = FR::tr(St, PK, k0, i0, l);    // S   (row i, k = j)
                const typename FR::t adS = FR::tr(dSt, PK, k0, i0, l);  // dS' (row i, k = j)
                MM::mma(A1[ib], aS, bO);
                MM::mma(A2[ib], aS, bX);
                MM::mma(A3[ib], adS, bD);
                if (R == 0) {  // R6 partial: channel i0 + l%16, the fragment's k (= value columns)
                    float acc = 0.f;
#pragma unroll
                    for (int e = 0; e < FR::N; ++e) acc += FR::at(aS, e) * FR::at(adS, e);
                    sm.r6x[g][i0 + rl] += acc;
                }
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int S = 2 * half + u;
                if (S <= R) {
                    const typename FR::t bDs = FR::tr(sm.u.j.DlT, PC, k0, 16 * S, l);  // Delta (col s, k = j)
                    MM::mma(R4[u], bO, bDs);
                    MM::mma(R5[u], bX, bDs);
                }
            }
        }
        // the next block into the other buffer while the slow waves finish this one (one buffer:
        // after every wave is done with it)
        if (jq + 1 < NJ) {
            if constexpr (NBUF == 1) lds_barrier();
            stage(NBUF == 1 ? 0 : (bq ^ 1), (jq + 1) % NS);
            fetch_next(jq + 1 + NS, (jq + 1) % NS);
        }
        lds_barrier();
    }
    if constexpr (NS == 2) {
        if constexpr (STG) {  // the value tiles are dead (the loop ends with a barrier)
#pragma unroll
            for (int jq = 0; jq < NJ; ++jq) {
                const int jc = jq * DVH + 16 * half + 4 * g;
                *(typename RW::t*)(sm.u.s.x.vw.dV + r * PV + jc) = dvk[jq];
                if (!w_sc) *(typename RW::t*)(sm.u.s.x.vw.dW + r * PV + jc) = dwk[jq];
            }
        } else if (valid) {
#pragma unroll
            for (int jq = 0; jq < NJ; ++jq) {
                const long o = (tok0 + (long)r * H) * DV + jq * DVH + 16 * half + 4 * g;
                *(typename RW::t*)((OT*)p.dv + o) = dvk[jq];
                if (!w_sc) *(typename RW::t*)((OT*)p.dw + o) = dwk[jq];
            }
        }
    }
    if constexpr (QKB_LDS) {  // raw q, k, b rows into the places of Qbar, Kbar, Ebar (same layout)
#pragma unroll
        for (int m = 0; m < QVEC; ++m) {
            const int x = tid + m * NT, rr = x / (DK / VEC), i = (x % (DK / VEC)) * VEC;
            *(i32x4*)(sm.u.g.Qb + rr * PK + i) = rQ[m];
            *(i32x4*)(sm.u.g.Kb + rr * PK + i) = rK[m];
            if (!b_sc) *(i32x4*)(sm.u.g.Eb + rr * PK + i) = rB[m];
        }
        lds_barrier();  // (also publishes the dv, dw staging)
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib) {
            const int i0 = 16 * (ibase + ib) + 4 * g;
            qr[ib] = *(const typename RW::t*)(sm.u.g.Qb + r * PK + i0);
            kr[ib] = *(const typename RW::t*)(sm.u.g.Kb + r * PK + i0);
            if (!b_sc) br[ib] = *(const typename RW::t*)(sm.u.g.Eb + r * PK + i0);
        }
    }

    if constexpr (!EARLY) scan_la();
    // fused prologue: this wave's half of the squared row norms of q and k (lanes 16g + rl of both
    // channel halves), exchanged through the same barrier as the block totals
    if (PRO) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib) {
            const f32x4 q4 = RW::widen(qr[ib]), k4 = RW::widen(kr[ib]);
            sq += (q4[0] * q4[0] + q4[1] * q4[1]) + (q4[2] * q4[2] + q4[3] * q4[3]);
            sk += (k4[0] * k4[0] + k4[1] * k4[1]) + (k4[2] * k4[2] + k4[3] * k4[3]);
        }
        sq += shfl_xor_l(sq, 16, l);
        sq += shfl_xor_l(sq, 32, l);
        sk += shfl_xor_l(sk, 16, l);
        sk += shfl_xor_l(sk, 32, l);
        if (g == 0) {
            sm.nrm[half][r][0] = sq;
            sm.nrm[half][r][1] = sk;
        }
    }
    if constexpr (!EARLY) {  // publishes the block totals (and the prologue's row norms)
        lds_barrier();
        decay_tables();
    } else if constexpr (STG && NS == 2 && !QKB_LDS) {
        lds_barrier();
    }
    if constexpr (STG && NS == 2) {  // dv, dw as whole token rows; they drain during the Gram phase
        constexpr int UPV = DV / VEC;
#pragma unroll
        for (int m = 0; m < C * UPV / NT; ++m) {
            const int x = tid + m * NT, rr = x / UPV, j = (x % UPV) * VEC;
            if ((long)c * C + rr < T) {
                const long o = (tok0 + (long)rr * H) * DV + j;
                store_stream((i32x4*)((OT*)p.dv + o), *(const i32x4*)(sm.u.s.x.vw.dV + rr * PV + j));
                if (!w_sc) store_stream((i32x4*)((OT*)p.dw + o), *(const i32x4*)(sm.u.s.x.vw.dW + rr * PV + j));
            }
        }
    }
    // deep-decay path for the whole chunk (uniform over the workgroup): right Gram factors
    // referenced to the end of their block and the diagonal blocks entry by entry, so that no
    // factor exceeds one
    bool deep = false;
#pragma unroll
    for (int x = 0; x < 8; ++x) deep |= sm.deep[x] != 0;
    deep = __builtin_amdgcn_readfirstlane(deep);

    // ---- fused prologue: the reciprocal row norms of q and k
    float rq = 1.f, rk = 1.f;
    if (PRO) {
        rq = rsqrtf(sm.nrm[0][r][0] + sm.nrm[1][r][0] + p.pro.norm_eps);
        rk = rsqrtf(sm.nrm[0][r][1] + sm.nrm[1][r][1] + p.pro.norm_eps);
    }
    // the activations the forward used: q, k normalised, b through the sigmoid (computed on the
    // first use and kept, in fp32 as the forward used it)
    f32x4 bsg[PRO ? NIBH : 1];
    auto act = [&](int ib, f32x4& q4, f32x4& k4, f32x4& b4, bool first) __attribute__((always_inline)) {
        q4 = RW::widen(qr[ib]);
        k4 = RW::widen(kr[ib]);
        b4 = RW::widen(br[ib]);
        if (PRO) {
            q4 *= rq;
            k4 *= rk;
            if (first) {
#pragma unroll
                for (int e = 0; e < 4; ++e) b4[e] = sigmoid_f(b4[e]);
                bsg[PRO ? ib : 0] = b4;
            } else {
                b4 = bsg[PRO ? ib : 0];
            }
        }
    };

    // ---- decay-absorbed key tiles (the value tiles are dead) and the dP^T, dA^T tiles
#pragma unroll
    for (int ib = 0; ib < NIBH; ++ib) {
        const int i0 = 16 * (ibase + ib) + 4 * g;
        f32x4 q4, k4, b4;
        act(ib, q4, k4, b4, true);
        f32x4 eb, qb, kb;
        f32x4 tb = {0.f, 0.f, 0.f, 0.f};  // deep-decay path: right factor referenced to the block end
        if (deep) tb = *(const f32x4*)(&sm.tot[R][i0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = valid ? __expf(sc[ib][e]) : 0.f;
            const float y = valid ? __expf(tb[e] - sc[ib][e]) : 0.f;
            eb[e] = b4[e] * k4[e] * x;
            qb[e] = q4[e] * x;
            kb[e] = k4[e] * y;
        }
        store4(sm.u.g.Eb + r * PK + i0, eb);
        store4(sm.u.g.Qb + r * PK + i0, qb);
        store4(sm.u.g.Kb + r * PK + i0, kb);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int S = 2 * half + u;
        f32x4 pm = {0.f, 0.f, 0.f, 0.f}, am = {0.f, 0.f, 0.f, 0.f};
        if (S <= R) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rr = 16 * R + acc_row(e, l), ss = 16 * S + acc_col(l);
                pm[e] = ss <= rr ? R4[u][e] : 0.f;
                am[e] = ss < rr ? -R5[u][e] : 0.f;
            }
        }
        store_acc_T(sm.u.g.dPT, PC, 16 * S, 16 * R, pm, l);
        store_acc_T(sm.u.g.dAT, PC, 16 * S, 16 * R, am, l);
    }
    lds_barrier();
    if (tid < DK) sm.r6[tid] = (sm.r6x[0][tid] + sm.r6x[1][tid]) + (sm.r6x[2][tid] + sm.r6x[3][tid]);

    // ---- A1 <- exp(ref_R) R1 + dP Kbar,  A2 <- -exp(ref_R) R2 + dA Kbar,  A4 <- dP^T Qbar + dA^T Ebar
#pragma unroll
    for (int ib = 0; ib < NIBH; ++ib) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float gr = sm.gRt[R][16 * (ibase + ib) + acc_row(e, l)];
            A1[ib][e] *= gr;
            A2[ib][e] *= -gr;
        }
    }
    for (int k0 = 0; k0 < 16 * R + 16; k0 += KS) {
        const typename FR::t bP = FR::tr(sm.u.g.dPT, PC, k0, 16 * R, l);  // dP (col r, k = s)
        const typename FR::t bA = FR::tr(sm.u.g.dAT, PC, k0, 16 * R, l);  // dA (col r, k = s)
        const int Sl = (k0 + KPL * g) / 16;                             // token block of this lane's k
        // cross-block factor exp(ref_R - ref_S), or exp(ref_R - ref_{S+1}) on the deep-decay path
        // (whose diagonal block is added entry by entry in the epilogue)
        const int cS = deep ? Sl + 1 : Sl;
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib) {
            const int i0 = 16 * (ibase + ib);
            typename FR::t a = FR::tr(sm.u.g.Kb, PK, k0, i0, l);            // Kbar^T (row i, k = s)
            if (deep && Sl == R) a = FR::scale(a, 0.f);
            else if (cS < R) a = FR::scale(a, sm.ctab[R * (R - 1) / 2 + cS][i0 + rl]);
            MM::mma(A1[ib], a, bP);
            MM::mma(A2[ib], a, bA);
        }
    }
    f32x4 A4[NIBH];  // G3 (channel x token s)
#pragma unroll
    for (int ib = 0; ib < NIBH; ++ib) A4[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int k0 = kbeg; k0 < C; k0 += KS) {
        const typename FR::t bP = FR::kc(sm.u.g.dPT, PC, 16 * R, k0, l);  // dP (col s, k = r)
        const typename FR::t bA = FR::kc(sm.u.g.dAT, PC, 16 * R, k0, l);  // dA (col s, k = r)
        const int Rl = (k0 + KPL * g) / 16;
        const int cR = deep ? R + 1 : R;  // as above, with this wave's block on the right
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib) {
            const int i0 = 16 * (ibase + ib);
            typename FR::t aq = FR::tr(sm.u.g.Qb, PK, k0, i0, l);           // Qbar^T (row i, k = r)
            typename FR::t ae = FR::tr(sm.u.g.Eb, PK, k0, i0, l);           // Ebar^T (row i, k = r)
            if (deep && Rl == R) {
                aq = FR::scale(aq, 0.f);
                ae = FR::scale(ae, 0.f);
            } else if (Rl > cR) {
                const float cs = sm.ctab[Rl * (Rl - 1) / 2 + cR][i0 + rl];
                aq = FR::scale(aq, cs);
                ae = FR::scale(ae, cs);
            }
            MM::mma(A4[ib], aq, bP);
            MM::mma(A4[ib], ae, bA);
        }
    }

    // ---- epilogue: lane = token r, channels 16 (ibase + ib) + 4g + e.  dq, dk and db go through
    //      the Gram tiles in LDS (dead once every wave is past the products) and reach HBM as
    //      whole token rows; with the fused prologue dq and dk also wait there for their row dot
    //      products (a cross-wave exchange)
    lds_barrier();
    OT* const stq = sm.u.g.Kb;  // staging [r][i], pitch PK: dq, dk, db
    OT* const stk = sm.u.g.Qb;
    OT* const stb = sm.u.g.Eb;
    f32x4 dG[NIBH];
    const long orow = row * DK;
    float db_acc = 0.f;
    f32x4 dqs[PRO ? NIBH : 1], dks[PRO ? NIBH : 1];  // prologue: gradients held for the norm step
    float Dq = 0.f, Dk = 0.f;                          // prologue: qhat . dq, khat . dk partials
#pragma unroll
    for (int ib = 0; ib < NIBH; ++ib) {
        const int i0 = 16 * (ibase + ib) + 4 * g;
        f32x4 q4, k4, b4;
        act(ib, q4, k4, b4, false);
        if (!valid) q4 = k4 = b4 = f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 hr = *(const f32x4*)(&sm.hRt[R][i0]);
        // deep-decay path: the diagonal-block terms, each with exp(G_r - G_s) <= 1 (s <= r, same
        // block), from lane 16 g + s%16 of this wave (same channels); right factors from single
        // exponents
        f32x4 xq = {0.f, 0.f, 0.f, 0.f}, xe = xq, xkb = xq;  // diagonal-block terms (deep path)
        f32x4 ykb, ykt;  // right factors of the dKbar and dKtilde sums
        if (deep) {
            const f32x4 e4 = b4 * k4, l4 = sc[ib];
            const OT* dPT = sm.u.g.dPT;
            const OT* dAT = sm.u.g.dAT;
#pragma unroll 1
            for (int u = 0; u < 16; ++u) {
                const int src = 16 * g + u, s_ = 16 * R + u;
                const float pRT = to_f(dPT[s_ * PC + r]), aRT = to_f(dAT[s_ * PC + r]);  // dP_rs, dA_rs
                const float pTR = to_f(dPT[r * PC + s_]), aTR = to_f(dAT[r * PC + s_]);  // dP_sr, dA_sr
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float ks_ = __shfl(k4[e], src), qs_ = __shfl(q4[e], src);
                    const float es_ = __shfl(e4[e], src), ls_ = __shfl(l4[e], src);
                    const float flo = __expf(fminf(l4[e] - ls_, 0.f)), fhi = __expf(fminf(ls_ - l4[e], 0.f));
                    xq[e] += pRT * ks_ * flo;
                    xe[e] += aRT * ks_ * flo;
                    xkb[e] += (pTR * qs_ + aTR * es_) * fhi;
                }
            }
            const f32x4 tb = *(const f32x4*)(&sm.tot[R][i0]), hl = *(const f32x4*)(&sm.hRl[R][i0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ykb[e] = __expf(tb[e] - sc[ib][e]);
                ykt[e] = __expf(hl[e] - sc[ib][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                ykb[e] = __expf(-sc[ib][e]);
                ykt[e] = hr[e] * ykb[e];
            }
        }
        f32x4 dqv, dkv, dbv, kdk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x = __expf(sc[ib][e]);
            const float dq = x * A1[ib][e] + xq[e];
            const float de = x * A2[ib][e] + xe[e];
            const float dkb = ykb[e] * A4[ib][e] + xkb[e];
            const float dkt = ykt[e] * A3[ib][e];
            dqv[e] = dq;
            dkv[e] = dkb + dkt + b4[e] * de;
            dbv[e] = k4[e] * de;
            dG[ib][e] = row_rscan16(q4[e] * dq + b4[e] * k4[e] * de - k4[e] * (dkb + dkt));
            kdk[e] = row_rscan16(k4[e] * dkt);
        }
        if (PRO) {  // b = sigmoid(b pre-activation); q, k wait for their row dots
#pragma unroll
            for (int e = 0; e < 4; ++e) dbv[e] *= b4[e] * (1.f - b4[e]);
            dqs[PRO ? ib : 0] = dqv;
            dks[PRO ? ib : 0] = dkv;
            Dq += (q4[0] * dqv[0] + q4[1] * dqv[1]) + (q4[2] * dqv[2] + q4[3] * dqv[3]);
            Dk += (k4[0] * dkv[0] + k4[1] * dkv[1]) + (k4[2] * dkv[2] + k4[3] * dkv[3]);
        }
        if (b_sc) db_acc += (dbv[0] + dbv[1]) + (dbv[2] + dbv[3]);
        if (!PRO) {
            store4(stq + r * PK + i0, dqv);
            store4(stk + r * PK + i0, dkv);
        }
        if (!b_sc) store4(stb + r * PK + i0, dbv);
        if (rl == 0) {
            *(f32x4*)(&sm.btot[R][i0]) = dG[ib];
            *(f32x4*)(&sm.ktot[R][i0]) = kdk;
        }
    }
    // scalar gates: the gradient is the sum over this token's channels (lanes 16g + rl of both
    // channel halves)
    if (b_sc || w_sc) {
        db_acc += shfl_xor_l(db_acc, 16, l);
        db_acc += shfl_xor_l(db_acc, 32, l);
        dw_acc += shfl_xor_l(dw_acc, 16, l);
        dw_acc += shfl_xor_l(dw_acc, 32, l);
        if (g == 0) {
            sm.gred[half][r][0] = db_acc;
            sm.gred[half][r][1] = dw_acc;
        }
    }
    if (PRO) {
        Dq += shfl_xor_l(Dq, 16, l);
        Dq += shfl_xor_l(Dq, 32, l);
        Dk += shfl_xor_l(Dk, 16, l);
        Dk += shfl_xor_l(Dk, 32, l);
        if (g == 0) {
            sm.nrm[half][r][2] = Dq;
            sm.nrm[half][r][3] = Dk;
        }
    }
    lds_barrier();
    if (PRO) {  // d q_pre = r_q (dq - qhat (qhat . dq)), the same for k
        const float Dqt = sm.nrm[0][r][2] + sm.nrm[1][r][2], Dkt = sm.nrm[0][r][3] + sm.nrm[1][r][3];
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib) {
            const int i0 = 16 * (ibase + ib) + 4 * g;
            f32x4 q4, k4, b4;
            act(ib, q4, k4, b4, false);
            store4(stq + r * PK + i0, rq * (dqs[PRO ? ib : 0] - q4 * Dqt));
            store4(stk + r * PK + i0, rk * (dks[PRO ? ib : 0] - k4 * Dkt));
        }
    }
    float dl_acc = 0.f;
    if (valid) {
#pragma unroll
        for (int ib = 0; ib < NIBH; ++ib) {
            const int i0 = 16 * (ibase + ib) + 4 * g;
            // + dgamma . gamma, the key-side block totals and the erase totals of the later blocks
            f32x4 dl = dG[ib] + *(const f32x4*)&sm.r6[i0] * *(const f32x4*)&sm.hRt[0][i0];
#pragma unroll
            for (int Rp = 0; Rp < 4; ++Rp) {
                dl += *(const f32x4*)&sm.ktot[Rp][i0];
                if (Rp > R) dl += *(const f32x4*)&sm.btot[Rp][i0];
            }
            if (PRO && !a_sc) dl *= dsa[PRO ? ib : 0];  // d a = d log alpha . (-c sigmoid(a))
            if (a_sc) {
                dl_acc += (dl[0] + dl[1]) + (dl[2] + dl[3]);
            } else if constexpr (STG) {  // dv, dw have left the staging tiles (barriers since)
                *(f32x4*)(sm.u.s.x.dL + r * PL + i0) = dl;
            } else {
                *(f32x4*)(p.dla + orow + i0) = dl;
            }
        }
    }
    if (a_sc) {
        dl_acc += shfl_xor_l(dl_acc, 16, l);
        dl_acc += shfl_xor_l(dl_acc, 32, l);
        if (g == 0) sm.gred[half][r][2] = dl_acc;
        lds_barrier();
    }
    if ((b_sc || w_sc || a_sc) && half == 0 && g == 0 && valid) {
        if (b_sc) ((OT*)p.db)[row] = from_f<OT>(sm.gred[0][r][0] + sm.gred[1][r][0]);
        if (w_sc) ((OT*)p.dw)[row] = from_f<OT>(sm.gred[0][r][1] + sm.gred[1][r][1]);
        if (a_sc) {
            const float d = sm.gred[0][r][2] + sm.gred[1][r][2];
            p.dla[row] = PRO ? d * (-p.pro.decay_scale * sigmoid_f(p.la[row])) : d;
        }
    }
    // ---- the staged dq, dk, db (and dlog alpha) rows to HBM
    lds_barrier();
    {
        constexpr int UPR = DK / VEC;  // 16-byte units per token row
#pragma unroll
        for (int m = 0; m < C * UPR / NT; ++m) {
            const int x = tid + m * NT, rr = x / UPR, i = (x % UPR) * VEC;
            if ((long)c * C + rr < T) {
                const long o = (tok0 + (long)rr * H) * DK + i;
                store_stream((i32x4*)((OT*)p.dq + o), *(const i32x4*)(stq + rr * PK + i));
                store_stream((i32x4*)((OT*)p.dk + o), *(const i32x4*)(stk + rr * PK + i));
                if (!b_sc) store_stream((i32x4*)((OT*)p.db + o), *(const i32x4*)(stb + rr * PK + i));
            }
        }
    }
    if constexpr (STG) {
        if (!a_sc) {
            constexpr int UPL = DK / 4;  // 16-byte units per fp32 row
#pragma unroll
            for (int m = 0; m < C * UPL / NT; ++m) {
                const int x = tid + m * NT, rr = x / UPL, i = (x % UPL) * 4;
                if ((long)c * C + rr < T)
                    store_stream((f32x4*)(p.dla + (tok0 + (long)rr * H) * DK + i), *(const f32x4*)(sm.u.s.x.dL + rr * PL + i));
            }
        }
    }

}

template <typename OT, int DK, int DV>
static hipError_t launch_bgrad(const BwdParams& p, hipStream_t s) {
    const long nblk = (long)p.B * p.H * p.ncr;
    if (nblk == 0) return hipSuccess;
    auto go = [&](auto mode) {
        hipLaunchKernelGGL((gdr2_bgrad_kernel<OT, DK, DV, 32, decltype(mode)::value>), dim3(nblk), dim3(kBgThreads), 0, s, p);
    };
    with_mode<sizeof(OT) == 2>(p.prologue, p.gates, go);  // the fp32 path reads the gate bits
    return hipGetLastError();
}

hipError_t bgrad_dispatch(int bf, int dk, int dv, const BwdParams& p, hipStream_t s) {
    if (bf) {
        if (dk == 128 && dv == 128) return launch_bgrad<bf16, 128, 128>(p, s);
        if (dk == 128 && dv == 64) return launch_bgrad<bf16, 128, 64>(p, s);
        if (dk == 64 && dv == 128) return launch_bgrad<bf16, 64, 128>(p, s);
        if (dk == 64 && dv == 64) return launch_bgrad<bf16, 64, 64>(p, s);
    } else {
        if (dk == 128 && dv == 128) return launch_bgrad<float, 128, 128>(p, s);
        if (dk == 128 && dv == 64) return launch_bgrad<float, 128, 64>(p, s);
        if (dk == 64 && dv == 128) return launch_bgrad<float, 64, 128>(p, s);
        if (dk == 64 && dv == 64) return launch_bgrad<float, 64, 64>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
