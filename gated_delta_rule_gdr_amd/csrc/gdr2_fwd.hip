// gdr2_fwd.hip -- chunkwise forward of the Gated Delta Rule-2 layer for gfx950.
//
// Recurrence (per batch b, head h; S is d_k x d_v): the forum summary "Gated DeltaNet-2:
// Decoupling Erase and Write Gates in Linear Attention for Better Memory Editing" (zhichai.net),
// section "Gated Delta Rule-2", prints
//     S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T ,  o_t = S_t^T q_t.
// The ainews.random.gg article on Gated DeltaNet-2, section "Chunkwise training and gate-aware
// backward", says the cumulative channel-wise decay of a chunk is absorbed into the two factors of
// each rank-one erase, so that a chunk is a product of asymmetric factors I - kbar_r ebar_r^T, in a
// WY form, with chunk size 64.  Written out for one chunk of C = 64 tokens entered with state S
// (G_r = in-chunk inclusive cumsum of log alpha, e = b . k, z = w . v, gamma = exp(G_C)):
//     A_rs = sum_i e_ri k_si exp(G_ri - G_si)   (r > s),     T = (I + A)^-1 (unit lower)
//     P_rs = sum_i q_ri k_si exp(G_ri - G_si)   (r >= s)
//     X    = Z - (E . e^G) S
//     Delta = T X
//     O    = (Q . e^G) S + P Delta
//     S'   = Diag(gamma) S + (K . e^{G_C - G})^T Delta
// (Delta = T Z - (T Ebar) S is the WY pair U - Y S, evaluated as T (Z - Ebar S) so that the C x d_k
// factor Y never has to be formed.)
//
// Parallel structure: one workgroup (4 waves) walks the chunks of one (b, h) chain for one slice of
// DVS value columns -- the carry is independent per value column -- and recomputes the key-side
// quantities (A, P, T) per slice.  The state slice lives in MFMA accumulators (fp32) and, as the
// bf16/fp32 MFMA operand, transposed in LDS.
//
// Exponent ranges: per 16-row block R the reference point ref_R = G at the row before the block
// (0 for the first block).  Left Gram operands carry exp(G_r - ref_R) <= 1, right operands carry
// exp(ref_S - G_s) (the decay over at most 16 tokens, inverted) times exp(ref_R - ref_S) <= 1.  The
// only factor above one is the inverse decay across one 16-token block, which stays finite in fp32
// as long as that decay is above exp(-88) on every channel.
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <typename OT, int DK, int DVS>
struct FwdCfg {
    static constexpr int C = kChunk;
    static constexpr int PAD = 16 / (int)sizeof(OT);
    static constexpr int PK = DK + PAD;     // pitch of [*][DK] operand tiles
    static constexpr int PC = C + PAD;      // pitch of [*][C] operand tiles
    static constexpr int PAF = C + 1;       // pitch of the fp32 A / T matrix
    static constexpr int CG = DK / 4;       // 4-channel groups
    static constexpr int RG = kThreads / CG;  // row groups
    static constexpr int RPT = C / RG;      // rows per thread in the key-side prep
    static constexpr int NJB = DVS / 16;    // 16-column blocks of the slice
    static constexpr int NIB = DK / 16;
    static constexpr int BPW = NIB * NJB / kWaves;  // state blocks per wave
    static constexpr int RZ = C * DVS / kThreads;   // rows per thread in the value prep
    static constexpr int PO = DVS + PAD;
    static_assert(RPT * RG == C && RPT >= 1 && 16 % RPT == 0, "key prep mapping");
    static_assert(BPW >= 1 && BPW * kWaves == NIB * NJB, "state block mapping");
    static_assert(RZ % 4 == 0, "value prep mapping");
};

template <typename OT, int DK, int DVS>
struct alignas(16) FwdSmem {
    using Cf = FwdCfg<OT, DK, DVS>;
    OT Ebk[kChunk * Cf::PK];   // e_r . exp(G_r - ref_R)        [r][i]
    OT Qbk[kChunk * Cf::PK];   // q_r . exp(G_r - ref_R)        [r][i]
    OT Kbk[kChunk * Cf::PK];   // k_s . exp(ref_S - G_s)        [s][i]
    OT KtT[DK * Cf::PC];       // k_r . exp(G_C - G_r), transposed [i][r]
    OT ZT[DVS * Cf::PC];       // z = w . v, transposed         [j][r]
    OT XT[DVS * Cf::PC];       // X^T                           [j][r]
    OT DT[DVS * Cf::PC];       // Delta^T                       [j][r]
    OT ST[DVS * Cf::PK];       // S^T (operand copy of the state) [j][i]
    OT Tm[kChunk * Cf::PC];    // T                             [r][s]
    OT Pm[kChunk * Cf::PC];    // P                             [r][s]
    OT Ost[kChunk * Cf::PO];   // output staging                [r][j]
    float Af[kChunk * Cf::PAF];  // A (strict lower), then T in fp32 (see tblk)
    float Mf[kWaves][16 * 17];   // per-wave scratch of the solve
    float tot[Cf::RG * DK];      // per row-group log-decay totals
    float ctab[6 * DK];          // exp(ref_R - ref_S), R > S
    float gR[4 * DK];            // exp(ref_R)
    float gam[DK];               // exp(G_C)
};

// Location of block T_RS of the inverse inside Af: diagonal blocks overwrite A_RR, off-diagonal
// blocks live in the (unused) strictly upper block (S, R) so that A_RK stays readable.
template <int PAF>
__device__ __forceinline__ float* tblk(float* Af, int R, int S) {
    return R == S ? Af + 16 * R * PAF + 16 * R : Af + 16 * S * PAF + 16 * R;
}

// T = (I + A)^-1 for the strictly lower 64 x 64 A held in Af (fp32), 16 x 16 blocked:
// diagonal blocks by forward substitution (wave R, lane = column), then
// T_RS = -T_RR sum_{S <= K < R} A_RK T_KS level by level with fp32 MFMA.  Ends with a barrier.
template <int PAF>
__device__ void solve_unit_lower_64(float* Af, float (*Mf)[16 * 17]) {
    const int w = wave_id(), l = lane_id();
    {
        float* Ab = Af + 16 * w * PAF + 16 * w;
        const int c = l & 15;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc -= Ab[r * PAF + s] * x[s];
            x[r] = acc;
        }
        wave_sync();
        if (l < 16) {
#pragma unroll
            for (int r = 0; r < 16; ++r) Ab[r * PAF + c] = x[r];
        }
    }
    lds_barrier();
    // levels d = 1, 2, 3: pairs (R, S = R - d)
#pragma unroll
    for (int d = 1; d <= 3; ++d) {
        if (w < 4 - d) {
            const int S = w, R = w + d;
            f32x4 m = {0.f, 0.f, 0.f, 0.f};
            for (int K = S; K < R; ++K) {
                const float* tks = tblk<PAF>(Af, K, S);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    mma32(m, fa32(Af, PAF, 16 * R, 16 * K + 4 * kk), fb32(tks, PAF, 4 * kk, 0));
            }
            float* M = Mf[w];
#pragma unroll
            for (int e = 0; e < 4; ++e) M[acc_row(e) * 17 + acc_col()] = m[e];
            wave_sync();
            f32x4 n = {0.f, 0.f, 0.f, 0.f};
            const float* trr = tblk<PAF>(Af, R, R);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) mma32(n, fa32(trr, PAF, 0, 4 * kk), fb32(M, 17, 4 * kk, 0));
            float* trs = tblk<PAF>(Af, R, S);
#pragma unroll
            for (int e = 0; e < 4; ++e) trs[acc_row(e) * PAF + acc_col()] = -n[e];
        }
        lds_barrier();
    }
}

template <typename OT, int DK, int DVS>
__global__ __launch_bounds__(kThreads, 1) void gdr2_fwd_kernel(FwdParams p) {
    using Cf = FwdCfg<OT, DK, DVS>;
    using MM = Mfma<OT>;
    constexpr int C = kChunk, PK = Cf::PK, PC = Cf::PC, PAF = Cf::PAF, RG = Cf::RG;
    constexpr int RPT = Cf::RPT, NJB = Cf::NJB, BPW = Cf::BPW, RZ = Cf::RZ, PO = Cf::PO;
    constexpr int KS = MM::KS;
    __shared__ FwdSmem<OT, DK, DVS> sm;

    const int tid = threadIdx.x, w = wave_id();
    const int work = xcd_swizzle(blockIdx.x, gridDim.x);
    const int chain = work / p.NS, slice = work % p.NS;
    const int bb = chain / p.H, h = chain % p.H;
    const int j0 = slice * DVS;
    const long T = p.T, H = p.H, DV = p.DV;
    const long tokstride_k = H * DK, tokstride_v = H * DV;
    const OT* q = (const OT*)p.q + ((long)bb * T * H + h) * DK;
    const OT* k = (const OT*)p.k + ((long)bb * T * H + h) * DK;
    const OT* bg = (const OT*)p.b + ((long)bb * T * H + h) * DK;
    const float* la = p.la + ((long)bb * T * H + h) * DK;
    const OT* v = (const OT*)p.v + ((long)bb * T * H + h) * DV + j0;
    const OT* wg = (const OT*)p.w + ((long)bb * T * H + h) * DV + j0;
    OT* o = p.o ? (OT*)p.o + ((long)bb * T * H + h) * DV + j0 : nullptr;

    // ---- state slice: accumulators, wave w owns blocks w*BPW .. w*BPW+BPW-1 of (NIB x NJB)
    f32x4 Sacc[BPW];
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
        const int bi = w * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s0 = 0.f;
            if (p.S0) s0 = p.S0[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()];
            Sacc[u][e] = s0;
        }
        store_acc_T(sm.ST, PK, 16 * jb, 16 * ib, Sacc[u]);
    }
    // upper (never written) blocks of T and P are zero for every chunk
    for (int x = tid; x < C * C; x += kThreads) {
        const int r = x / C, s = x % C;
        if ((s >> 4) > (r >> 4)) {
            sm.Tm[r * PC + s] = from_f<OT>(0.f);
            sm.Pm[r * PC + s] = from_f<OT>(0.f);
        }
    }

    // thread mapping of the key-side prep: 4 channels x RPT rows
    const int cg = tid % Cf::CG, rg = tid / Cf::CG;
    const int i0 = 4 * cg, rbase = rg * RPT;
    const int Rblk = rbase / 16;
    // thread mapping of the value prep: one column x RZ rows
    const int jz = tid % DVS, rz0 = (tid / DVS) * RZ;

    f32x4 qr[RPT], kr[RPT], br[RPT], lr[RPT];
    float vz[RZ], wz[RZ];
#define GDR2_LOAD_CHUNK(cidx)                                                        \
    {                                                                                \
        const long t0_ = (long)(cidx) * C;                                           \
        _Pragma("unroll") for (int u = 0; u < RPT; ++u) {                            \
            const long t = t0_ + rbase + u;                                          \
            const bool ok = t < T;                                                   \
            const long tt = ok ? t : 0;                                              \
            qr[u] = load4(q + tt * tokstride_k + i0);                                \
            kr[u] = load4(k + tt * tokstride_k + i0);                                \
            br[u] = load4(bg + tt * tokstride_k + i0);                               \
            lr[u] = load4(la + tt * tokstride_k + i0);                               \
            if (!ok) qr[u] = kr[u] = br[u] = lr[u] = f32x4{0.f, 0.f, 0.f, 0.f};      \
        }                                                                            \
        _Pragma("unroll") for (int u = 0; u < RZ; ++u) {                             \
            const long t = t0_ + rz0 + u;                                            \
            const bool ok = t < T;                                                   \
            const long tt = ok ? t : 0;                                              \
            vz[u] = ok ? to_f(v[tt * tokstride_v + jz]) : 0.f;                       \
            wz[u] = ok ? to_f(wg[tt * tokstride_v + jz]) : 0.f;                      \
        }                                                                            \
    }

    const int NC = p.NC;
    if (NC > 0) GDR2_LOAD_CHUNK(0);
    lds_barrier();

    for (int c = 0; c < NC; ++c) {
        const long t0 = (long)c * C;
        // ---- checkpoint of the chunk-entry state (operand precision), layout [chain][c][j][i]
        if (p.states) {
            OT* dst = (OT*)p.states + (((long)chain * NC + c) * DV + j0) * DK;
            constexpr int VEC = 16 / (int)sizeof(OT);
            for (int x = tid; x < DVS * DK / VEC; x += kThreads) {
                const int j = (x * VEC) / DK, i = (x * VEC) % DK;
                *(uint4*)(dst + (long)j * DK + i) = *(const uint4*)(sm.ST + j * PK + i);
            }
        }
        // ---- key-side prep: cumulative log decay and the decay-absorbed factors
        f32x4 G[RPT];
        {
            f32x4 run = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                run += lr[u];
                G[u] = run;
            }
            *(f32x4*)(sm.tot + rg * DK + i0) = run;
#pragma unroll
            for (int u = 0; u < RZ; ++u) vz[u] *= wz[u];  // z = w . v
        }
        lds_barrier();
        f32x4 pre = {0.f, 0.f, 0.f, 0.f}, refR = {0.f, 0.f, 0.f, 0.f}, GC = {0.f, 0.f, 0.f, 0.f};
        f32x4 refs[4];
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const f32x4 tg = *(const f32x4*)(sm.tot + g * DK + i0);
            if ((g * RPT) % 16 == 0) refs[(g * RPT) / 16] = GC;
            if (g < rg) pre += tg;
            GC += tg;
        }
#pragma unroll
        for (int R = 0; R < 4; ++R)
            if (R == Rblk) refR = refs[R];
        {
            f32x4 gRv, hR;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                gRv[j] = __expf(refR[j]);
                hR[j] = __expf(GC[j] - refR[j]);
            }
            OT kt[4][RPT];
#pragma unroll
            for (int u = 0; u < RPT; ++u) {
                const int r = rbase + u;
                f32x4 eb, qb, kb;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float g = G[u][j] + pre[j];
                    const float x = __expf(g - refR[j]);
                    const float y = __expf(refR[j] - g);
                    eb[j] = br[u][j] * kr[u][j] * x;
                    qb[j] = qr[u][j] * x;
                    kb[j] = kr[u][j] * y;
                    kt[j][u] = from_f<OT>(kb[j] * hR[j]);
                }
                store4(sm.Ebk + r * PK + i0, eb);
                store4(sm.Qbk + r * PK + i0, qb);
                store4(sm.Kbk + r * PK + i0, kb);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                OT* dst = sm.KtT + (i0 + j) * PC + rbase;
#pragma unroll
                for (int u = 0; u < RPT; ++u) dst[u] = kt[j][u];
            }
            if (rg == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = i0 + j;
                    sm.gam[i] = __expf(GC[j]);
#pragma unroll
                    for (int R = 0; R < 4; ++R) {
                        sm.gR[R * DK + i] = __expf(refs[R][j]);
#pragma unroll
                        for (int S = 0; S < R; ++S)
                            sm.ctab[(R * (R - 1) / 2 + S) * DK + i] = __expf(refs[R][j] - refs[S][j]);
                    }
                }
            }
            OT* zd = sm.ZT + jz * PC + rz0;
#pragma unroll
            for (int u = 0; u < RZ; ++u) zd[u] = from_f<OT>(vz[u]);
        }
        // registers are free: prefetch the next chunk while this one computes
        if (c + 1 < NC) GDR2_LOAD_CHUNK(c + 1);
        lds_barrier();

        // ---- A = strict_lower(Ebar Kbar^T), P = lower(Qbar Kbar^T), 16 x 16 blocks (R, S <= R)
        {
            // (R,S) pairs per wave: {(0,0),(3,0),(3,3)}, {(1,0),(1,1),(3,1)}, {(2,0),(2,1)}, {(2,2),(3,2)}
            constexpr int pr[4][3] = {{0, 3, 3}, {1, 1, 3}, {2, 2, -1}, {2, 3, -1}};
            constexpr int ps[4][3] = {{0, 0, 3}, {0, 1, 1}, {0, 1, -1}, {2, 2, -1}};
#pragma unroll
            for (int n = 0; n < 3; ++n) {
                int R = 0, S = 0;
                switch (w) {
                    case 0: R = pr[0][n]; S = ps[0][n]; break;
                    case 1: R = pr[1][n]; S = ps[1][n]; break;
                    case 2: R = pr[2][n]; S = ps[2][n]; break;
                    default: R = pr[3][n]; S = ps[3][n]; break;
                }
                if (R < 0) continue;
                f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
                const float* cs = sm.ctab + (R * (R - 1) / 2 + S) * DK;
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += KS) {
                    typename MM::frag bK = (S < R) ? MM::load_scaled(sm.Kbk, PK, 16 * S, k0, cs)
                                                   : MM::load(sm.Kbk, PK, 16 * S, k0);
                    MM::mma(aA, MM::load(sm.Ebk, PK, 16 * R, k0), bK);
                    MM::mma(aP, MM::load(sm.Qbk, PK, 16 * R, k0), bK);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = acc_row(e), s = acc_col();
                    sm.Af[(16 * R + r) * PAF + 16 * S + s] = (S < R || s < r) ? aA[e] : 0.f;
                    sm.Pm[(16 * R + r) * PC + 16 * S + s] = from_f<OT>((S < R || s <= r) ? aP[e] : 0.f);
                }
            }
        }
        lds_barrier();
        solve_unit_lower_64<PAF>(sm.Af, sm.Mf);
        // T (lower incl.) into the operand tile
        for (int x = tid; x < 10 * 256; x += kThreads) {
            const int blk = x >> 8, e = x & 255, rr = e >> 4, ss = e & 15;
            const int R = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
            const int S = blk - R * (R + 1) / 2;
            sm.Tm[(16 * R + rr) * PC + 16 * S + ss] = from_f<OT>(tblk<PAF>(sm.Af, R, S)[rr * PAF + ss]);
        }
        lds_barrier();

        // ---- value side: wave w owns token block R = w
        const int R = w;
        f32x4 aW[NJB], aO[NJB];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) aW[jb] = aO[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            const float* gsc = sm.gR + R * DK;
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += KS) {
                typename MM::frag aE = MM::load_scaled(sm.Ebk, PK, 16 * R, k0, gsc);
                typename MM::frag aQ = MM::load_scaled(sm.Qbk, PK, 16 * R, k0, gsc);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) {
                    typename MM::frag bS = MM::load(sm.ST, PK, 16 * jb, k0);
                    MM::mma(aW[jb], aE, bS);
                    MM::mma(aO[jb], aQ, bS);
                }
            }
        }
        // X = Z - Ebar S
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            const OT* zp = sm.ZT + (16 * jb + acc_col()) * PC + 16 * R + acc_row(0);
            f32x4 xv;
#pragma unroll
            for (int e = 0; e < 4; ++e) xv[e] = to_f(zp[e]) - aW[jb][e];
            store_acc_T(sm.XT, PC, 16 * jb, 16 * R, xv);
        }
        lds_barrier();
        // Delta = T X (T lower triangular: k over tokens < 16R + 16)
        {
            f32x4 aD[NJB];
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) aD[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int kend = ((16 * R + 16 + KS - 1) / KS) * KS;
            for (int k0 = 0; k0 < kend; k0 += KS) {
                typename MM::frag aT = MM::load(sm.Tm, PC, 16 * R, k0);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) MM::mma(aD[jb], aT, MM::load(sm.XT, PC, 16 * jb, k0));
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) store_acc_T(sm.DT, PC, 16 * jb, 16 * R, aD[jb]);
        }
        lds_barrier();
        // O = Qbar S + P Delta
        {
            const int kend = ((16 * R + 16 + KS - 1) / KS) * KS;
            for (int k0 = 0; k0 < kend; k0 += KS) {
                typename MM::frag aP = MM::load(sm.Pm, PC, 16 * R, k0);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) MM::mma(aO[jb], aP, MM::load(sm.DT, PC, 16 * jb, k0));
            }
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.Ost[(16 * R + acc_row(e)) * PO + 16 * jb + acc_col()] = from_f<OT>(aO[jb][e]);
        }
        // S' = Diag(gamma) S + Ktilde^T Delta
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = w * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[u][e] *= sm.gam[16 * ib + acc_row(e)];
#pragma unroll
            for (int k0 = 0; k0 < C; k0 += KS)
                MM::mma(Sacc[u], MM::load(sm.KtT, PC, 16 * ib, k0), MM::load(sm.DT, PC, 16 * jb, k0));
            store_acc_T(sm.ST, PK, 16 * jb, 16 * ib, Sacc[u]);
        }
        lds_barrier();
        // ---- output tile to HBM
        {
            constexpr int NV = C * DVS / 4;
            for (int x = tid; x < NV; x += kThreads) {
                const int r = (x * 4) / DVS, j = (x * 4) % DVS;
                const long t = t0 + r;
                if (t < T && o) {
                    const OT* s = sm.Ost + r * PO + j;
                    store4(o + t * tokstride_v + j, f32x4{to_f(s[0]), to_f(s[1]), to_f(s[2]), to_f(s[3])});
                }
            }
        }
    }
    // ---- final state (fp32)
    if (p.ST) {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = w * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.ST[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()] = Sacc[u][e];
        }
    }
}

#undef GDR2_LOAD_CHUNK

template <typename OT, int DK, int DVS>
static hipError_t launch_fwd(const FwdParams& p, hipStream_t stream) {
    const int nblk = p.B * p.H * p.NS;
    hipLaunchKernelGGL((gdr2_fwd_kernel<OT, DK, DVS>), dim3(nblk), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

int fwd_slice_width(int dtype_bf16, int dk, int dv, long chains) {
    if (!dtype_bf16) return 16;
    const int cands_128[2] = {32, 16};
    const int cands_64[3] = {64, 32, 16};
    const int* cands = dk == 128 ? cands_128 : cands_64;
    const int n = dk == 128 ? 2 : 3;
    for (int x = 0; x < n; ++x)
        if (cands[x] <= dv && chains * (dv / cands[x]) >= 256) return cands[x];
    return 16;
}

hipError_t fwd_dispatch(int dtype_bf16, int dk, int dvs, const FwdParams& p, hipStream_t s) {
    if (dtype_bf16) {
        if (dk == 128 && dvs == 32) return launch_fwd<bf16, 128, 32>(p, s);
        if (dk == 128 && dvs == 16) return launch_fwd<bf16, 128, 16>(p, s);
        if (dk == 64 && dvs == 64) return launch_fwd<bf16, 64, 64>(p, s);
        if (dk == 64 && dvs == 32) return launch_fwd<bf16, 64, 32>(p, s);
        if (dk == 64 && dvs == 16) return launch_fwd<bf16, 64, 16>(p, s);
    } else {
        if (dk == 64 && dvs == 16) return launch_fwd<float, 64, 16>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
