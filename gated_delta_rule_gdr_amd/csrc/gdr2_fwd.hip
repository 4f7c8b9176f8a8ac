// gdr2_fwd.hip -- chunked forward of the Gated Delta Rule-2 layer for gfx950.
//
// Recurrence (per batch b, head h; S is d_k x d_v): the forum summary "Gated DeltaNet-2:
// Decoupling Erase and Write Gates in Linear Attention for Better Memory Editing" (zhichai.net),
// section "Gated Delta Rule-2", prints
//     S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T ,  o_t = S_t^T q_t.
// The ainews.random.gg article on Gated DeltaNet-2, section "Chunkwise training and gate-aware
// backward", says the cumulative channel-wise decay of a chunk is absorbed into the two factors of
// each rank-one erase, so that a chunk is a product of asymmetric factors I - kbar_r ebar_r^T in a
// WY form, with chunk size 64.  Written out for one chunk of C = 64 tokens entered with state S
// (G_r = in-chunk inclusive cumsum of log alpha, e = b . k, z = w . v, gamma = exp(G_C)):
//     A_rs = sum_i e_ri k_si exp(G_ri - G_si)   (r > s),     T = (I + A)^-1 (unit lower)
//     P_rs = sum_i q_ri k_si exp(G_ri - G_si)   (r >= s)
//     Y = T (E . e^G),  U = T Z                 (the WY pair)
//     Delta = U - Y S
//     O     = (Q . e^G) S + P Delta
//     S'    = Diag(gamma) S + (K . e^{G_C - G})^T Delta
//
// Two kernels:
//   gdr2_wy_kernel     one workgroup per (chain, chunk), all chunks in parallel: gate prep, the
//                      Gram products A and P on MFMA, the 64 x 64 unit-lower solve, Y and U.
//                      Writes the per-chunk factors (-Y, Qbar, Ktilde, P, T, U, gamma).  It is
//                      compiled on its own, in gdr2_wy.hip (its own scheduling flags).
//   gdr2_carry_kernel  one workgroup per (chain, slice of value columns), sequential over chunks:
//                      Delta, O and the state update, the state slice held in MFMA accumulators.
//                      The carry is independent per value column, so slices run in parallel.
//
// Exponent ranges: per 16-row block R the reference point ref_R = G at the row before the block
// (0 for the first block).  Left Gram operands carry exp(G_r - ref_R) <= 1, right operands carry
// exp(ref_S - G_s) (the inverse of the decay across at most 16 tokens) times exp(ref_R - ref_S)
// <= 1.  The only factor above one stays finite in fp32 as long as the decay across one 16-token
// block is above exp(-88) on every channel.
#include <mutex>

#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"
#include "gdr2_wy.hpp"

namespace gdr2 {

// Static device scratch of the no-allocation forward-only entry point: the per-chunk factors of
// one call (the region a workspace argument brings in for the other entry points).  Every device
// the library runs on holds its own copy until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: only the address from hipGetSymbolAddress is used.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {  // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = p;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

template <typename OT, int DK, int DVS>
struct CarryCfg {
    static constexpr int C = kChunk;
    static constexpr int KS = Mfma<OT>::KS;
    static constexpr int PAD = 16 / (int)sizeof(OT);
    static constexpr int PK = DK + PAD, PC = C + PAD, PO = DVS + PAD;
    static constexpr int NKS = DK / KS, NCK = C / KS;
    static constexpr int NJB = DVS / 16, NIB = DK / 16;
    static constexpr int BPW = NIB * NJB / kWaves;
    static constexpr int KVEC = C * DK * (int)sizeof(OT) / 16 / kThreads;  // 16-byte vectors per thread
    static_assert(BPW >= 1 && BPW * kWaves == NIB * NJB, "state block mapping");
    static_assert(KVEC * kThreads * 16 == C * DK * (int)sizeof(OT), "K staging mapping");
};

template <typename OT, int DK, int DVS>
struct alignas(16) CarrySmem {
    using Cf = CarryCfg<OT, DK, DVS>;
    OT ST[DVS * Cf::PK];      // S^T, operand copy of the state slice   [j][i]
    OT DT[DVS * Cf::PC];      // Delta^T                                 [j][r]
    OT Kt[kChunk * Cf::PK];   // Ktilde of the chunk                     [r][i]
    OT Ost[kChunk * Cf::PO];  // output staging                          [r][j]
    float gam[DK];
};

template <typename OT, int DK, int DVS>
__global__ __launch_bounds__(kThreads, 1) void gdr2_carry_kernel(FwdParams p) {
    using Cf = CarryCfg<OT, DK, DVS>;
    using MM = Mfma<OT>;
    using FR = Frag<OT>;
    constexpr int C = kChunk, KS = Cf::KS, PK = Cf::PK, PC = Cf::PC, PO = Cf::PO;
    constexpr int NKS = Cf::NKS, NCK = Cf::NCK, NJB = Cf::NJB, BPW = Cf::BPW, KVEC = Cf::KVEC;
    constexpr int VEC = 16 / (int)sizeof(OT);
    __shared__ CarrySmem<OT, DK, DVS> sm;

    const int tid = threadIdx.x, R = wave_id(), l = lane_id();
    const int work = xcd_swizzle(blockIdx.x, gridDim.x);
    const int chain = work / p.NS, slice = work % p.NS;
    const int bb = chain / p.H, h = chain % p.H;
    const int j0 = slice * DVS;
    const long T = p.T, H = p.H, DV = p.DV;
    const int NC = p.NC;
    OT* o = p.o ? (OT*)p.o + ((long)bb * T * H + h) * DV + j0 : nullptr;

    f32x4 Sacc[BPW];
#pragma unroll
    for (int u = 0; u < BPW; ++u) {
        const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s0 = 0.f;
            if (p.S0) s0 = p.S0[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()];
            Sacc[u][e] = s0;
        }
        store_acc_T(sm.ST, PK, 16 * jb, 16 * ib, Sacc[u]);
    }

    // Factor registers: two buffers used in turn, so that the loads for chunk c+1 are in flight
    // (into the other buffer) while chunk c computes.
    struct Buf {
        typename FR::t Y[NKS], Q[NKS], P[NCK];
        typename Raw4<OT>::t U[NJB];
        i32x4 K[KVEC];
        f32x4 g;
    };
    auto fetch = [&](Buf& b, int cc) __attribute__((always_inline)) {
        const long cix = (long)chain * NC + cc;
        const OT* Yc = (const OT*)p.wy.Yh + cix * C * DK;
        const OT* Qc = (const OT*)p.wy.Qg + cix * C * DK;
        const OT* Pc = (const OT*)p.wy.P + cix * C * C;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            b.Y[ks] = FFrag<OT>::fkc(Yc, DK, 16 * R, ks * KS);
            b.Q[ks] = FFrag<OT>::fkc(Qc, DK, 16 * R, ks * KS);
        }
#pragma unroll
        for (int kk = 0; kk < NCK; ++kk) b.P[kk] = FFrag<OT>::fkc(Pc, C, 16 * R, kk * KS);
        const OT* Uc = (const OT*)p.wy.U + cix * C * DV;
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
            b.U[jb] = *(const typename Raw4<OT>::t*)(Uc + ((long)(R * (DV / 16) + slice * NJB + jb) * 64 + l) * 4);
        const OT* Kc = (const OT*)p.wy.Kt + cix * C * DK;
#pragma unroll
        for (int m = 0; m < KVEC; ++m) b.K[m] = *(const i32x4*)(Kc + (long)(tid + m * kThreads) * VEC);
        if (tid < DK / 4) b.g = *(const f32x4*)(p.wy.gam + cix * DK + 4 * tid);
    };
    auto chunk = [&](const Buf& cur, Buf& nxt, int c) __attribute__((always_inline)) {
        const long t0 = (long)c * C;
        // ---- step 1: stage Ktilde / gamma, checkpoint, Delta = U - Y S, O = Qbar S
#pragma unroll
        for (int m = 0; m < KVEC; ++m) {  // fragment order -> row-major
            const int x = tid + m * kThreads;
            *(i32x4*)(sm.Kt + FLay<OT>::unit_row(x, DK) * PK + FLay<OT>::unit_col(x, DK)) = cur.K[m];
        }
        if (tid < DK / 4) *(f32x4*)(sm.gam + 4 * tid) = cur.g;
        if (c + 1 < NC) fetch(nxt, c + 1);
        if (p.states) {
            OT* dst = (OT*)p.states + (((long)chain * NC + c) * DV + j0) * DK;
            constexpr int NSV = DVS * DK / VEC;
#pragma unroll
            for (int x0 = 0; x0 < NSV; x0 += kThreads) {
                const int x = x0 + tid;
                if (NSV % kThreads == 0 || x < NSV) {
                    const int j = (x * VEC) / DK, i = (x * VEC) % DK;
                    *(i32x4*)(dst + (long)j * DK + i) = *(const i32x4*)(sm.ST + j * PK + i);
                }
            }
        }
        f32x4 aD[NJB], aO[NJB];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            aD[jb] = Raw4<OT>::widen(cur.U[jb]);
            aO[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                typename FR::t bS = FR::kc(sm.ST, PK, 16 * jb, ks * KS);
                MM::mma(aD[jb], cur.Y[ks], bS);
                MM::mma(aO[jb], cur.Q[ks], bS);
            }
        }
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) store_acc_T(sm.DT, PC, 16 * jb, 16 * R, aD[jb]);
        lds_barrier();

        // ---- step 2: O += P Delta, S' = Diag(gamma) S + Ktilde^T Delta
#pragma unroll
        for (int kk = 0; kk < NCK; ++kk) {
            if (kk * KS < 16 * R + 16) {
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) MM::mma(aO[jb], cur.P[kk], FR::kc(sm.DT, PC, 16 * jb, kk * KS));
            }
        }
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.Ost[(16 * R + acc_row(e)) * PO + 16 * jb + acc_col()] = from_f<OT>(aO[jb][e]);
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e) Sacc[u][e] *= sm.gam[16 * ib + acc_row(e)];
#pragma unroll
            for (int kk = 0; kk < NCK; ++kk)
                MM::mma(Sacc[u], FR::tr(sm.Kt, PK, kk * KS, 16 * ib), FR::kc(sm.DT, PC, 16 * jb, kk * KS));
            store_acc_T(sm.ST, PK, 16 * jb, 16 * ib, Sacc[u]);
        }
        lds_barrier();
        // ---- output tile to HBM
        if (o) {
            constexpr int NV = C * DVS / 4;
#pragma unroll
            for (int x0 = 0; x0 < NV; x0 += kThreads) {
                const int x = x0 + tid;
                const int rr = (x * 4) / DVS, j = (x * 4) % DVS;
                const long t = t0 + rr;
                if ((NV % kThreads == 0 || x < NV) && t < T) {
                    const OT* sp = sm.Ost + rr * PO + j;
                    store4(o + t * H * DV + j, f32x4{to_f(sp[0]), to_f(sp[1]), to_f(sp[2]), to_f(sp[3])});
                }
            }
        }
    };

    Buf bA, bB;
    if (NC > 0) fetch(bA, 0);
    lds_barrier();
    for (int c = 0; c < NC; c += 2) {
        chunk(bA, bB, c);
        if (c + 1 < NC) chunk(bB, bA, c + 1);
    }
    if (p.ST) {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                p.ST[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()] = Sacc[u][e];
        }
    }
}

// --------------------------------------------------------------------------------------------
// State carry with loader waves (16-bit operands).  Eight waves: waves 0-3 compute (wave R owns
// token block R, as in gdr2_carry_kernel) and write the outputs; waves 4-7 only load.  While
// chunk c computes out of one LDS slot, the loader waves copy chunk c + 1 (loaded into their
// registers two steps earlier) into the other slot and issue the loads of chunk c + 3, so a
// load has two steps to arrive.  The compute waves issue no global load, so the memory pipeline
// never stalls them, and the loader waves issue no store, so their waits cover loads only.
template <int DK, int DVS>
struct CarryLCfg {
    static constexpr int C = kChunk, KS = 32;
    static constexpr int PK = DK + 8, PC = C + 8, PO = DVS + 8;
    static constexpr int NKS = DK / KS, NCK = C / KS, NJB = DVS / 16, NIB = DK / 16;
    static constexpr int BPW = NIB * NJB / kWaves;
    // slot layout (bf16 elements): Y, Q, K [C][DK] and P [C][C] in fragment order, then the U
    // slice [4 token blocks][NJB][64 lanes][4] (accumulator order)
    static constexpr int OY = 0, OQ = C * DK, OK = 2 * C * DK, OP = 3 * C * DK, OU = OP + C * C;
    static constexpr int SLOT = OU + C * DVS;
    // 16-byte units of one chunk: the slot, then gamma (DK fp32)
    static constexpr int UM = C * DK / 8, UP = C * C / 8, UU = C * DVS / 8, UG = DK / 4;
    static constexpr int NUNIT = 3 * UM + UP + UU + UG;
    static constexpr int LPT = (NUNIT + kThreads - 1) / kThreads;   // units per loader thread
    static_assert(BPW >= 1 && BPW * kWaves == NIB * NJB, "state block mapping");
    static_assert(UM % kThreads == 0 && UP % kThreads == 0, "loader unit regions");
};

template <int DK, int DVS>
struct alignas(16) CarryLSmem {
    using Cf = CarryLCfg<DK, DVS>;
    bf16 slot[2][Cf::SLOT];
    float gam[2][DK];
    bf16 ST[DVS * Cf::PK];     // S^T operand copy   [j][i]
    bf16 DT[DVS * Cf::PC];     // Delta^T            [j][r]
    bf16 Ost[kChunk * Cf::PO]; // output staging     [r][j]
};

template <int DK, int DVS>
__global__ __launch_bounds__(2 * kThreads, 1) void gdr2_carry_lds_kernel(FwdParams p) {
    using Cf = CarryLCfg<DK, DVS>;
    using MM = Mfma<bf16>;
    using FR = Frag<bf16>;
    using FF = FFrag<bf16>;
    constexpr int C = kChunk, KS = Cf::KS, PK = Cf::PK, PC = Cf::PC, PO = Cf::PO;
    constexpr int NKS = Cf::NKS, NCK = Cf::NCK, NJB = Cf::NJB, BPW = Cf::BPW, LPT = Cf::LPT;
    __shared__ CarryLSmem<DK, DVS> sm;

    const int tid = threadIdx.x, w = wave_id(), l = lane_id();
    const bool loader = w >= kWaves;
    const int R = w & 3, lt = tid & (kThreads - 1);
    const int work = xcd_swizzle(blockIdx.x, gridDim.x);
    const int chain = work / p.NS, slice = work % p.NS;
    const int bb = chain / p.H, h = chain % p.H;
    const int j0 = slice * DVS;
    const long T = p.T, H = p.H, DV = p.DV;
    const int NC = p.NC, c0 = p.c0, NR = p.ncr;  // chunks [c0, c0 + NR) of NC
    bf16* o = p.o ? (bf16*)p.o + ((long)bb * T * H + h) * DV + j0 : nullptr;

    // ---- loader: unit x = lt + kThreads * m of chunk cc (the region of x depends on m only)
    auto src_unit = [&](int cc, int m) __attribute__((always_inline)) -> const i32x4* {
        const long cix = (long)chain * NC + cc;
        int x = lt + kThreads * m;
        if (x >= Cf::NUNIT) x = Cf::NUNIT - 1;  // padding lanes reload the last unit
        if (x < 3 * Cf::UM) {
            const int mat = x / Cf::UM, u = x % Cf::UM;
            const bf16* base = mat == 0 ? (const bf16*)p.wy.Yh : mat == 1 ? (const bf16*)p.wy.Qg : (const bf16*)p.wy.Kt;
            return (const i32x4*)(base + cix * C * DK + u * 8);
        }
        x -= 3 * Cf::UM;
        if (x < Cf::UP) return (const i32x4*)((const bf16*)p.wy.P + cix * C * C + x * 8);
        x -= Cf::UP;
        if (x < Cf::UU) {
            const int rb = x / (NJB * 32), within = x % (NJB * 32);
            return (const i32x4*)((const bf16*)p.wy.U + cix * C * DV +
                                  ((long)(rb * (DV / 16) + slice * NJB) * 64) * 4 + within * 8);
        }
        x -= Cf::UU;
        return (const i32x4*)(p.wy.gam + cix * DK + 4 * x);
    };
    auto put_unit = [&](int sl, int m, const i32x4& v) __attribute__((always_inline)) {
        int x = lt + kThreads * m;
        if (x >= Cf::NUNIT) return;
        if (x < 3 * Cf::UM + Cf::UP + Cf::UU) {
            *(i32x4*)(sm.slot[sl] + x * 8) = v;  // Y, Q, K, P, U are contiguous in the slot
        } else {
            *(i32x4*)(sm.gam[sl] + 4 * (x - 3 * Cf::UM - Cf::UP - Cf::UU)) = v;
        }
    };
    i32x4 lbA[LPT], lbB[LPT];  // loader registers: chunk k >= 1 lives in lbA (k odd) or lbB (k even)

    f32x4 Sacc[BPW];
    if (!loader) {
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float s0 = 0.f;
                if (p.S0) s0 = p.S0[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()];
                Sacc[u][e] = s0;
            }
            store_acc_T(sm.ST, PK, 16 * jb, 16 * ib, Sacc[u]);
        }
    } else if (NR > 0) {
        // chunk c0 into slot 0 (through lbB), then chunks c0 + 1 and c0 + 2 into the registers
        // (clamped to the range)
#pragma unroll
        for (int m = 0; m < LPT; ++m) lbB[m] = *src_unit(c0, m);
#pragma unroll
        for (int m = 0; m < LPT; ++m) put_unit(0, m, lbB[m]);
#pragma unroll
        for (int m = 0; m < LPT; ++m) lbA[m] = *src_unit(c0 + (NR > 1 ? 1 : NR - 1), m);
#pragma unroll
        for (int m = 0; m < LPT; ++m) lbB[m] = *src_unit(c0 + (NR > 2 ? 2 : NR - 1), m);
    }
    lds_barrier();

    // loader step cc (counted from c0): chunk cc + 1 (registers `cur`) into slot (cc + 1) & 1,
    // then the loads of chunk cc + 3 into the same registers (clamped to the range's last chunk,
    // so that every step issues the same loads and the waits stay exact, and nothing outside the
    // range is read), half before and half after the mid-step barrier
    auto loader_step = [&](int cc, i32x4* cur) __attribute__((always_inline)) {
        if (cc + 1 < NR) {
#pragma unroll
            for (int m = 0; m < LPT; ++m) put_unit((cc + 1) & 1, m, cur[m]);
        }
        const int c3 = c0 + (cc + 3 < NR ? cc + 3 : NR - 1);
#pragma unroll
        for (int m = 0; m < LPT / 2; ++m) cur[m] = *src_unit(c3, m);
        lds_barrier();
#pragma unroll
        for (int m = LPT / 2; m < LPT; ++m) cur[m] = *src_unit(c3, m);
        lds_barrier();
    };
    auto compute_step = [&](int c, int sl) __attribute__((always_inline)) {
        const long t0 = (long)c * C;
        // outputs of the previous step: checkpoint of the state entering chunk c, O of chunk c-1
        // (of this launch's range)
        if (p.states) {
            bf16* dst = (bf16*)p.states + (((long)chain * NC + c) * DV + j0) * DK;
            constexpr int NSV = DVS * DK / 8;
#pragma unroll
            for (int x0 = 0; x0 < NSV; x0 += kThreads) {
                const int x = x0 + tid;
                if (NSV % kThreads == 0 || x < NSV) {
                    const int j = (x * 8) / DK, i = (x * 8) % DK;
                    store_stream((i32x4*)(dst + (long)j * DK + i), *(const i32x4*)(sm.ST + j * PK + i));
                }
            }
        }
        if (o && c > c0) {
            constexpr int NV = C * DVS / 8;
#pragma unroll
            for (int x0 = 0; x0 < NV; x0 += kThreads) {
                const int x = x0 + tid;
                const int rr = (x * 8) / DVS, j = (x * 8) % DVS;
                const long t = t0 - C + rr;
                if ((NV % kThreads == 0 || x < NV) && t < T)
                    *(i32x4*)(o + t * H * DV + j) = *(const i32x4*)(sm.Ost + rr * PO + j);
            }
        }
        const bf16* Ys = sm.slot[sl] + Cf::OY;
        const bf16* Qs = sm.slot[sl] + Cf::OQ;
        const bf16* Ks = sm.slot[sl] + Cf::OK;
        const bf16* Ps = sm.slot[sl] + Cf::OP;
        const bf16* Us = sm.slot[sl] + Cf::OU;
        // ---- Delta = U - Y S (stored -Y), O = Qbar S
        f32x4 aD[NJB], aO[NJB];
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
            aD[jb] = Raw4<bf16>::widen(*(const bf16x4*)(Us + ((R * NJB + jb) * 64 + l) * 4));
            aO[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            const bf16x8 ay = FF::fkc(Ys, DK, 16 * R, ks * KS), aq = FF::fkc(Qs, DK, 16 * R, ks * KS);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                const bf16x8 bS = FR::kc(sm.ST, PK, 16 * jb, ks * KS);
                MM::mma(aD[jb], ay, bS);
                MM::mma(aO[jb], aq, bS);
            }
        }
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb) store_acc_T(sm.DT, PC, 16 * jb, 16 * R, aD[jb]);
        lds_barrier();
        // ---- O += P Delta, S' = Diag(gamma) S + Ktilde^T Delta.  Every operand fragment is read
        // from LDS once: Delta^T per (k-step, value block), Ktilde^T per (key block, k-step) -- this
        // wave's state blocks come in groups of NJB that share one key block.
        bf16x8 dtf[NCK][NJB];
#pragma unroll
        for (int kk = 0; kk < NCK; ++kk)
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) dtf[kk][jb] = FR::kc(sm.DT, PC, 16 * jb, kk * KS);
#pragma unroll
        for (int kk = 0; kk < NCK; ++kk) {
            if (kk * KS < 16 * R + 16) {
                const bf16x8 ap = FF::fkc(Ps, C, 16 * R, kk * KS);
#pragma unroll
                for (int jb = 0; jb < NJB; ++jb) MM::mma(aO[jb], ap, dtf[kk][jb]);
            }
        }
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                sm.Ost[(16 * R + acc_row(e)) * PO + 16 * jb + acc_col()] = (bf16)aO[jb][e];
#pragma unroll
        for (int v = 0; v < BPW / NJB; ++v) {
            const int ib = R * BPW / NJB + v;
            const f32x4 gm = *(const f32x4*)(sm.gam[sl] + 16 * ib + 4 * (l >> 4));
            bf16x8 kf[NCK];
#pragma unroll
            for (int kk = 0; kk < NCK; ++kk) kf[kk] = FF::ftr(Ks, DK, kk * KS, 16 * ib);
#pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
                f32x4& acc = Sacc[v * NJB + jb];
                acc *= gm;
#pragma unroll
                for (int kk = 0; kk < NCK; ++kk) MM::mma(acc, kf[kk], dtf[kk][jb]);
            }
        }
#pragma unroll
        for (int u = 0; u < BPW; ++u) {
            const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
            store_acc_T(sm.ST, PK, 16 * jb, 16 * ib, Sacc[u]);
        }
        lds_barrier();
    };

    // Steps run in pairs (the register alternation); a step past the range's last chunk only keeps
    // the barrier count of the two roles equal.
    const int NCR = (NR + 1) / 2 * 2;
    if (loader) {
        for (int c = 0; c < NCR; c += 2) {
            loader_step(c, lbA);
            loader_step(c + 1, lbB);
        }
    } else {
        for (int c = 0; c < NCR; c += 2) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                if (c + u < NR) {
                    compute_step(c0 + c + u, (c + u) & 1);
                } else {
                    lds_barrier();
                    lds_barrier();
                }
            }
        }
        if (o && NR > 0) {  // output tile of the range's last chunk
            const long t0 = (long)(c0 + NR - 1) * C;
            constexpr int NV = C * DVS / 8;
#pragma unroll
            for (int x0 = 0; x0 < NV; x0 += kThreads) {
                const int x = x0 + tid;
                const int rr = (x * 8) / DVS, j = (x * 8) % DVS;
                const long t = t0 + rr;
                if ((NV % kThreads == 0 || x < NV) && t < T)
                    *(i32x4*)(o + t * H * DV + j) = *(const i32x4*)(sm.Ost + rr * PO + j);
            }
        }
        if (p.ST) {
#pragma unroll
            for (int u = 0; u < BPW; ++u) {
                const int bi = R * BPW + u, ib = bi / NJB, jb = bi % NJB;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p.ST[((long)chain * DK + 16 * ib + acc_row(e)) * DV + j0 + 16 * jb + acc_col()] = Sacc[u][e];
            }
        }
    }
}

template <typename OT, int DK, int DVS>
static hipError_t launch_carry(const FwdParams& p, hipStream_t s) {
    const long nblk = (long)p.B * p.H * p.NS;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((gdr2_carry_kernel<OT, DK, DVS>), dim3(nblk), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int DK, int DVS>
static hipError_t launch_carry_lds(const FwdParams& p, hipStream_t s) {
    const long nblk = (long)p.B * p.H * p.NS;
    if (nblk == 0) return hipSuccess;
    hipLaunchKernelGGL((gdr2_carry_lds_kernel<DK, DVS>), dim3(nblk), dim3(2 * kThreads), 0, s, p);
    return hipGetLastError();
}

int carry_slice_width(int bf, int dk, int dv, long chains) {
    // widest slice that still gives >= 256 workgroups; 64-wide slices only where the bf16
    // two-slot LDS carry fits (d_k = 64)
    const int cands[3] = {64, 32, 16};
    for (int x = (bf && dk == 64) ? 0 : 1; x < 3; ++x)
        if (cands[x] <= dv && chains * (dv / cands[x]) >= 256) return cands[x];
    return 16;
}

hipError_t carry_fwd_dispatch(int bf, int dk, int dvs, const FwdParams& p, hipStream_t s) {
    if (bf) {
        if (dk == 128 && dvs == 32) return launch_carry_lds<128, 32>(p, s);
        if (dk == 128 && dvs == 16) return launch_carry_lds<128, 16>(p, s);
        if (dk == 64 && dvs == 64) return launch_carry_lds<64, 64>(p, s);
        if (dk == 64 && dvs == 32) return launch_carry_lds<64, 32>(p, s);
        if (dk == 64 && dvs == 16) return launch_carry_lds<64, 16>(p, s);
    } else {
        if (dk == 128 && dvs == 32) return launch_carry<float, 128, 32>(p, s);
        if (dk == 128 && dvs == 16) return launch_carry<float, 128, 16>(p, s);
        if (dk == 64 && dvs == 32) return launch_carry<float, 64, 32>(p, s);
        if (dk == 64 && dvs == 16) return launch_carry<float, 64, 16>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
