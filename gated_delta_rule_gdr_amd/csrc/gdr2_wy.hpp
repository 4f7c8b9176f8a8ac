// gdr2_wy.hpp -- per-chunk WY factors of the Gated Delta Rule-2 chunk form (device code).
//
// One workgroup (4 waves) handles one chunk of C = 64 tokens of one (batch, head) chain.  Wave R
// owns token rows 16R .. 16R+15; lane l owns row 16R + l%16 and, of every channel vector, the
// channels ks*KS + KPL*(l/16) + j -- exactly the MFMA operand layout, so the gate prep feeds the
// Gram products straight from registers.
//
// Chunk algebra (per chunk; G_r = inclusive cumsum of log alpha inside the chunk, e = b . k,
// z = w . v): the cumulative channel-wise decay is absorbed into the two factors of each rank-one
// erase (ainews.random.gg article on Gated DeltaNet-2, section "Chunkwise training and gate-aware
// backward"):
//     A_rs = sum_i e_ri exp(G_ri - G_si) k_si   (r > s)      T = (I + A)^-1
//     P_rs = sum_i q_ri exp(G_ri - G_si) k_si   (r >= s)
//     Y = T (E . e^G),   U = T Z,   Qbar = Q . e^G,   Ktilde = K . e^{G_C - G},   gamma = e^{G_C}.
#pragma once
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <typename OT, int DK, int DV>
struct WyCfg {
    static constexpr int C = kChunk;
    static constexpr int KS = Mfma<OT>::KS, KPL = Mfma<OT>::KPL;
    static constexpr int PAD = 16 / (int)sizeof(OT);
    static constexpr int PK = DK + PAD, PV = DV + PAD, PC = C + PAD;
    static constexpr int PAF = C + 4;                      // fp32 A / T pitch, 16-byte rows
    static constexpr int NKS = DK / KS, NVS = DV / KS;     // k-steps over key / value channels
    static constexpr int NCH = NKS * KPL, NCV = NVS * KPL; // channels per lane (DK/4, DV/4)
};

template <typename OT, int DK, int DV>
struct alignas(16) WySmem {
    using Cf = WyCfg<OT, DK, DV>;
    union {
        OT Kb[kChunk * Cf::PK];  // phase 1: k . exp(ref_S - G)          [s][i]
        struct {
            OT Eg[kChunk * Cf::PK];  // phase 2: e . exp(G)              [s][i]
            OT Z[kChunk * Cf::PV];   // phase 2: z = w . v               [s][j]
        } e;
    } u;
    float Af[kChunk * Cf::PAF];  // A (strict lower), then T in fp32 (see tblk)
    OT Tm[kChunk * Cf::PC];      // T in operand precision           [r][s]
    float Mf[kWaves][16 * 17];   // per-wave scratch of the solve
    float tot[4][DK];            // per-block log-decay totals
    float ctab[6][DK];           // exp(ref_R - ref_S), R > S
    float gRt[4][DK];            // exp(ref_R)
    float hRt[4][DK];            // exp(G_C - ref_R)
    float hRl[4][DK];            // G_C - ref_R (deep-decay path)
    int deep[4];                 // block R decays by more than exp(-kDeepDecay) on some channel
};

// Location of block T_RS of the inverse inside Af: diagonal blocks overwrite A_RR, off-diagonal
// blocks live in the (unused) strictly upper block (S, R) so that A_RK stays readable.
template <int PAF>
__device__ __forceinline__ float* tblk(float* Af, int R, int S) {
    return R == S ? Af + 16 * R * PAF + 16 * R : Af + 16 * S * PAF + 16 * R;
}

// fp32 16x16 block products on the 16x16x4 MFMA with the k order 4g + j (g = lane / 16, j = the
// MFMA step): lane (i = lane % 16, g) supplies X[i][4g + j] of the left block -- a 16-byte read of
// its row -- and Y[4g + j][i] of the right one, which is element j of the accumulator that holds
// Y in the calling wave.  A product therefore feeds the next one from registers.
__device__ __forceinline__ f32x4 lhs4_f32(const float* X, int p, int l) {
    return *(const f32x4*)(X + (l & 15) * p + 4 * (l >> 4));
}
__device__ __forceinline__ f32x4 rhs4_f32(const float* Y, int p, int l) {
    const float* y = Y + 4 * (l >> 4) * p + (l & 15);
    return f32x4{y[0], y[p], y[2 * p], y[3 * p]};
}
__device__ __forceinline__ void mm16_f32(f32x4& c, const f32x4& a, const f32x4& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) mma32(c, a[j], b[j]);
}

// Zero the blocks of Tm above the diagonal (T is lower triangular).  Nothing else touches Tm
// before the solve, so this runs at the start of the workgroup, off the solve's path.
template <typename OT, int PC>
__device__ __forceinline__ void zero_upper_T(OT* Tm) {
    constexpr int V = 16 / (int)sizeof(OT), PER_ROW = 16 / V;  // 16-byte stores per block row
    for (int x = threadIdx.x; x < 6 * 16 * PER_ROW; x += kThreads) {
        const int blk = x / (16 * PER_ROW), e = x % (16 * PER_ROW);
        const int R = blk < 3 ? 0 : blk < 5 ? 1 : 2;
        const int S = blk < 3 ? blk + 1 : blk < 5 ? blk - 1 : 3;
        *(i32x4*)(Tm + (16 * R + e / PER_ROW) * PC + 16 * S + (e % PER_ROW) * V) = i32x4{0, 0, 0, 0};
    }
}

// T = (I + A)^-1 for the strictly lower 64 x 64 A held in Af (fp32), 16 x 16 blocked; the upper
// blocks of Tm must already be zero (zero_upper_T).  Diagonal blocks by forward substitution
// (wave R, lane = column), then the off-diagonal blocks from T_RS = -T_RR sum_{S <= K < R} A_RK T_KS
// in three barrier-separated steps that keep all four waves busy:
//     1: T10 = -T11 (A10 T00), T32 = -T33 (A32 T22), M21 = A21 T11, M31 = A31 T11,
//        and the first terms of M20 = A20 T00 + A21 T10, M30 = A30 T00 + A31 T10;
//     2: M20, M30 completed, T21 = -T22 M21, T31 = -(T32 M21 + T33 M31);
//     3: T20 = -T22 M20, T30 = -(T32 M20 + T33 M30).
// T is written in operand precision to Tm (row-major); the fp32 copies in Af are kept only for the
// blocks a later step reads (the diagonal, T10, T32).  Ends with a barrier.
template <typename OT, int PAF, int PC>
__device__ __forceinline__ void solve_unit_lower_64(float* Af, float (*Mf)[16 * 17], OT* Tm) {
    const int w = wave_id(), l = lane_id(), g = l >> 4, c = l & 15;
    const auto A = [&](int R, int S) { return Af + 16 * R * PAF + 16 * S; };  // A_RS, R > S
    const auto T = [&](int R, int S) { return tblk<PAF>(Af, R, S); };
    const auto put_T = [&](int R, int S, const f32x4& v, bool keep_f32) {
        float* t = T(R, S);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (keep_f32) t[acc_row(e, l) * PAF + acc_col(l)] = v[e];
            Tm[(16 * R + acc_row(e, l)) * PC + 16 * S + acc_col(l)] = from_f<OT>(v[e]);
        }
    };
    const auto put_M = [&](float* M, const f32x4& v) {
#pragma unroll
        for (int e = 0; e < 4; ++e) M[acc_row(e, l) * 17 + acc_col(l)] = v[e];
    };
    const auto neg = [](const f32x4& v) { return f32x4{-v[0], -v[1], -v[2], -v[3]}; };
    constexpr f32x4 Z4 = {0.f, 0.f, 0.f, 0.f};

    // diagonal block T_ww, column c (the four lane groups compute it alike; group g keeps rows
    // 4g .. 4g+3, which is T_ww in accumulator layout)
    f32x4 tw;
    {
        const float* Ab = A(w, w);
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == c) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s) acc -= Ab[r * PAF + s] * x[s];
            x[r] = acc;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tw[i] = g == 0 ? x[i] : g == 1 ? x[4 + i] : g == 2 ? x[8 + i] : x[12 + i];
    }
    wave_sync();  // A_ww is read in full before T_ww overwrites it
    put_T(w, w, tw, true);
    lds_barrier();

    f32x4 m0 = Z4, m1 = Z4;
    if (w == 0) {
        mm16_f32(m0, lhs4_f32(A(1, 0), PAF, l), tw);
        mm16_f32(m1, lhs4_f32(T(1, 1), PAF, l), m0);
        put_T(1, 0, neg(m1), true);
    } else if (w == 1) {
        mm16_f32(m0, lhs4_f32(A(2, 1), PAF, l), tw);
        mm16_f32(m1, lhs4_f32(A(3, 1), PAF, l), tw);
        put_M(Mf[2], m0);
        put_M(Mf[3], m1);
    } else if (w == 2) {
        mm16_f32(m0, lhs4_f32(A(3, 2), PAF, l), tw);
        mm16_f32(m1, lhs4_f32(T(3, 3), PAF, l), m0);
        put_T(3, 2, neg(m1), true);
    } else {
        const f32x4 t00 = rhs4_f32(T(0, 0), PAF, l);
        mm16_f32(m0, lhs4_f32(A(2, 0), PAF, l), t00);
        mm16_f32(m1, lhs4_f32(A(3, 0), PAF, l), t00);
    }
    lds_barrier();

    if (w == 3) {
        const f32x4 t10 = rhs4_f32(T(1, 0), PAF, l);
        mm16_f32(m0, lhs4_f32(A(2, 1), PAF, l), t10);
        mm16_f32(m1, lhs4_f32(A(3, 1), PAF, l), t10);
        put_M(Mf[0], m0);
        put_M(Mf[1], m1);
    } else if (w == 0) {
        f32x4 n = Z4;
        mm16_f32(n, lhs4_f32(T(2, 2), PAF, l), rhs4_f32(Mf[2], 17, l));
        put_T(2, 1, neg(n), false);
    } else if (w == 1) {
        f32x4 n = Z4;
        mm16_f32(n, lhs4_f32(T(3, 2), PAF, l), rhs4_f32(Mf[2], 17, l));
        mm16_f32(n, lhs4_f32(T(3, 3), PAF, l), rhs4_f32(Mf[3], 17, l));
        put_T(3, 1, neg(n), false);
    }
    lds_barrier();

    if (w == 0) {
        f32x4 n = Z4;
        mm16_f32(n, lhs4_f32(T(2, 2), PAF, l), rhs4_f32(Mf[0], 17, l));
        put_T(2, 0, neg(n), false);
    } else if (w == 1) {
        f32x4 n = Z4;
        mm16_f32(n, lhs4_f32(T(3, 2), PAF, l), rhs4_f32(Mf[0], 17, l));
        mm16_f32(n, lhs4_f32(T(3, 3), PAF, l), rhs4_f32(Mf[1], 17, l));
        put_T(3, 0, neg(n), false);
    }
    lds_barrier();
}

// The KPL values of k-step ks that lane group g owns in a row: channels ks*KS + KPL*g + j.
template <typename OT>
__device__ __forceinline__ void load_lane(const OT* row, int ks, int g, float* out) {
    if constexpr (sizeof(OT) == 2) {
        bf16x8 x = *(const bf16x8*)(row + ks * 32 + 8 * g);
#pragma unroll
        for (int j = 0; j < 8; ++j) out[j] = (float)x[j];
    } else {
        out[0] = row[ks * 4 + g];
    }
}
template <typename OT>
__device__ __forceinline__ void load_lane_f32(const float* row, int ks, int g, float* out) {
    if constexpr (sizeof(OT) == 2) {
        f32x4 a = *(const f32x4*)(row + ks * 32 + 8 * g), b = *(const f32x4*)(row + ks * 32 + 8 * g + 4);
        out[0] = a[0]; out[1] = a[1]; out[2] = a[2]; out[3] = a[3];
        out[4] = b[0]; out[5] = b[1]; out[6] = b[2]; out[7] = b[3];
    } else {
        out[0] = row[ks * 4 + g];
    }
}
template <typename OT>
__device__ __forceinline__ void store_lane(OT* row, int ks, int g, const float* v) {
    if constexpr (sizeof(OT) == 2) {
        *(bf16x8*)(row + ks * 32 + 8 * g) = Frag<bf16>::from_f32(v);
    } else {
        row[ks * 4 + g] = v[0];
    }
}
// The same KPL values stored into a fragment-order tile of `cols` columns (row r).
template <typename OT, bool STREAM>
__device__ __forceinline__ void store_lane_F(OT* tile, int cols, int r, int ks, int g, const float* v) {
    if constexpr (sizeof(OT) == 2) {
        bf16x8* d = (bf16x8*)(tile + FLay<OT>::off(r, ks * 32 + 8 * g, cols));
        if constexpr (STREAM) store_stream(d, Frag<bf16>::from_f32(v));
        else *d = Frag<bf16>::from_f32(v);
    } else {
        tile[FLay<OT>::off(r, ks * 4 + g, cols)] = v[0];
    }
}
__device__ __forceinline__ void store_lane_f32(float* row, int ks, int g, const float* v, int kpl) {
    if (kpl == 8) {
        *(f32x4*)(row + ks * 32 + 8 * g) = f32x4{v[0], v[1], v[2], v[3]};
        *(f32x4*)(row + ks * 32 + 8 * g + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
        row[ks * 4 + g] = v[0];
    }
}

// Where one workgroup's chunk lives.
template <typename OT, int DK, int DV>
struct WyChunk {
    int chain, c, R, l, rl, g, r;
    long T, H, DVl, row, cix;
    bool valid;
    const OT *q, *k, *b, *v, *w;
    const float* la;
    int gates;
    Prologue pro;
    // chunks [c0, c0 + ncr) of the NC of the sequence, one workgroup each
    __device__ WyChunk(int B, int H_, long T_, long DV_, int NC, int c0, int ncr, int gates_, Prologue pro_, int bid,
                       const void* q_, const void* k_, const void* b_, const float* la_, const void* v_,
                       const void* w_) {
        gates = gates_;
        pro = pro_;
        (void)B;
        // heads fastest: concurrent workgroups share the token rows of the [B, T, H, D] inputs
        const int h = bid % H_, bb = bid / (H_ * ncr);
        c = c0 + (bid / H_) % ncr;
        chain = bb * H_ + h;
        R = wave_id();
        l = lane_id();
        rl = l & 15;
        g = l >> 4;
        T = T_;
        H = H_;
        DVl = DV_;
        r = 16 * R + rl;
        const long t = (long)c * kChunk + r;
        valid = t < T;
        const long tt = valid ? t : T - 1;
        row = ((long)bb * T + tt) * H + h;
        cix = (long)chain * NC + c;
        q = (const OT*)q_ + row * DK;
        k = (const OT*)k_ + row * DK;
        b = (const OT*)b_ + row * ((gates & kEraseScalar) ? 1 : DK);
        la = la_ + row * ((gates & kDecayScalar) ? 1 : DK);
        v = (const OT*)v_ + row * DV_;
        w = (const OT*)w_ + row * ((gates & kWriteScalar) ? 1 : DV_);
    }
};

// Compute and store the WY factors of one chunk (see the file comment); every thread of the
// workgroup calls it.  MODE (kModePlain / kModeGates / kModePrologue / kModePrologueChannel /
// kModeFixedGates + bits): the plain, fixed-gates and channel-wise prologue instances have no gate
// branches, so their loads issue back to back; the others read the gate bits at run time.  STREAM: write the
// factor tiles with streaming stores (a
// separate instance: a run-time choice between the two store kinds is folded into one plain
// store by the compiler).
template <typename OT, int DK, int DV, int MODE, bool STREAM>
__device__ __forceinline__ void wy_factors(WySmem<OT, DK, DV>& sm, const WyChunk<OT, DK, DV>& ch, const WyBufs& wy) {
    using Cf = WyCfg<OT, DK, DV>;
    using MM = Mfma<OT>;
    using FR = Frag<OT>;
    constexpr int C = kChunk, KS = Cf::KS, KPL = Cf::KPL, PK = Cf::PK, PV = Cf::PV;
    constexpr int PC = Cf::PC, PAF = Cf::PAF, NKS = Cf::NKS, NVS = Cf::NVS, NCH = Cf::NCH;
    constexpr int NCV = Cf::NCV;
    const int R = ch.R, l = ch.l, rl = ch.rl, g = ch.g, r = ch.r;
    const long cix = ch.cix, DVl = ch.DVl;
    constexpr bool GS = MODE != kModePlain, PRO = mode_prologue(MODE);

    zero_upper_T<OT, PC>(sm.Tm);
    float qv[NCH], kv[NCH], bv[NCH], lv[NCH], zv[NCV];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        load_lane<OT>(ch.q, ks, g, qv + ks * KPL);
        load_lane<OT>(ch.k, ks, g, kv + ks * KPL);
        if (GS && (gate_bits<MODE>(ch.gates) & kEraseScalar)) {
            const float bs = to_f(ch.b[0]);
#pragma unroll
            for (int j = 0; j < KPL; ++j) bv[ks * KPL + j] = bs;
        } else {
            load_lane<OT>(ch.b, ks, g, bv + ks * KPL);
        }
        if (GS && (gate_bits<MODE>(ch.gates) & kDecayScalar)) {
            const float ls = ch.la[0];
#pragma unroll
            for (int j = 0; j < KPL; ++j) lv[ks * KPL + j] = ls;
        } else {
            load_lane_f32<OT>(ch.la, ks, g, lv + ks * KPL);
        }
    }
#pragma unroll
    for (int ks = 0; ks < NVS; ++ks) {
        float vv[KPL], wv[KPL];
        load_lane<OT>(ch.v, ks, g, vv);
        if (GS && (gate_bits<MODE>(ch.gates) & kWriteScalar)) {
            const float ws = to_f(ch.w[0]);
#pragma unroll
            for (int j = 0; j < KPL; ++j) wv[j] = ws;
        } else {
            load_lane<OT>(ch.w, ks, g, wv);
        }
        if (PRO) {
#pragma unroll
            for (int j = 0; j < KPL; ++j) wv[j] = sigmoid_f(wv[j]);
        }
#pragma unroll
        for (int j = 0; j < KPL; ++j) zv[ks * KPL + j] = ch.valid ? vv[j] * wv[j] : 0.f;
    }
    if (PRO) {  // fused prologue: L2-normalised q, k; sigmoid gates; log alpha from softplus
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int n = 0; n < NCH; ++n) {
            sq += qv[n] * qv[n];
            sk += kv[n] * kv[n];
        }
        // the row's channels sit in the four lanes rl + 16 g
        sq += __shfl_xor(sq, 16);
        sq += __shfl_xor(sq, 32);
        sk += __shfl_xor(sk, 16);
        sk += __shfl_xor(sk, 32);
        const float rq = rsqrtf(sq + ch.pro.norm_eps), rk = rsqrtf(sk + ch.pro.norm_eps);
#pragma unroll
        for (int n = 0; n < NCH; ++n) {
            qv[n] *= rq;
            kv[n] *= rk;
            bv[n] = sigmoid_f(bv[n]);
            lv[n] = -ch.pro.decay_scale * softplus_f(lv[n]);
        }
    }
    if (!ch.valid) {
#pragma unroll
        for (int n = 0; n < NCH; ++n) qv[n] = kv[n] = bv[n] = lv[n] = 0.f;
    }
    // in-block inclusive cumsum of log alpha (16 lanes = 16 rows) and the block totals
#pragma unroll
    for (int n = 0; n < NCH; ++n) lv[n] = row_scan16(lv[n]);  // lv := G_r - ref_R
    {   // does this block decay past the fast path's range on some channel?
        float mn = 0.f;
#pragma unroll
        for (int n = 0; n < NCH; ++n) mn = fminf(mn, lv[n]);
        const unsigned long long deep = __ballot(rl == 15 && mn < -kDeepDecay);
        if (l == 0) sm.deep[R] = deep != 0ull;
    }
    if (rl == 15) {
#pragma unroll
        for (int n = 0; n < NCH; ++n) sm.tot[R][(n / KPL) * KS + KPL * g + n % KPL] = lv[n];
    }
    lds_barrier();
    // deep-decay path for the whole chunk (uniform over the workgroup)
    const bool deep = __builtin_amdgcn_readfirstlane((sm.deep[0] | sm.deep[1] | sm.deep[2] | sm.deep[3]) != 0);

    // per-channel tables from the block totals: ref_R = sum of earlier block totals,
    // exp(ref_R), exp(G_C - ref_R), exp(ref_R - ref_S) (R > S) and gamma = exp(G_C)
    for (int chn = threadIdx.x; chn < DK; chn += kThreads) {
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
        wy.gam[cix * DK + chn] = __expf(run);
    }
    OT* const pt = (OT*)wy.P + cix * C * C;  // P tile, fragment order
    if (deep) {
        // Diagonal 16 x 16 blocks of A and P entry by entry, each term carrying
        // exp(G_r - G_s) <= 1 (s <= r, same block): row s's k and G come from lane 16 g + s%16,
        // which holds the same channels.  A rolled loop over s keeps the register footprint of
        // this rare path small.
        float myA[4] = {0.f, 0.f, 0.f, 0.f}, myP[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int t = 0; t < 16; ++t) {
            const int src = 16 * g + t;
            float a = 0.f, pp = 0.f;
#pragma unroll
            for (int n = 0; n < NCH; ++n) {
                const float ks_ = __shfl(kv[n], src), ls_ = __shfl(lv[n], src);
                const float f = ks_ * __expf(fminf(lv[n] - ls_, 0.f));
                a += bv[n] * kv[n] * f;
                pp += qv[n] * f;
            }
            a += __shfl_xor(a, 16);
            a += __shfl_xor(a, 32);
            pp += __shfl_xor(pp, 16);
            pp += __shfl_xor(pp, 32);
            const bool mine = (t >> 2) == g;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                myA[e] = (mine && (t & 3) == e) ? a : myA[e];
                myP[e] = (mine && (t & 3) == e) ? pp : myP[e];
            }
        }
        f32x4 am, pm;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s_ = 16 * R + 4 * g + e;
            am[e] = s_ < r ? myA[e] : 0.f;
            pm[e] = s_ <= r ? myP[e] : 0.f;
        }
        *(f32x4*)(sm.Af + r * PAF + 16 * R + 4 * g) = am;
        store4(pt + FLay<OT>::off(r, 16 * R + 4 * g, C), pm);
    }
    lds_barrier();

    // decay-absorbed factors
    typename FR::t Ef[NKS], Qf[NKS];  // e . exp(G - ref_R), q . exp(G - ref_R) (Gram operands)
    float eg[NCH];                     // e . exp(G), kept for Y
    OT* qg_out = (OT*)wy.Qg + cix * C * DK;  // fragment-order tiles
    OT* kt_out = (OT*)wy.Kt + cix * C * DK;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        float ebk[KPL], qbk[KPL], kbk[KPL], qg[KPL], kt[KPL], gR[KPL], hR[KPL];
        load_lane_f32<OT>(sm.gRt[R], ks, g, gR);
        if (deep) {
            // right Gram operand referenced to the end of its block, exp(G_end - G_s) <= 1, and
            // Ktilde = k exp(G_C - G_r) from one exponent
            float tb[KPL], hl[KPL];
            load_lane_f32<OT>(sm.tot[R], ks, g, tb);
            load_lane_f32<OT>(sm.hRl[R], ks, g, hl);
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int n = ks * KPL + j;
                const float x = __expf(lv[n]);
                const float e = bv[n] * kv[n];
                ebk[j] = e * x;
                qbk[j] = qv[n] * x;
                kbk[j] = kv[n] * __expf(tb[j] - lv[n]);
                eg[n] = ebk[j] * gR[j];
                qg[j] = qbk[j] * gR[j];
                kt[j] = kv[n] * __expf(hl[j] - lv[n]);
            }
        } else {
            load_lane_f32<OT>(sm.hRt[R], ks, g, hR);
#pragma unroll
            for (int j = 0; j < KPL; ++j) {
                const int n = ks * KPL + j;
                const float x = __expf(lv[n]), y = __expf(-lv[n]);
                const float e = bv[n] * kv[n];
                ebk[j] = e * x;
                qbk[j] = qv[n] * x;
                kbk[j] = kv[n] * y;
                eg[n] = ebk[j] * gR[j];
                qg[j] = qbk[j] * gR[j];
                kt[j] = kbk[j] * hR[j];
            }
        }
        Ef[ks] = FR::from_f32(ebk);
        Qf[ks] = FR::from_f32(qbk);
        store_lane<OT>(sm.u.Kb + r * PK, ks, g, kbk);
        store_lane_F<OT, STREAM>(qg_out, DK, r, ks, g, qg);
        store_lane_F<OT, STREAM>(kt_out, DK, r, ks, g, kt);
    }
    lds_barrier();

    // A^T and P^T blocks (S, R) for S <= R: rows s of block S, columns r of block R.  The right
    // operand of block S carries exp(ref_S - G_s) with the cross-block factor exp(ref_R - ref_S)
    // -- on the deep-decay path exp(G_end(S) - G_s) with exp(ref_R - ref_{S+1}) (the diagonal
    // blocks are done then).
    {
#pragma unroll
        for (int S = 0; S < 4; ++S) {
            if (S > R) {
                OT* d = pt + FLay<OT>::off(r, 16 * S + 4 * g, C);  // zero block above the diagonal
                store4(d, f32x4{0.f, 0.f, 0.f, 0.f});
                continue;
            }
            if (deep && S == R) continue;
            f32x4 aA = {0.f, 0.f, 0.f, 0.f}, aP = {0.f, 0.f, 0.f, 0.f};
            const int cS = deep ? S + 1 : S;  // ctab column of the cross-block factor
            const float* cs = cS < R ? sm.ctab[R * (R - 1) / 2 + cS] : nullptr;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                typename FR::t a = FR::kc(sm.u.Kb, PK, 16 * S, ks * KS);
                if (cS < R) a = FR::scale(a, cs + ks * KS + KPL * g);
                MM::mma(aA, a, Ef[ks]);
                MM::mma(aP, a, Qf[ks]);
            }
            f32x4 am, pm;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int s = 16 * S + 4 * g + e;
                am[e] = (S < R || s < r) ? aA[e] : 0.f;
                pm[e] = (S < R || s <= r) ? aP[e] : 0.f;
            }
            *(f32x4*)(sm.Af + r * PAF + 16 * S + 4 * g) = am;
            store4(pt + FLay<OT>::off(r, 16 * S + 4 * g, C), pm);
        }
    }
    lds_barrier();
    solve_unit_lower_64<OT, PAF, PC>(sm.Af, sm.Mf, sm.Tm);

    // stage e . exp(G) and z for the WY products (Kb is dead now), copy T out
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) store_lane<OT>(sm.u.e.Eg + r * PK, ks, g, eg + ks * KPL);
#pragma unroll
    for (int ks = 0; ks < NVS; ++ks) store_lane<OT>(sm.u.e.Z + r * PV, ks, g, zv + ks * KPL);
    {
        OT* tg = (OT*)wy.Tm + cix * C * C;
        constexpr int VEC = 16 / (int)sizeof(OT);
        for (int x = threadIdx.x; x < C * C / VEC; x += kThreads) {  // fragment order
            const int rr = FLay<OT>::unit_row(x, C), ss = FLay<OT>::unit_col(x, C);
            i32x4* d = (i32x4*)(tg + (long)x * VEC);
            if constexpr (STREAM) store_stream(d, *(const i32x4*)(sm.Tm + rr * PC + ss));
            else *d = *(const i32x4*)(sm.Tm + rr * PC + ss);
        }
    }
    lds_barrier();

    // Y^T = Ebar^T T^T (stored negated, row-major -Y[r][i]) and U = T Z (accumulator order)
    const int kend = ((16 * R + 16 + KS - 1) / KS) * KS;
    {
        OT* yt = (OT*)wy.Yh + cix * C * DK;  // fragment order
#pragma unroll
        for (int ib = 0; ib < DK / 16; ++ib) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < kend; k0 += KS)
                MM::mma(acc, FR::tr(sm.u.e.Eg, PK, k0, 16 * ib), FR::kc(sm.Tm, PC, 16 * R, k0));
            OT* d = yt + FLay<OT>::off(r, 16 * ib + 4 * g, DK);
            if constexpr (STREAM) store4_stream(d, f32x4{-acc[0], -acc[1], -acc[2], -acc[3]});
            else store4(d, f32x4{-acc[0], -acc[1], -acc[2], -acc[3]});
        }
    }
    {
        OT* ub = (OT*)wy.U + cix * C * DVl;
#pragma unroll
        for (int jb = 0; jb < DV / 16; ++jb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < kend; k0 += KS)
                MM::mma(acc, FR::kc(sm.Tm, PC, 16 * R, k0), FR::tr(sm.u.e.Z, PV, k0, 16 * jb));
            OT* d = ub + ((long)(R * (DV / 16) + jb) * 64 + l) * 4;
            if constexpr (STREAM) store4_stream(d, acc);
            else store4(d, acc);
        }
    }
}

}  // namespace gdr2
