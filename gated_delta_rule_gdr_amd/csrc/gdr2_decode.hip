// gdr2_decode.hip -- one recurrent Gated Delta Rule-2 token for many independent sequences.
//
// Decoding runs the recurrence one token at a time in constant memory (forum summary "Gated
// DeltaNet-2: Decoupling Erase and Write Gates in Linear Attention for Better Memory Editing",
// section "The Memory Dilemma"; abstract on thelatestinai.com).  Per (sequence, head), with the
// decay applied before the edit (ainews.random.gg article, section "Gated Delta Rule-2: two gates
// instead of one"):
//     Sbar = Diag(alpha) S;  r = Sbar^T (b . k);  S <- Sbar + k (w . v - r)^T;  o = S^T q.
// Value column j of the new state depends only on column j of the old one, through two length-d_k
// reductions r_j = sum_i alpha_i e_i S_ij and p_j = sum_i alpha_i q_i S_ij; then
//     S_ij <- alpha_i S_ij + k_i (z_j - r_j),   o_j = p_j + (q . k)(z_j - r_j).
// The kernel is a pure stream over the fp32 state: every element is read once and written once
// (in place when S_in == S_out), from registers, with 16-byte coalesced accesses.
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

template <typename IT, int DK, int DV, int MODE>
__global__ __launch_bounds__(kThreads) void gdr2_decode_kernel(DecodeParams p) {
    constexpr bool GS = MODE != kModePlain, PRO = MODE == kModePrologue;
    constexpr int CGR = DV / 4;           // 4-column groups
    constexpr int RGR = kThreads / CGR;   // row groups
    constexpr int RPT = DK / RGR;         // rows per thread
    static_assert(RPT * RGR == DK, "mapping");
    __shared__ float red_r[RGR][DV];
    __shared__ float red_p[RGR][DV];
    __shared__ float red_qk[RGR];
    __shared__ float red_n[RGR][2];  // fused prologue: |q|^2, |k|^2 partials

    const long nh = blockIdx.x;
    const int tid = threadIdx.x;
    const int jg = tid % CGR, ig = tid / CGR;
    const int j0 = 4 * jg, ibase = ig * RPT;
    const IT* q = (const IT*)p.q + nh * DK;
    const IT* k = (const IT*)p.k + nh * DK;
    // a scalar gate is one value per (sequence, head): index 0 with a zero channel stride
    // (GS instances only; the channel-wise instance has unit strides known at compile time)
    const int sb = (GS && (p.gates & kEraseScalar)) ? 0 : 1, sa = (GS && (p.gates & kDecayScalar)) ? 0 : 1;
    const int sw = (GS && (p.gates & kWriteScalar)) ? 0 : 1;
    const IT* b = (const IT*)p.b + nh * (sb ? DK : 1);
    const float* la = p.la + nh * (sa ? DK : 1);
    const IT* v = (const IT*)p.v + nh * DV;
    const IT* w = (const IT*)p.w + nh * (sw ? DV : 1);
    const float* Sin = p.S_in ? p.S_in + nh * DK * DV : nullptr;
    float* Sout = p.S_out + nh * DK * DV;

    f32x4 s[RPT];
    if (Sin) {
#pragma unroll
        for (int u = 0; u < RPT; ++u) s[u] = *(const f32x4*)(Sin + (ibase + u) * DV + j0);
    }
    float kk[RPT];
    f32x4 pr = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
    float pqk = 0.f, nq = 0.f, nk = 0.f;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int i = ibase + u;
        // with the fused prologue q, k are raw (their norms scale the sums below afterwards),
        // b and log alpha are pre-activations
        const float lai = PRO ? -p.pro.decay_scale * softplus_f(la[sa * i]) : la[sa * i];
        const float a = __expf(lai);
        const float ki = to_f(k[i]), qi = to_f(q[i]);
        const float bi = PRO ? sigmoid_f(to_f(b[sb * i])) : to_f(b[sb * i]);
        const float e = bi * ki;
        kk[u] = ki;
        pqk += qi * ki;
        nq += qi * qi;
        nk += ki * ki;
        if (!Sin) s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            s[u][j] *= a;  // decay first
            pr[j] += e * s[u][j];
            pp[j] += qi * s[u][j];
        }
    }
    *(f32x4*)&red_r[ig][j0] = pr;
    *(f32x4*)&red_p[ig][j0] = pp;
    if (jg == 0) {
        red_qk[ig] = pqk;
        red_n[ig][0] = nq;
        red_n[ig][1] = nk;
    }
    __syncthreads();
    f32x4 r = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
    float qk = 0.f;
    float tq = 0.f, tk = 0.f;
#pragma unroll
    for (int g = 0; g < RGR; ++g) {
        r += *(const f32x4*)&red_r[g][j0];
        pq += *(const f32x4*)&red_p[g][j0];
        qk += red_qk[g];
        if (PRO) {
            tq += red_n[g][0];
            tk += red_n[g][1];
        }
    }
    if (PRO) {  // q, k were raw: scale every sum by the row norms
        const float rq = rsqrtf(tq + p.pro.norm_eps), rk = rsqrtf(tk + p.pro.norm_eps);
        r *= rk;
        pq *= rq;
        qk *= rq * rk;
#pragma unroll
        for (int u = 0; u < RPT; ++u) kk[u] *= rk;
    }
    f32x4 u4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float wj = PRO ? sigmoid_f(to_f(w[sw * (j0 + j)])) : to_f(w[sw * (j0 + j)]);
        u4[j] = wj * to_f(v[j0 + j]) - r[j];
    }
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        f32x4 x;
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = s[u][j] + kk[u] * u4[j];
        *(f32x4*)(Sout + (ibase + u) * DV + j0) = x;
    }
    if (ig == 0) {
        f32x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = pq[j] + qk * u4[j];
        store4((IT*)p.o + nh * DV + j0, ov);
    }
}

template <typename IT, int DK, int DV>
static hipError_t launch_decode(const DecodeParams& p, hipStream_t s) {
    if (p.prologue)
        hipLaunchKernelGGL((gdr2_decode_kernel<IT, DK, DV, kModePrologue>), dim3(p.N * p.H), dim3(kThreads), 0, s, p);
    else if (p.gates)
        hipLaunchKernelGGL((gdr2_decode_kernel<IT, DK, DV, kModeGates>), dim3(p.N * p.H), dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((gdr2_decode_kernel<IT, DK, DV, kModePlain>), dim3(p.N * p.H), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t decode_dispatch(int bf, int dk, int dv, const DecodeParams& p, hipStream_t s) {
    if (bf) {
        if (dk == 128 && dv == 128) return launch_decode<bf16, 128, 128>(p, s);
        if (dk == 128 && dv == 64) return launch_decode<bf16, 128, 64>(p, s);
        if (dk == 64 && dv == 128) return launch_decode<bf16, 64, 128>(p, s);
        if (dk == 64 && dv == 64) return launch_decode<bf16, 64, 64>(p, s);
    } else {
        if (dk == 128 && dv == 128) return launch_decode<float, 128, 128>(p, s);
        if (dk == 128 && dv == 64) return launch_decode<float, 128, 64>(p, s);
        if (dk == 64 && dv == 128) return launch_decode<float, 64, 128>(p, s);
        if (dk == 64 && dv == 64) return launch_decode<float, 64, 64>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
