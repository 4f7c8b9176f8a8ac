// gdr2_epilogue.hip -- the block's output epilogue after the GDR-2 mixer (gfx950).
//
// The ainews.random.gg article on Gated DeltaNet-2, section "Block design and hybrid model":
// the recurrent output is RMS-normalised and multiplied by a SiLU output gate before the output
// projection.  Per row (one token of one head, d_v channels), with a per-channel weight shared by
// all heads:
//     rs  = 1 / sqrt(mean_j o_j^2 + eps)
//     y_j = o_j * rs * weight_j * silu(g_j),          silu(x) = x * sigmoid(x)
// and its vector-Jacobian product for the cotangent dy:
//     a_j = dy_j * weight_j * silu(g_j)
//     do_j = rs * (a_j - o_j * rs^2 * mean_i(a_i o_i))
//     dg_j = dy_j * o_j * rs * weight_j * silu'(g_j),  silu'(x) = s (1 + x (1 - s)), s = sigmoid(x)
//     dweight_j = sum over rows of dy_j * o_j * rs * silu(g_j)
//
// One wave per row at a time, each lane holding d_v / 64 consecutive channels; the row sums are
// wave reductions.  Both passes are pure streams.  The weight gradient is reduced without
// atomics: every workgroup writes its partial sums (its waves combined in LDS), and a second
// small kernel adds the partials in a fixed order, so the result is bitwise deterministic.
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

constexpr int kEpiRowsPerWave = 16;  // rows a wave handles

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    return x;
}

template <typename OT, int DV>
__global__ __launch_bounds__(kThreads) void gdr2_epi_fwd_kernel(EpiParams p) {
    constexpr int CPL = DV / 64;  // channels per lane
    const int l = lane_id();
    const long wave = (long)blockIdx.x * kWaves + wave_id();
    const OT* o = (const OT*)p.o;
    const OT* gt = (const OT*)p.g;
    OT* y = (OT*)p.y;
    float wt[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) wt[c] = p.weight[l * CPL + c];
    for (int i = 0; i < kEpiRowsPerWave; ++i) {
        const long row = wave * kEpiRowsPerWave + i;
        if (row >= p.rows) break;
        const long base = row * DV + l * CPL;
        float ov[CPL], gv[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            ov[c] = to_f(o[base + c]);
            gv[c] = to_f(gt[base + c]);
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) ss += ov[c] * ov[c];
        ss = wave_sum(ss);
        const float rs = rsqrtf(ss / DV + p.eps);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float s = sigmoid_f(gv[c]);
            y[base + c] = from_f<OT>(ov[c] * rs * wt[c] * gv[c] * s);
        }
    }
}

template <typename OT, int DV>
__global__ __launch_bounds__(kThreads) void gdr2_epi_bwd_kernel(EpiParams p) {
    constexpr int CPL = DV / 64;
    const int l = lane_id();
    const long wave = (long)blockIdx.x * kWaves + wave_id();
    const OT* o = (const OT*)p.o;
    const OT* gt = (const OT*)p.g;
    const OT* dy = (const OT*)p.dy;
    OT* dox = (OT*)p.dox;
    OT* dg = (OT*)p.dg;
    __shared__ float part[kWaves][DV];
    float wt[CPL], dwp[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        wt[c] = p.weight[l * CPL + c];
        dwp[c] = 0.f;
    }
    for (int i = 0; i < kEpiRowsPerWave; ++i) {
        const long row = wave * kEpiRowsPerWave + i;
        if (row >= p.rows) break;
        const long base = row * DV + l * CPL;
        float ov[CPL], gv[CPL], dv_[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            ov[c] = to_f(o[base + c]);
            gv[c] = to_f(gt[base + c]);
            dv_[c] = to_f(dy[base + c]);
        }
        float ss = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) ss += ov[c] * ov[c];
        ss = wave_sum(ss);
        const float rs = rsqrtf(ss / DV + p.eps);
        float a[CPL], ao = 0.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const float s = sigmoid_f(gv[c]);
            const float sl = gv[c] * s;
            a[c] = dv_[c] * wt[c] * sl;
            ao += a[c] * ov[c];
            const float n = ov[c] * rs;
            dwp[c] += dv_[c] * n * sl;
            dg[base + c] = from_f<OT>(dv_[c] * n * wt[c] * s * (1.f + gv[c] * (1.f - s)));
        }
        ao = wave_sum(ao) / DV;
#pragma unroll
        for (int c = 0; c < CPL; ++c) dox[base + c] = from_f<OT>(rs * (a[c] - ov[c] * rs * rs * ao));
    }
    // this workgroup's weight-gradient partial: [workgroup][DV], its waves added in order
#pragma unroll
    for (int c = 0; c < CPL; ++c) part[wave_id()][l * CPL + c] = dwp[c];
    __syncthreads();
    for (int j = threadIdx.x; j < DV; j += kThreads) {
        float acc = 0.f;
#pragma unroll
        for (int wv = 0; wv < kWaves; ++wv) acc += part[wv][j];
        p.dw_part[(long)blockIdx.x * DV + j] = acc;
    }
}

// dweight_j = sum of the workgroup partials: one workgroup per channel j, each thread a strided
// subset, then a fixed-order tree in LDS
template <int DV>
__global__ __launch_bounds__(kThreads) void gdr2_epi_dw_reduce_kernel(EpiParams p, long nparts) {
    __shared__ float red[kThreads];
    const int j = blockIdx.x, t = threadIdx.x;
    float acc = 0.f;
    for (long x = t; x < nparts; x += kThreads) acc += p.dw_part[x * DV + j];
    red[t] = acc;
    __syncthreads();
    for (int m = kThreads / 2; m >= 1; m >>= 1) {
        if (t < m) red[t] += red[t + m];
        __syncthreads();
    }
    if (t == 0) p.dweight[j] = red[0];
}

// workgroups of the epilogue kernels for `rows` rows (= weight-gradient partials of the backward)
long epi_blocks(long rows) {
    const long waves = (rows + kEpiRowsPerWave - 1) / kEpiRowsPerWave;
    return (waves + kWaves - 1) / kWaves;
}

template <typename OT, int DV>
static hipError_t launch_epi(const EpiParams& p, bool bwd, hipStream_t s) {
    const long nblk = epi_blocks(p.rows);
    if (!bwd && nblk == 0) return hipSuccess;
    if (!bwd) {
        hipLaunchKernelGGL((gdr2_epi_fwd_kernel<OT, DV>), dim3(nblk), dim3(kThreads), 0, s, p);
        return hipGetLastError();
    }
    if (nblk > 0) {
        hipLaunchKernelGGL((gdr2_epi_bwd_kernel<OT, DV>), dim3(nblk), dim3(kThreads), 0, s, p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gdr2_epi_dw_reduce_kernel<DV>), dim3(DV), dim3(kThreads), 0, s, p, nblk);
    return hipGetLastError();
}

hipError_t epi_dispatch(int bf, int dv, bool bwd, const EpiParams& p, hipStream_t s) {
    if (bf) {
        if (dv == 128) return launch_epi<bf16, 128>(p, bwd, s);
        if (dv == 64) return launch_epi<bf16, 64>(p, bwd, s);
    } else {
        if (dv == 128) return launch_epi<float, 128>(p, bwd, s);
        if (dv == 64) return launch_epi<float, 64>(p, bwd, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
