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
// Sixteen lanes per row (a lane holds d_v / 16 consecutive channels, one 16-byte load for bf16 at
// d_v = 128), four rows per wave step and two steps' rows loaded together; the row sums are
// 16-lane DPP reductions.  Both passes are pure streams.  The weight gradient is reduced without
// atomics: every workgroup writes its partial sums (its waves combined in LDS), and a second
// small kernel adds the partials in a fixed order, so the result is bitwise deterministic.
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"

namespace gdr2 {

constexpr int kEpiRowsPerWave = 32;  // rows a wave handles: 4 steps of 8 rows (2 per lane group)

// sum over the 16 lanes of the caller's DPP row, in every lane of the row
__device__ __forceinline__ float row_sum16(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xf, 0xf, false));  // row_half_mirror
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xf, 0xf, false));  // row_mirror
    return x;
}

// N consecutive elements of a row to fp32 and back (one or two vector accesses)
template <typename OT, int N>
__device__ __forceinline__ void load_n(const OT* p, float* v) {
    if constexpr (sizeof(OT) == 2 && N == 8) {
        const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
        for (int c = 0; c < 8; ++c) v[c] = (float)x[c];
    } else if constexpr (sizeof(OT) == 2 && N == 4) {
        const bf16x4 x = *(const bf16x4*)p;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = (float)x[c];
    } else {
#pragma unroll
        for (int c = 0; c < N; c += 4) {
            const f32x4 x = *(const f32x4*)((const float*)p + c);
            v[c] = x[0]; v[c + 1] = x[1]; v[c + 2] = x[2]; v[c + 3] = x[3];
        }
    }
}
template <typename OT, int N>
__device__ __forceinline__ void store_n(OT* p, const float* v) {
    if constexpr (sizeof(OT) == 2 && N == 8) {
        bf16x8 x;
#pragma unroll
        for (int c = 0; c < 8; ++c) x[c] = (bf16)v[c];
        *(bf16x8*)p = x;
    } else if constexpr (sizeof(OT) == 2 && N == 4) {
        *(bf16x4*)p = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
    } else {
#pragma unroll
        for (int c = 0; c < N; c += 4) *(f32x4*)((float*)p + c) = f32x4{v[c], v[c + 1], v[c + 2], v[c + 3]};
    }
}

template <typename OT, int DV>
__global__ __launch_bounds__(kThreads) void gdr2_epi_fwd_kernel(EpiParams p) {
    constexpr int CPL = DV / 16;  // channels per lane
    const int l = lane_id(), g = l >> 4, ch = (l & 15) * CPL;
    const long wave = (long)blockIdx.x * kWaves + wave_id();
    const OT* __restrict__ o = (const OT*)p.o;
    const OT* __restrict__ gt = (const OT*)p.g;
    OT* __restrict__ y = (OT*)p.y;
    float wt[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) wt[c] = p.weight[ch + c];
#pragma unroll
    for (int it = 0; it < kEpiRowsPerWave / 8; ++it) {
        const long r0 = wave * kEpiRowsPerWave + it * 8 + g;  // rows r0 and r0 + 4 of this lane group
        // loads from a row clamped into range (no branch, so all of them are in flight together);
        // rows past the end are not stored
        float ov[2][CPL], gv[2][CPL];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const long rl = r0 + 4 * u < p.rows ? r0 + 4 * u : p.rows - 1;
            load_n<OT, CPL>(o + rl * DV + ch, ov[u]);
            load_n<OT, CPL>(gt + rl * DV + ch, gv[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const long row = r0 + 4 * u;
            if (row < p.rows) {
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) ss += ov[u][c] * ov[u][c];
                const float rs = rsqrtf(row_sum16(ss) / DV + p.eps);
                float yv[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) yv[c] = ov[u][c] * rs * wt[c] * gv[u][c] * sigmoid_f(gv[u][c]);
                store_n<OT, CPL>(y + row * DV + ch, yv);
            }
        }
    }
}

template <typename OT, int DV>
__global__ __launch_bounds__(kThreads) void gdr2_epi_bwd_kernel(EpiParams p) {
    constexpr int CPL = DV / 16;
    const int l = lane_id(), g = l >> 4, ch = (l & 15) * CPL;
    const long wave = (long)blockIdx.x * kWaves + wave_id();
    const OT* __restrict__ o = (const OT*)p.o;
    const OT* __restrict__ gt = (const OT*)p.g;
    const OT* __restrict__ dy = (const OT*)p.dy;
    OT* __restrict__ dox = (OT*)p.dox;
    OT* __restrict__ dg = (OT*)p.dg;
    __shared__ float part[kWaves][DV];
    float wt[CPL], dwp[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        wt[c] = p.weight[ch + c];
        dwp[c] = 0.f;
    }
#pragma unroll
    for (int it = 0; it < kEpiRowsPerWave / 8; ++it) {
        const long r0 = wave * kEpiRowsPerWave + it * 8 + g;
        float ov[2][CPL], gv[2][CPL], dv_[2][CPL];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const long rl = r0 + 4 * u < p.rows ? r0 + 4 * u : p.rows - 1;
            load_n<OT, CPL>(o + rl * DV + ch, ov[u]);
            load_n<OT, CPL>(gt + rl * DV + ch, gv[u]);
            load_n<OT, CPL>(dy + rl * DV + ch, dv_[u]);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const long row = r0 + 4 * u;
            if (row < p.rows) {
                float ss = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) ss += ov[u][c] * ov[u][c];
                const float rs = rsqrtf(row_sum16(ss) / DV + p.eps);
                float a[CPL], dgv[CPL], ao = 0.f;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const float s = sigmoid_f(gv[u][c]);
                    const float sl = gv[u][c] * s;
                    a[c] = dv_[u][c] * wt[c] * sl;
                    ao += a[c] * ov[u][c];
                    const float n = ov[u][c] * rs;
                    dwp[c] += dv_[u][c] * n * sl;
                    dgv[c] = dv_[u][c] * n * wt[c] * s * (1.f + gv[u][c] * (1.f - s));
                }
                store_n<OT, CPL>(dg + row * DV + ch, dgv);
                ao = row_sum16(ao) / DV;
                float dov[CPL];
#pragma unroll
                for (int c = 0; c < CPL; ++c) dov[c] = rs * (a[c] - ov[u][c] * rs * rs * ao);
                store_n<OT, CPL>(dox + row * DV + ch, dov);
            }
        }
    }
    // this workgroup's weight-gradient partial: the four lane groups of a wave, then its waves,
    // added in a fixed order
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
        dwp[c] += __shfl_xor(dwp[c], 16);
        dwp[c] += __shfl_xor(dwp[c], 32);
    }
    if (g == 0) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) part[wave_id()][ch + c] = dwp[c];
    }
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
