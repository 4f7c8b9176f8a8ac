// gdr2_wy.hip -- the chunk-parallel factor kernel of the chunked forward (gfx950): one workgroup
// per (chain, chunk) computes the decay-absorbed WY factors of its chunk (the equations are
// written out at the top of gdr2_fwd.hip and in gdr2_wy.hpp).  It sits in a file of its own so
// that it is compiled with its own scheduling flags (see build.py): scheduled for long clauses of
// memory instructions it runs 3 % faster, while the state carry beside it in gdr2_fwd.hip does
// not gain from that schedule.
#include "gdr2_common.hpp"
#include "gdr2_kernels.hpp"
#include "gdr2_wy.hpp"

namespace gdr2 {

template <typename OT, int DK, int DV, int MODE, bool STREAM>
__global__ __launch_bounds__(kThreads, 2) void gdr2_wy_kernel(FwdParams p) {
    __shared__ WySmem<OT, DK, DV> sm;
    WyChunk<OT, DK, DV> ch(p.B, p.H, p.T, p.DV, p.NC, p.c0, p.ncr, gate_bits<MODE>(p.gates), p.pro, blockIdx.x, p.q,
                           p.k, p.b, p.la, p.v, p.w);
    wy_factors<OT, DK, DV, MODE, STREAM>(sm, ch, p.wy);
}

template <typename OT, int DK, int DV, bool STREAM>
static void launch_wy_mode(const FwdParams& p, long nblk, hipStream_t s) {
    auto go = [&](auto mode) {
        hipLaunchKernelGGL((gdr2_wy_kernel<OT, DK, DV, decltype(mode)::value, STREAM>), dim3(nblk), dim3(kThreads), 0, s, p);
    };
    with_mode<sizeof(OT) == 2>(p.prologue, p.gates, go);  // the fp32 path reads the gate bits
}
template <typename OT, int DK, int DV>
static hipError_t launch_wy(const FwdParams& p, hipStream_t s) {
    const long nblk = (long)p.B * p.H * p.ncr;
    if (nblk == 0) return hipSuccess;
    // streaming instances for the 16-bit path only (the fp32 path is the precision path)
    if (sizeof(OT) == 2 && p.stream) launch_wy_mode<OT, DK, DV, sizeof(OT) == 2>(p, nblk, s);
    else launch_wy_mode<OT, DK, DV, false>(p, nblk, s);
    return hipGetLastError();
}

hipError_t wy_dispatch(int bf, int dk, int dv, const FwdParams& p, hipStream_t s) {
    if (bf) {
        if (dk == 128 && dv == 128) return launch_wy<bf16, 128, 128>(p, s);
        if (dk == 128 && dv == 64) return launch_wy<bf16, 128, 64>(p, s);
        if (dk == 64 && dv == 128) return launch_wy<bf16, 64, 128>(p, s);
        if (dk == 64 && dv == 64) return launch_wy<bf16, 64, 64>(p, s);
    } else {
        if (dk == 128 && dv == 128) return launch_wy<float, 128, 128>(p, s);
        if (dk == 128 && dv == 64) return launch_wy<float, 128, 64>(p, s);
        if (dk == 64 && dv == 128) return launch_wy<float, 64, 128>(p, s);
        if (dk == 64 && dv == 64) return launch_wy<float, 64, 64>(p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace gdr2
