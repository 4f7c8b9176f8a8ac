// gdr2_kernels.hpp -- host-side launch interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <type_traits>

namespace gdr2 {

// Gate shapes (bit mask, same values as gdr2_gates in gdr2.h): a set bit means that gate is one
// value per (batch, token, head) instead of one per channel.
constexpr int kEraseScalar = 1;   // b
constexpr int kWriteScalar = 2;   // w
constexpr int kDecayScalar = 4;   // log alpha

// Kernel instances: plain (every gate channel-wise, post-activation inputs), scalar gates with the
// gate bits read at run time (kModeGates), fused prologue (pre-activation inputs, gate bits at run
// time), and, for the 16-bit path of the factor and chunk-gradient kernels, whose run-time gate
// branches cost them about a fifth of their time: scalar gates with the bits fixed at compile
// time (kModeFixedGates + bits) and the fused prologue with every gate channel-wise
// (kModePrologueChannel).
constexpr int kModePlain = 0, kModeGates = 1, kModePrologue = 2, kModePrologueChannel = 3;
constexpr int kModeFixedGates = 8;

__host__ __device__ constexpr bool mode_prologue(int mode) {
    return mode == kModePrologue || mode == kModePrologueChannel;
}
// The gate bits an instance works with: none for the plain and channel-wise prologue instances,
// its own for a fixed-gates instance, the run-time ones otherwise.
template <int MODE>
__host__ __device__ constexpr int gate_bits(int run_time) {
    return MODE == kModePlain || MODE == kModePrologueChannel ? 0
           : MODE >= kModeFixedGates                          ? MODE - kModeFixedGates
                                                              : run_time;
}

// Calls f(std::integral_constant<int, MODE>{}) with the instance MODE that serves a call with the
// given fused-prologue flag and gate bits (validated: bits 0..2 only): with FIXED (the 16-bit
// path) the gate bits of a scalar-gate call and of a channel-wise prologue call are template
// constants; without, they are read at run time.
template <bool FIXED, typename F>
inline void with_mode(int prologue, int gates, F&& f) {
    if constexpr (FIXED) {
        switch (prologue ? (gates == 0 ? 8 : -1) : gates) {
        case 1: f(std::integral_constant<int, kModeFixedGates + 1>{}); return;
        case 2: f(std::integral_constant<int, kModeFixedGates + 2>{}); return;
        case 3: f(std::integral_constant<int, kModeFixedGates + 3>{}); return;
        case 4: f(std::integral_constant<int, kModeFixedGates + 4>{}); return;
        case 5: f(std::integral_constant<int, kModeFixedGates + 5>{}); return;
        case 6: f(std::integral_constant<int, kModeFixedGates + 6>{}); return;
        case 7: f(std::integral_constant<int, kModeFixedGates + 7>{}); return;
        case 8: f(std::integral_constant<int, kModePrologueChannel>{}); return;
        default: break;  // no gates without the prologue, or the prologue with scalar gates
        }
    }
    if (prologue) f(std::integral_constant<int, kModePrologue>{});
    else if (!FIXED && gates) f(std::integral_constant<int, FIXED ? kModePlain : kModeGates>{});
    else f(std::integral_constant<int, kModePlain>{});
}

// Fused prologue parameters: q, k scaled by (sum of squares + norm_eps)^-1/2, b = sigmoid(b),
// w = sigmoid(w), log alpha = -decay_scale * softplus(a).
struct Prologue {
    float decay_scale, norm_eps;
};

// Per-chunk WY factors written by the chunk-parallel factor kernel and read by the state-carry
// kernels (forward and backward) and the chunk-gradient kernel.  Element type = input dtype
// except gam.  Every array is indexed [chain = b*H + h][chunk][...]; the [C][*] tiles are in
// fragment order (FLay in gdr2_common.hpp).
struct WyBufs {
    void* Yh;    // -Y = -(T Ebar),                          [C][DK]
    void* Qg;    // Qbar = Q . exp(G),                        [C][DK]
    void* Kt;    // Ktilde = K . exp(G_C - G),                [C][DK]
    void* P;     // P = lower(Qbar Kbar^T),                   [C][C]
    void* Tm;    // T = (I + A)^-1,                           [C][C]
    void* U;     // U = T Z in MFMA accumulator order,        [4][DV/16][64 lanes][4]
    float* gam;  // gamma = exp(G_C),                         [DK] fp32
};

struct FwdParams {
    int B, H, NS, NC;   // batch, heads, value slices per chain, chunks
    int c0, ncr;        // chunks this launch covers: [c0, c0 + ncr) (the factor kernel, the 16-bit
                        // carry); the fp32 carry always covers all NC
    int gates;          // gate shapes (kEraseScalar | kWriteScalar | kDecayScalar)
    int prologue;       // inputs are pre-activations (see Prologue)
    Prologue pro;
    long T, DV;         // tokens, value width (DK is a template parameter)
    const void *q, *k, *v, *b, *w;  // input dtype
    const float* la;    // log decay, fp32
    const float* S0;    // [B,H,DK,DV] fp32 or null
    void* o;            // [B,T,H,DV] input dtype or null
    float* ST;          // [B,H,DK,DV] fp32 or null
    void* states;       // [B*H][NC][DV][DK] input dtype (chunk-entry states, transposed)
    WyBufs wy;
    int stream;         // write the factor tiles past the L2 (see kStreamFactorBytes)
};

// Factor tiles are streamed past the caches (nontemporal stores) when they take at least this
// many bytes: then they do not fit the 256 MB memory-side cache and the carry reads them from HBM
// anyway, and streaming spares the next kernel the write-back of their dirty L2 lines (carry 135
// -> 121 us at B=4 T=4096 H=16 d=128, 335 MB of factors).  Smaller sets stay cached for the carry
// (at B=2 T=2048, 84 MB, the carry takes 42 us with cached factors and 58 us with streamed ones).
constexpr size_t kStreamFactorBytes = (size_t)256 << 20;

struct DecodeParams {
    long N, H;
    int gates, prologue;
    Prologue pro;
    const void *q, *k, *v, *b, *w;
    const float* la;
    const float* S_in;  // may equal S_out; null = zero state
    float* S_out;
    void* o;
};

struct BwdParams {
    int B, H, NS, NC;
    int c0, ncr;          // chunks this launch covers: [c0, c0 + ncr) (the 16-bit state-gradient
                          // carry, the chunk-gradient kernel); the fp32 carry always covers all NC
    int gates, prologue;
    Prologue pro;
    long T, DV;
    const void *q, *k, *v, *b, *w;
    const float* la;
    const void* states;   // chunk-entry states [B*H][NC][DV][DK] (input dtype)
    WyBufs wy;            // factors of the forward
    const void* dO;       // [B,T,H,DV]
    const float* dST;     // [B,H,DK,DV] fp32 or null
    void* dSx;            // per-chunk exit-state gradients [B*H][NC][DV][DK] (input dtype)
    float* dS0;           // [B,H,DK,DV] fp32 or null
    void *dq, *dk, *dv, *db, *dw;
    float* dla;
};

// Output epilogue: y = RMSNorm(o) * weight * silu(g) per row of DV channels, and its backward.
struct EpiParams {
    long rows;              // B * T * H
    float eps;
    const void *o, *g;      // [rows][DV] input dtype
    const float* weight;    // [DV] fp32
    void* y;                // forward output [rows][DV]
    const void* dy;         // backward: cotangent of y
    void *dox, *dg;         // backward outputs [rows][DV]
    float* dweight;         // backward output [DV] fp32
    float* dw_part;         // backward workspace [epi_blocks(rows)][DV] fp32
};

// No-allocation forward-only entry point: bytes of its static device scratch, and the scratch's
// device address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
hipError_t noalloc_scratch(void** ptr);

// forward: factor kernel (chunk-parallel) + state carry (sequential over chunks)
hipError_t wy_dispatch(int dtype_bf16, int dk, int dv, const FwdParams& p, hipStream_t s);
int carry_slice_width(int dtype_bf16, int dk, int dv, long chains);
hipError_t carry_fwd_dispatch(int dtype_bf16, int dk, int dvs, const FwdParams& p, hipStream_t s);
hipError_t decode_dispatch(int dtype_bf16, int dk, int dv, const DecodeParams& p, hipStream_t s);
hipError_t dstate_dispatch(int dtype_bf16, int dk, int dvs, const BwdParams& p, hipStream_t s);
hipError_t bgrad_dispatch(int dtype_bf16, int dk, int dv, const BwdParams& p, hipStream_t s);
long epi_blocks(long rows);
hipError_t epi_dispatch(int dtype_bf16, int dv, bool bwd, const EpiParams& p, hipStream_t s);

}  // namespace gdr2
