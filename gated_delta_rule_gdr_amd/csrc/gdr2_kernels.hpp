// gdr2_kernels.hpp -- host-side launch interface between the C ABI and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>

namespace gdr2 {

struct FwdParams {
    int B, H, NS, NC;   // batch, heads, value slices per chain, chunks
    long T, DV;         // tokens, value width (DK is a template parameter)
    const void *q, *k, *v, *b, *w;  // input dtype
    const float* la;    // log decay, fp32
    const float* S0;    // [B,H,DK,DV] fp32 or null
    void* o;            // [B,T,H,DV] input dtype
    float* ST;          // [B,H,DK,DV] fp32 or null
    void* states;       // [B*H][NC][DV][DK] input dtype or null (chunk-entry states, transposed)
};

struct DecodeParams {
    long N, H;
    const void *q, *k, *v, *b, *w;
    const float* la;
    const float* S_in;  // may equal S_out; null = zero state
    float* S_out;
    void* o;
};

struct BwdParams {
    int B, H, NS, NC;
    long T, DV;
    const void *q, *k, *v, *b, *w;
    const float* la;
    const void* states;   // chunk-entry states [B*H][NC][DV][DK] (input dtype)
    const void* dO;       // [B,T,H,DV]
    const float* dST;     // [B,H,DK,DV] fp32 or null
    void* dSx;            // per-chunk exit-state gradients [B*H][NC][DV][DK] (input dtype)
    float* dS0;           // [B,H,DK,DV] fp32 or null
    void *dq, *dk, *dv, *db, *dw;
    float* dla;
};

int fwd_slice_width(int dtype_bf16, int dk, int dv, long chains);
hipError_t fwd_dispatch(int dtype_bf16, int dk, int dvs, const FwdParams& p, hipStream_t s);
hipError_t decode_dispatch(int dtype_bf16, int dk, int dv, const DecodeParams& p, hipStream_t s);
int bwd_slice_width(int dtype_bf16, int dk, int dv, long chains);
hipError_t bwd_dispatch(int dtype_bf16, int dk, int dvs, const BwdParams& p, hipStream_t s);

}  // namespace gdr2
