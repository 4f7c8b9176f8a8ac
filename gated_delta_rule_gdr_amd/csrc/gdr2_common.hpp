// gdr2_common.hpp -- device building blocks shared by the GDR-2 kernels (gfx950 only).
//
// Matrix-core tiles: every contraction uses the 16x16 MFMA family with fp32 accumulation,
//   bf16 operands: v_mfma_f32_16x16x32_bf16 (K step 32, 8 operand values per lane),
//   fp32 operands: v_mfma_f32_16x16x4_f32  (K step 4, 1 operand value per lane).
// Lane layout (wave64, l = lane):
//   A operand  : row  l%16, k = kbase + KPL*(l/16) + j   (j < KPL)
//   B operand  : col  l%16, k = kbase + KPL*(l/16) + j
//   accumulator: col  l%16, rows 4*(l/16) + i            (i < 4)
// Every operand tile in LDS is therefore stored "k-contiguous": A as [m][k], B as [n][k], with a
// 16-byte row pad so that the 16 rows a fragment load touches fall in different banks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr2 {

constexpr int kChunk = 64;  // tokens per chunk
constexpr int kThreads = 256;
constexpr int kWaves = 4;

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));  // 16 raw bytes

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
__device__ __forceinline__ int wave_id() { return threadIdx.x >> 6; }

// ------------------------------------------------------------------ element conversions
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }  // RNE

// Four consecutive elements from global memory, widened to fp32 (8-byte or 16-byte load).
__device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }
__device__ __forceinline__ f32x4 load4(const bf16* p) {
    bf16x4 v = *(const bf16x4*)p;
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
}
__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
// Four raw elements kept undecoded in registers (a prefetch must not be widened before use).
template <typename OT> struct Raw4;
template <> struct Raw4<float> {
    typedef f32x4 t;
    static __device__ __forceinline__ f32x4 widen(const t& x) { return x; }
    static __device__ __forceinline__ t narrow(const f32x4& x) { return x; }
};
template <> struct Raw4<bf16> {
    typedef bf16x4 t;
    static __device__ __forceinline__ f32x4 widen(const t& x) {
        return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    }
    static __device__ __forceinline__ t narrow(const f32x4& x) {
        return t{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    }
};
__device__ __forceinline__ void store4(bf16* p, f32x4 v) {
    *(bf16x4*)p = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Streaming (nontemporal) stores for outputs that a later kernel reads back, written by whole
// cache lines per wave instruction: they go past the L2 instead of sitting in it as dirty lines
// that the next kernel then has to write back while it runs.  (Partial-line pieces are not
// streamed: written past the L2 they become many small memory writes.)
template <typename T>
__device__ __forceinline__ void store_stream(T* p, const T& v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void store4_stream(bf16* p, f32x4 v) {
    store_stream((bf16x4*)p, bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]});
}
__device__ __forceinline__ void store4_stream(float* p, f32x4 v) { store_stream((f32x4*)p, v); }

// ------------------------------------------------------------------ MFMA wrappers
template <typename OT> struct Mfma;

template <> struct Mfma<bf16> {
    static constexpr int KS = 32;   // K per instruction
    static constexpr int KPL = 8;   // K values per lane
    typedef bf16x8 frag;
    // fragment of a k-contiguous tile: row (m0 + l%16), k = k0 + 8*(l/16) .. +7
    static __device__ __forceinline__ frag load(const bf16* t, int pitch, int m0, int k0) {
        int l = lane_id();
        return *(const bf16x8*)(t + (m0 + (l & 15)) * pitch + k0 + 8 * (l >> 4));
    }
    // same, each value multiplied by s[k] (fp32) before rounding back to bf16
    static __device__ __forceinline__ frag load_scaled(const bf16* t, int pitch, int m0, int k0,
                                                        const float* s) {
        int l = lane_id();
        int kk = k0 + 8 * (l >> 4);
        bf16x8 v = *(const bf16x8*)(t + (m0 + (l & 15)) * pitch + kk);
        f32x4 s0 = *(const f32x4*)(s + kk), s1 = *(const f32x4*)(s + kk + 4);
        bf16x8 r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[j] = (bf16)((float)v[j] * s0[j]);
            r[j + 4] = (bf16)((float)v[j + 4] * s1[j]);
        }
        return r;
    }
    static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Mfma<float> {
    static constexpr int KS = 4;
    static constexpr int KPL = 1;
    typedef float frag;
    static __device__ __forceinline__ frag load(const float* t, int pitch, int m0, int k0) {
        int l = lane_id();
        return t[(m0 + (l & 15)) * pitch + k0 + (l >> 4)];
    }
    static __device__ __forceinline__ frag load_scaled(const float* t, int pitch, int m0, int k0,
                                                        const float* s) {
        int l = lane_id();
        int kk = k0 + (l >> 4);
        return t[(m0 + (l & 15)) * pitch + kk] * s[kk];
    }
    static __device__ __forceinline__ void mma(f32x4& c, const frag& a, const frag& b) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};

// fp32 16x16x4 fragment loads from a row-major fp32 tile, used by the triangular solve:
//   A operand from X[m][k] (pitch p), B operand from Y[k][n] (pitch p).
__device__ __forceinline__ float fa32(const float* X, int p, int m0, int k0) {
    int l = lane_id();
    return X[(m0 + (l & 15)) * p + k0 + (l >> 4)];
}
__device__ __forceinline__ float fb32(const float* Y, int p, int k0, int n0) {
    int l = lane_id();
    return Y[(k0 + (l >> 4)) * p + n0 + (l & 15)];
}
__device__ __forceinline__ void mma32(f32x4& c, float a, float b) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Accumulator element (i) of the calling lane: row and column inside its 16x16 block.  The
// helpers here also come with an explicit lane argument `l`, for kernels that keep the lane index
// in a value of their own.
__device__ __forceinline__ int acc_row(int i, int l) { return 4 * (l >> 4) + i; }
__device__ __forceinline__ int acc_col(int l) { return l & 15; }
__device__ __forceinline__ int acc_row(int i) { return acc_row(i, lane_id()); }
__device__ __forceinline__ int acc_col() { return acc_col(lane_id()); }

// Write a 16x16 accumulator block transposed into a k-contiguous tile: dst[n][m] (n = column of
// the block, m = row); the four rows of a lane are contiguous in dst, one 8/16-byte store.
template <typename OT>
__device__ __forceinline__ void store_acc_T(OT* dst, int pitch, int n0, int m0, const f32x4& c, int l) {
    OT* p = dst + (n0 + (l & 15)) * pitch + m0 + 4 * (l >> 4);
    if constexpr (sizeof(OT) == 2) {
        *(bf16x4*)p = bf16x4{(bf16)c[0], (bf16)c[1], (bf16)c[2], (bf16)c[3]};
    } else {
        *(f32x4*)p = c;
    }
}
template <typename OT>
__device__ __forceinline__ void store_acc_T(OT* dst, int pitch, int n0, int m0, const f32x4& c) {
    store_acc_T(dst, pitch, n0, m0, c, lane_id());
}

// x of lane (l ^ m) through ds_bpermute, with the caller's lane index
__device__ __forceinline__ float shfl_xor_l(float x, int m, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((l ^ m) << 2, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Map a linear workgroup index so that the `group` consecutive work items that share key-side
// data land on the same XCD (workgroups are dispatched round-robin over the 8 XCDs; each XCD
// has its own L2).  Identity when the grid does not split evenly.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
    if (nblocks % 8 != 0) return bid;
    int per = nblocks / 8;
    return (bid % 8) * per + bid / 8;
}

}  // namespace gdr2

namespace gdr2 {
// Workgroup barrier that waits only for this wave's LDS traffic (lgkmcnt(0)) and leaves global
// loads in flight, so that next-chunk prefetches survive it.  The empty asm with a memory clobber
// keeps the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    // workgroup fences limited to LDS: they order the LDS accesses around the barrier and wait
    // for LDS only (lgkmcnt), so global loads stay in flight across it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
}  // namespace gdr2

namespace gdr2 {
// ------------------------------------------------------------------ operand fragments
// Two kinds of LDS tiles feed MFMA operands (for A and B alike: index = l%16, k = KPL*(l/16)+j):
//   kc: "k-contiguous" tile X[idx][k]  -> one 16-byte read per lane (bf16) / one scalar (fp32)
//   tr: "k-major"      tile X[k][idx]  -> two ds_read_b64_tr_b16 per lane (bf16) / one scalar.
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane p of a group supplies the address of four
// 16-bit elements M[p][0..3]; lane i of the group receives M[4j + i/4][i%4] for j = 0..3.  With
// lane p pointing at X[kb + p/4][c0 + 4*(p%4)], lane i receives X[kb .. kb+3][c0 + i].
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x4 ds_read_tr4(const bf16* p) {
    s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
    return __builtin_bit_cast(bf16x4, v);
}

template <typename OT> struct Frag;
template <> struct Frag<bf16> {
    typedef bf16x8 t;
    static constexpr int N = 8;
    static __device__ __forceinline__ float at(const t& x, int e) { return (float)x[e]; }
    static __device__ __forceinline__ t kc(const bf16* X, int pitch, int i0, int k0, int l) {
        return *(const bf16x8*)(X + (i0 + (l & 15)) * pitch + k0 + 8 * (l >> 4));
    }
    static __device__ __forceinline__ t tr(const bf16* X, int pitch, int k0, int i0, int l) {
        const int p = l & 15, kb = k0 + 8 * (l >> 4) + (p >> 2);
        const bf16* a = X + kb * pitch + i0 + 4 * (p & 3);
        bf16x4 lo = ds_read_tr4(a), hi = ds_read_tr4(a + 4 * pitch);
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    static __device__ __forceinline__ t kc(const bf16* X, int pitch, int i0, int k0) { return kc(X, pitch, i0, k0, lane_id()); }
    static __device__ __forceinline__ t tr(const bf16* X, int pitch, int k0, int i0) { return tr(X, pitch, k0, i0, lane_id()); }
    // fragment straight from global memory, row-major [idx][k] with the given pitch
    static __device__ __forceinline__ t gkc(const bf16* X, long pitch, int i0, int k0) {
        const int l = lane_id();
        return *(const bf16x8*)(X + (long)(i0 + (l & 15)) * pitch + k0 + 8 * (l >> 4));
    }
    // fragment from 8 fp32 values, multiplied by 8 fp32 scales
    static __device__ __forceinline__ t from_f32(const float* v) {
        return bf16x8{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3],
                      (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
    }
    static __device__ __forceinline__ t scale(const t& x, const float* s) {
        t r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (bf16)((float)x[j] * s[j]);
        return r;
    }
    static __device__ __forceinline__ t scale(const t& x, float s) {
        t r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (bf16)((float)x[j] * s);
        return r;
    }
};
template <> struct Frag<float> {
    typedef float t;
    static constexpr int N = 1;
    static __device__ __forceinline__ float at(const t& x, int) { return x; }
    static __device__ __forceinline__ t kc(const float* X, int pitch, int i0, int k0, int l) {
        return X[(i0 + (l & 15)) * pitch + k0 + (l >> 4)];
    }
    static __device__ __forceinline__ t tr(const float* X, int pitch, int k0, int i0, int l) {
        return X[(k0 + (l >> 4)) * pitch + i0 + (l & 15)];
    }
    static __device__ __forceinline__ t kc(const float* X, int pitch, int i0, int k0) { return kc(X, pitch, i0, k0, lane_id()); }
    static __device__ __forceinline__ t tr(const float* X, int pitch, int k0, int i0) { return tr(X, pitch, k0, i0, lane_id()); }
    static __device__ __forceinline__ t gkc(const float* X, long pitch, int i0, int k0) {
        const int l = lane_id();
        return X[(long)(i0 + (l & 15)) * pitch + k0 + (l >> 4)];
    }
    static __device__ __forceinline__ t from_f32(const float* v) { return v[0]; }
    static __device__ __forceinline__ t scale(const t& x, const float* s) { return x * s[0]; }
    static __device__ __forceinline__ t scale(const t& x, float s) { return x * s; }
};

// ------------------------------------------------------------------ fragment-order tiles
// The per-chunk factor tiles ([64][cols], cols a multiple of KU) are stored in HBM in fragment
// order: a sequence of 1 KB pieces of 16 rows x KU columns (row-block major), and inside a piece
// the 16-byte unit u holds row u % 16, columns (u / 16) * VEC .. + VEC - 1.  Unit u is exactly
// what lane u needs for a bf16 MFMA operand fragment, so a fragment load is one contiguous 1 KB
// read (global or LDS) and a piece can be copied to LDS by one direct-to-LDS load per wave.
template <typename OT> struct FLay {
    static constexpr int ES = (int)sizeof(OT), VEC = 16 / ES, KU = 64 / ES;
    // element offset of (row, col) in a tile of `cols` columns
    static __device__ __forceinline__ int off(int row, int col, int cols) {
        return (((row >> 4) * (cols / KU) + col / KU) * 64 + ((col % KU) / VEC) * 16 + (row & 15)) * VEC +
               col % VEC;
    }
    // row and first column of 16-byte unit x
    static __device__ __forceinline__ int unit_row(int x, int cols) {
        const int piece = x >> 6;
        return (piece / (cols / KU)) * 16 + (x & 15);
    }
    static __device__ __forceinline__ int unit_col(int x, int cols) {
        const int piece = x >> 6;
        return (piece % (cols / KU)) * KU + ((x & 63) >> 4) * VEC;
    }
};

// Operand fragments read from a fragment-order tile of `cols` columns (LDS or global):
//   fkc(X, cols, i0, k0): rows i0 + l%16 of the tile, k = columns (as Frag::kc on a row-major tile)
//   ftr(X, cols, k0, i0): the transposed use, index = column i0 + l%16, k = rows (as Frag::tr)
template <typename OT> struct FFrag;
template <> struct FFrag<bf16> {
    typedef bf16x8 t;
    static __device__ __forceinline__ t fkc(const bf16* X, int cols, int i0, int k0, int l) {
        return *(const bf16x8*)(X + FLay<bf16>::off(i0 + (l & 15), k0 + 8 * (l >> 4), cols));
    }
    static __device__ __forceinline__ t fkc(const bf16* X, int cols, int i0, int k0) { return fkc(X, cols, i0, k0, lane_id()); }
    static __device__ __forceinline__ t ftr(const bf16* X, int cols, int k0, int i0) { return ftr(X, cols, k0, i0, lane_id()); }
    static __device__ __forceinline__ t ftr(const bf16* X, int cols, int k0, int i0, int l) {
        const int p = l & 15, kb = k0 + 8 * (l >> 4) + (p >> 2);
        const int c = i0 + 4 * (p & 3);
        bf16x4 lo = ds_read_tr4(X + FLay<bf16>::off(kb, c, cols));
        bf16x4 hi = ds_read_tr4(X + FLay<bf16>::off(kb + 4, c, cols));
        return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
};
template <> struct FFrag<float> {
    typedef float t;
    static __device__ __forceinline__ t fkc(const float* X, int cols, int i0, int k0, int l) {
        return X[FLay<float>::off(i0 + (l & 15), k0 + (l >> 4), cols)];
    }
    static __device__ __forceinline__ t ftr(const float* X, int cols, int k0, int i0, int l) {
        return X[FLay<float>::off(k0 + (l >> 4), i0 + (l & 15), cols)];
    }
    static __device__ __forceinline__ t fkc(const float* X, int cols, int i0, int k0) { return fkc(X, cols, i0, k0, lane_id()); }
    static __device__ __forceinline__ t ftr(const float* X, int cols, int k0, int i0) { return ftr(X, cols, k0, i0, lane_id()); }
};

// Activations of the fused prologue.
// sigmoid with the hardware reciprocal (v_rcp_f32, 1 ulp) instead of a correctly rounded divide
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
// softplus(x) = ln(1 + e^x) with the hardware log2 (v_log_f32); its argument is >= 1, so the
// denormal handling of a full logf is not needed
__device__ __forceinline__ float softplus_f(float x) {
    return x > 20.f ? x : 0.69314718f * __builtin_amdgcn_logf(1.f + __expf(x));
}

// ------------------------------------------------------------------ deep-decay support
// The Gram products split exp(G_r - G_s) (r >= s, G = in-chunk cumsum of log alpha) into a left
// factor exp(G_r - ref) <= 1 and a right factor exp(ref - G_s) >= 1 around one reference per
// 16-token block.  The right factor is bounded by the decay across the block; when any channel of
// a chunk decays by more than exp(-kDeepDecay) across one block, the kernels take a second path in
// which every factor is <= 1 (right operands referenced to the end of their block, diagonal
// blocks computed entry by entry).  exp(kDeepDecay) leaves a 1e12 margin below the fp32 range for
// the products and sums the fast path forms from such factors.
constexpr float kDeepDecay = 60.f;

// Compile-time loop: f(IC<i>{}) for i = B .. E-1 (for builtins that need constant operands).
template <int V> struct IC { static constexpr int value = V; };
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// Value of lane T of the caller's DPP row (lanes 16(l/16) .. +15): DPP row_newbcast.
template <int T>
__device__ __forceinline__ float row_bcast(float x) {
    static_assert(T >= 0 && T < 16, "lane of a 16-lane row");
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x150 + T,
                                                                 0xf, 0xf, false));
}

// Inclusive suffix sum over the 16 lanes of each DPP row: lane i gets the sum of lanes i..15.
__device__ __forceinline__ float row_rscan16(float x) {
    int v = __builtin_bit_cast(int, x);
    float y;
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x101, 0xf, 0xf, false));
    x += y; v = __builtin_bit_cast(int, x);
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x102, 0xf, 0xf, false));
    x += y; v = __builtin_bit_cast(int, x);
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x104, 0xf, 0xf, false));
    x += y; v = __builtin_bit_cast(int, x);
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x108, 0xf, 0xf, false));
    return x + y;
}

// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16g .. 16g+15).
__device__ __forceinline__ float row_scan16(float x) {
    int v = __builtin_bit_cast(int, x);
    float y;
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false));
    x += y; v = __builtin_bit_cast(int, x);
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false));
    x += y; v = __builtin_bit_cast(int, x);
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false));
    x += y; v = __builtin_bit_cast(int, x);
    y = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false));
    return x + y;
}
}  // namespace gdr2
