// Host-only driver for the C ABI's validation under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// The library's host code (gdr2_api.hip, compiled as plain C++) is linked against stand-ins for the
// kernel launchers: they count launches and touch no memory, so every entry point runs its full
// validation and size arithmetic on the host, valid calls included.  Each case states the status
// the header promises; any mismatch, sanitizer report or launch after a rejected call fails.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdr2.h"
#include "gdr2_kernels.hpp"

namespace gdr2 {
static long g_launches = 0;
hipError_t wy_dispatch(int, int, int, const FwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t carry_fwd_dispatch(int, int, int, const FwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t decode_dispatch(int, int, int, const DecodeParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t dstate_dispatch(int, int, int, const BwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t bgrad_dispatch(int, int, int, const BwdParams&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t epi_dispatch(int, int, bool, const EpiParams&, hipStream_t) { ++g_launches; return hipSuccess; }
// stand-ins for the two host-side sizing rules of the launchers (value slices of the state carry,
// workgroups of the output epilogue); any positive answer exercises the same validation
int carry_slice_width(int, int, int dv, long) { return dv >= 32 ? 32 : 16; }
long epi_blocks(long rows) { return (rows + 127) / 128; }
// stand-in address of the static scratch (never dereferenced: the launches are stand-ins too)
hipError_t noalloc_scratch(void** ptr) { *ptr = (void*)(uintptr_t)0x7f0000000000ull; return hipSuccess; }
}  // namespace gdr2

// stand-ins for the runtime calls of the pipelined long-sequence path (second stream, events):
// handles that are never dereferenced
extern "C" {
hipError_t hipGetDevice(int* dev) { *dev = 0; return hipSuccess; }
hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
    *s = (hipStream_t)(uintptr_t)0x5100;
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    static uintptr_t next = 0x6100;
    *e = (hipEvent_t)(next += 0x10);
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned int) { return hipSuccess; }
}

static int g_fail = 0;
#define EXPECT(call, want, launch)                                                              \
    do {                                                                                        \
        const long before = gdr2::g_launches;                                                  \
        const int got = (int)(call);                                                           \
        const bool launched = gdr2::g_launches != before;                                      \
        if (got != (want) || launched != (launch)) {                                            \
            std::printf("FAIL line %d: %s -> %d (want %d), launched %d\n", __LINE__, #call, got, \
                        (int)(want), (int)launched);                                            \
            ++g_fail;                                                                           \
        }                                                                                       \
    } while (0)

// 16-byte aligned host buffers standing in for device memory (never read by the library)
struct Buf {
    std::vector<unsigned char> raw;
    void* p;
    explicit Buf(size_t n) : raw(n + 64) { p = (void*)(((uintptr_t)raw.data() + 15) & ~(uintptr_t)15); }
    float* f() { return (float*)p; }
};

static void chunked_cases(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt) {
    const size_t es = gdr2_dtype_size(dt), nt = (size_t)(B * T * H), ns = (size_t)(B * H * dk * dv);
    Buf q(nt * dk * es), k(nt * dk * es), v(nt * dv * es), la(nt * dk * 4), b(nt * dk * es), w(nt * dv * es);
    Buf S0(ns * 4), o(nt * dv * es), ST(ns * 4), dO(nt * dv * es), dST(ns * 4), dS0(ns * 4);
    Buf dq(nt * dk * es), dk_(nt * dk * es), dv_(nt * dv * es), dla(nt * dk * 4), db(nt * dk * es), dw(nt * dv * es);
    const size_t fwb = gdr2_fwd_workspace_bytes(B, T, H, dk, dv, dt);
    const size_t inb = gdr2_fwd_infer_workspace_bytes(B, T, H, dk, dv, dt);
    const size_t bwb = gdr2_bwd_workspace_bytes(B, T, H, dk, dv, dt);
    const size_t rcb = gdr2_bwd_recompute_workspace_bytes(B, T, H, dk, dv, dt);
    if (inb > fwb || rcb != fwb + bwb) { std::printf("FAIL workspace sizes\n"); ++g_fail; }
    Buf fws(fwb + 16), bws(bwb + 16), rws(rcb + 16);
    const bool tok = T > 0;
    gdr2_prologue pro{0.1f, 1e-6f};
    for (unsigned gates = 0; gates < 8; ++gates) {
        for (int with_pro = 0; with_pro < 2; ++with_pro) {
            const gdr2_prologue* P = with_pro ? &pro : nullptr;
            EXPECT(gdr2_fwd_chunked_ex(B, T, H, dk, dv, dt, gates, P, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f(), o.p,
                                       ST.f(), fws.p, fwb, nullptr), GDR2_OK, true);
            EXPECT(gdr2_fwd_infer_ex(B, T, H, dk, dv, dt, gates, P, q.p, k.p, v.p, la.f(), b.p, w.p, nullptr, o.p,
                                     nullptr, fws.p, inb, nullptr), GDR2_OK, true);
            EXPECT(gdr2_bwd_chunked_ex(B, T, H, dk, dv, dt, gates, P, q.p, k.p, v.p, la.f(), b.p, w.p, fws.p, fwb,
                                       dO.p, dST.f(), dq.p, dk_.p, dv_.p, dla.f(), db.p, dw.p, dS0.f(), bws.p, bwb,
                                       nullptr), GDR2_OK, true);
            EXPECT(gdr2_bwd_chunked_recompute_ex(B, T, H, dk, dv, dt, gates, P, q.p, k.p, v.p, la.f(), b.p, w.p,
                                                 S0.f(), dO.p, dST.f(), dq.p, dk_.p, dv_.p, dla.f(), db.p, dw.p,
                                                 dS0.f(), rws.p, rcb, nullptr), GDR2_OK, true);
        }
    }
    if (tok) {
        EXPECT(gdr2_fwd_chunked(B, T, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f(), o.p, ST.f(),
                                fws.p, fwb - 1, nullptr), GDR2_E_WORKSPACE, false);
        EXPECT(gdr2_fwd_infer(B, T, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f(), o.p, ST.f(),
                              fws.p, inb - 1, nullptr), GDR2_E_WORKSPACE, false);
        EXPECT(gdr2_bwd_chunked_recompute(B, T, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f(), dO.p,
                                          nullptr, dq.p, dk_.p, dv_.p, dla.f(), db.p, dw.p, dS0.f(), rws.p,
                                          rcb - 1, nullptr), GDR2_E_WORKSPACE, false);
        EXPECT(gdr2_fwd_chunked(B, T, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f(), q.p, ST.f(),
                                fws.p, fwb, nullptr), GDR2_E_ALIAS, false);
        EXPECT(gdr2_bwd_chunked(B, T, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, fws.p, fwb, dO.p, nullptr,
                                dq.p, dk_.p, dv_.p, dla.f(), db.p, dw.p, dS0.f(), fws.p, bwb, nullptr),
               GDR2_E_ALIAS, false);
        EXPECT(gdr2_fwd_chunked(B, T, H, dk, dv, dt, nullptr, k.p, v.p, la.f(), b.p, w.p, S0.f(), o.p, ST.f(),
                                fws.p, fwb, nullptr), GDR2_E_NULL, false);
        EXPECT(gdr2_fwd_chunked(B, T, H, dk, dv, dt, (char*)q.p + 8, k.p, v.p, la.f(), b.p, w.p, S0.f(), o.p,
                                ST.f(), fws.p, fwb, nullptr), GDR2_E_ALIGN, false);
    }
    // the no-allocation forward-only call: same validation, factors in the library's scratch
    for (unsigned gates = 0; gates < 8; gates += 3)
        EXPECT(gdr2_fwd_infer_noalloc_ex(B, T, H, dk, dv, dt, gates, &pro, q.p, k.p, v.p, la.f(), b.p, w.p,
                                         S0.f(), o.p, ST.f(), nullptr), GDR2_OK, B * H > 0);
    if (tok) {
        EXPECT(gdr2_fwd_infer_noalloc_ex(B, T, H, dk, dv, dt, 0, nullptr, q.p, k.p, v.p, la.f(), b.p, w.p,
                                         S0.f(), q.p, ST.f(), nullptr), GDR2_E_ALIAS, false);
        EXPECT(gdr2_fwd_infer_noalloc_ex(B, T, H, dk, dv, dt, 0, nullptr, q.p, k.p, v.p, la.f(), b.p, w.p,
                                         S0.f(), nullptr, ST.f(), nullptr), GDR2_E_NULL, false);
    }
    // decode over the same buffers, one token per (sequence, head), in place
    if (tok) {
        EXPECT(gdr2_decode_step(B, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f(), S0.f(), o.p,
                                nullptr), GDR2_OK, true);
        EXPECT(gdr2_decode_step(B, H, dk, dv, dt, q.p, k.p, v.p, la.f(), b.p, w.p, S0.f() + 4, S0.f(), o.p,
                                nullptr), GDR2_E_ALIAS, false);
    }
    const int64_t rows = (int64_t)nt;
    const size_t ewb = gdr2_out_gate_bwd_workspace_bytes(rows, dv);
    Buf ews(ewb + 16), wt(dv * 4), dwt(dv * 4), gy(nt * dv * es), gdo(nt * dv * es), gdg(nt * dv * es);
    EXPECT(gdr2_out_gate_fwd(rows, dv, dt, o.p, dO.p, wt.f(), 1e-6f, v.p, nullptr), GDR2_OK, rows > 0);
    EXPECT(gdr2_out_gate_bwd(rows, dv, dt, o.p, dO.p, wt.f(), 1e-6f, gy.p, gdo.p, gdg.p, dwt.f(), ews.p, ewb,
                             nullptr), GDR2_OK, true);
    EXPECT(gdr2_out_gate_bwd(rows, dv, dt, o.p, dO.p, wt.f(), 1e-6f, gy.p, gdo.p, gdg.p, wt.f(), ews.p, ewb,
                             nullptr), GDR2_E_ALIAS, false);
}

static void huge_cases() {
    // sizes whose products overflow 64 bits must be rejected before any arithmetic wraps; the
    // pointers are never dereferenced
    void* P[24];
    for (int i = 0; i < 24; ++i) P[i] = (void*)(uintptr_t)(0x100000u * (i + 1));
    const int64_t big = (int64_t)1 << 40, huge = INT64_MAX;
    const int64_t shapes[][3] = {{big, 8, big}, {huge, 1, huge}, {1, (int64_t)1 << 41, 1}, {huge, huge, huge},
                                 {(int64_t)1 << 31, 64, (int64_t)1 << 31}, {1 << 20, (int64_t)1 << 31, 1}};
    for (const auto& s : shapes) {
        const int64_t B = s[0], T = s[1], H = s[2];
        if (gdr2_fwd_workspace_bytes(B, T, H, 128, 128, GDR2_BF16) != 0 ||
            gdr2_fwd_infer_workspace_bytes(B, T, H, 128, 128, GDR2_BF16) != 0 ||
            gdr2_bwd_workspace_bytes(B, T, H, 128, 128, GDR2_BF16) != 0 ||
            gdr2_bwd_recompute_workspace_bytes(B, T, H, 128, 128, GDR2_BF16) != 0) {
            std::printf("FAIL huge workspace query not 0\n");
            ++g_fail;
        }
        EXPECT(gdr2_fwd_chunked(B, T, H, 128, 128, GDR2_BF16, P[0], P[1], P[2], (float*)P[3], P[4], P[5],
                                nullptr, P[6], nullptr, P[7], SIZE_MAX, nullptr), GDR2_E_SHAPE, false);
        EXPECT(gdr2_fwd_infer(B, T, H, 128, 128, GDR2_BF16, P[0], P[1], P[2], (float*)P[3], P[4], P[5],
                              nullptr, P[6], nullptr, P[7], SIZE_MAX, nullptr), GDR2_E_SHAPE, false);
        EXPECT(gdr2_bwd_chunked(B, T, H, 128, 128, GDR2_BF16, P[0], P[1], P[2], (float*)P[3], P[4], P[5],
                                P[6], SIZE_MAX, P[7], nullptr, P[8], P[9], P[10], (float*)P[11], P[12], P[13],
                                nullptr, P[14], SIZE_MAX, nullptr), GDR2_E_SHAPE, false);
        EXPECT(gdr2_bwd_chunked_recompute(B, T, H, 128, 128, GDR2_BF16, P[0], P[1], P[2], (float*)P[3], P[4],
                                          P[5], nullptr, P[7], nullptr, P[8], P[9], P[10], (float*)P[11], P[12],
                                          P[13], nullptr, P[14], SIZE_MAX, nullptr), GDR2_E_SHAPE, false);
        if (B >= ((int64_t)1 << 31) && H >= 1)  // N*H beyond what one decode launch indexes
            EXPECT(gdr2_decode_step(B, H, 128, 128, GDR2_BF16, P[0], P[1], P[2], (float*)P[3], P[4], P[5],
                                    nullptr, (float*)P[6], P[7], nullptr), GDR2_E_SHAPE, false);
    }
    EXPECT(gdr2_out_gate_fwd(huge, 128, GDR2_BF16, P[0], P[1], (float*)P[2], 1e-6f, P[3], nullptr), GDR2_E_SHAPE,
           false);
    // factors beyond the no-allocation scratch: a valid shape that needs more than 128 MiB
    void* F[7];  // 4 GiB apart: the token tensors of this shape do not overlap
    for (int i = 0; i < 7; ++i) F[i] = (void*)(uintptr_t)(((uintptr_t)1 << 32) * (i + 1));
    EXPECT(gdr2_fwd_infer_noalloc_ex(1, 64 * 1700, 1, 128, 128, GDR2_BF16, 0, nullptr, F[0], F[1], F[2],
                                     (float*)F[3], F[4], F[5], nullptr, F[6], nullptr, nullptr),
           GDR2_E_TOO_LARGE, false);
    if (gdr2_out_gate_bwd_workspace_bytes(-5, 128) != 0) { std::printf("FAIL negative rows\n"); ++g_fail; }
}

int main() {
    const gdr2_dtype dts[2] = {GDR2_BF16, GDR2_F32};
    for (gdr2_dtype dt : dts) {
        chunked_cases(2, 70, 3, 128, 64, dt);
        chunked_cases(1, 1, 2, 64, 128, dt);
        chunked_cases(2, 0, 2, 64, 64, dt);
        chunked_cases(1, 64 * 256 + 6, 4, 64, 64, dt);  // bf16: the pipelined long-sequence path
    }
    huge_cases();
    std::printf("%s: %d failures, %ld launches\n", g_fail ? "FAIL" : "ok", g_fail, gdr2::g_launches);
    return g_fail ? 1 : 0;
}
