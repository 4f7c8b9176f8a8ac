// gdr2_api.hip -- the C ABI declared in include/gdr2.h: host-side validation, then kernel launch.
// Nothing here touches device memory before every check has passed.
#include "gdr2.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "gdr2_kernels.hpp"

namespace {

struct Range {
    const void* p;
    size_t n;
};

bool overlap(const Range& a, const Range& b) {
    if (!a.p || !b.p || a.n == 0 || b.n == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.n && b0 < a0 + a.n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool dims_ok(int64_t d) { return d == 64 || d == 128; }

// Any output overlapping any input or another output?
bool any_alias(const Range* outs, int no, const Range* ins, int ni) {
    for (int i = 0; i < no; ++i) {
        for (int j = 0; j < ni; ++j)
            if (overlap(outs[i], ins[j])) return true;
        for (int j = i + 1; j < no; ++j)
            if (overlap(outs[i], outs[j])) return true;
    }
    return false;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// a * b <= lim for a, b >= 0, decided without forming a product that could overflow
bool prod_le(int64_t a, int64_t b, int64_t lim) { return a == 0 || b <= lim / a; }

bool gates_ok(unsigned gates) { return (gates & ~7u) == 0; }

bool prologue_ok(const gdr2_prologue* pro) {
    if (!pro) return true;
    const float c = pro->decay_scale, e = pro->norm_eps;
    return c > 0.f && c < 1e30f && e > 0.f && e < 1e30f;
}

gdr2::Prologue prologue_of(const gdr2_prologue* pro) {
    gdr2::Prologue x;
    x.decay_scale = pro ? pro->decay_scale : 0.f;
    x.norm_eps = pro ? pro->norm_eps : 0.f;
    return x;
}

// Elements of b, w and log alpha (and of db, dw, dlog alpha) for `tokens` token-heads.
struct GateSizes {
    size_t nb, nw, na;
};
GateSizes gate_sizes(unsigned gates, size_t tokens, int64_t dk, int64_t dv) {
    return {(gates & GDR2_ERASE_SCALAR) ? tokens : tokens * dk,
            (gates & GDR2_WRITE_SCALAR) ? tokens : tokens * dv,
            (gates & GDR2_DECAY_SCALAR) ? tokens : tokens * dk};
}

}  // namespace

extern "C" {

size_t gdr2_dtype_size(gdr2_dtype dt) {
    return dt == GDR2_F32 ? 4 : dt == GDR2_BF16 ? 2 : 0;
}

int64_t gdr2_num_chunks(int64_t T) { return T <= 0 ? 0 : (T + GDR2_CHUNK - 1) / GDR2_CHUNK; }

const char* gdr2_status_string(gdr2_status s) {
    switch (s) {
        case GDR2_OK: return "ok";
        case GDR2_E_NULL: return "required pointer is NULL";
        case GDR2_E_SHAPE: return "invalid size";
        case GDR2_E_DTYPE: return "unknown dtype";
        case GDR2_E_UNSUPPORTED: return "unsupported head size / dtype combination";
        case GDR2_E_ALIGN: return "pointer not 16-byte aligned";
        case GDR2_E_ALIAS: return "output overlaps an input or another output";
        case GDR2_E_WORKSPACE: return "workspace missing or too small";
        case GDR2_E_HIP: return "HIP launch failed";
        case GDR2_E_VALUE: return "invalid scalar argument";
        case GDR2_E_TOO_LARGE: return "problem exceeds the no-allocation entry point's static scratch";
    }
    return "unknown status";
}

int gdr2_abi_version(void) { return GDR2_ABI_VERSION; }

// ------------------------------------------------------------------ pipelined long sequences
// When the 16-bit state carries occupy at most half of the compute units (few chains: a long
// sequence at a small batch), the composed calls split the chunks into ranges and run the
// chunk-parallel kernel of the later ranges on a second stream, on the idle compute units, while
// the carry walks the earlier ones on the caller's stream: the factor kernel beside the forward
// carry, the chunk-gradient kernel beside the backward state carry.  The carry hands its fp32
// state from one range to the next through a buffer at the end of the workspace, so the results
// are bitwise those of the unsplit calls.  The decision depends on the shapes only (the size
// queries need no device): at most kPipeMaxCarryWGs carry workgroups (half of MI355X's 256
// compute units), and at least two ranges of kPipeRangeChunks chunks and kPipeRangeChunkHeads
// chunk-heads each, so that every chunk-parallel launch still fills the other half of the chip
// and every range of the carry is long enough to pay for the switch between ranges.  More or
// shorter ranges cost more than they overlap: each new range of the carry has to win its compute
// units back from the chunk-parallel kernel queued beside it (fwd+bwd at B=1 T=32768 H=16: 2374
// us unsplit, 2277 / 2194 / 2236 us with 2 / 4 / 8 ranges, 2156 us once the side stream also waits
// for the first range's factors; at B=1 T=8192 H=16: 593 us unsplit, 633 / 605 us with four
// ranges of 32 / two of 64 chunks).
constexpr int64_t kPipeMaxCarryWGs = 128;
constexpr int64_t kPipeRangeChunks = 128;
constexpr int64_t kPipeRangeChunkHeads = 512;
constexpr int kPipeMaxPieces = 4;

static int pipe_pieces(int64_t chains, int64_t NC) {
    int64_t n = chains * NC / kPipeRangeChunkHeads;
    if (NC / kPipeRangeChunks < n) n = NC / kPipeRangeChunks;
    return (int)(n < kPipeMaxPieces ? n : kPipeMaxPieces);
}
static bool pipelined(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt) {
    if (dt != GDR2_BF16 || B <= 0 || H <= 0) return false;
    const int64_t chains = B * H;
    if (chains > kPipeMaxCarryWGs) return false;
    const int dvs = gdr2::carry_slice_width(1, (int)dk, (int)dv, chains);
    return chains * (dv / dvs) <= kPipeMaxCarryWGs && pipe_pieces(chains, gdr2_num_chunks(T)) >= 2;
}
static int pipe_bound(int64_t NC, int np, int k) { return (int)(NC * k / np); }  // chunk of range k

// The second stream and its events, one set per device, created on first use and kept until the
// process ends.  Calls that pipeline hold the device's lock while they enqueue, so that two host
// threads never interleave their records and waits on the shared events.
struct Pipe {
    hipStream_t side = nullptr;
    hipEvent_t ev[kPipeMaxPieces + 2] = {};
    std::mutex mu;
    bool tried = false, ok = false;
};
static Pipe* pipe_of_device() {
    static std::mutex mu;
    static Pipe per_device[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> g(mu);
    Pipe& P = per_device[dev];
    if (!P.tried) {
        P.tried = true;
        bool ok = hipStreamCreateWithFlags(&P.side, hipStreamNonBlocking) == hipSuccess;
        for (hipEvent_t& e : P.ev)
            ok = ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) == hipSuccess;
        P.ok = ok;
    }
    return P.ok ? &P : nullptr;
}

// Layout of the forward workspace: per-chunk WY factors, then the chunk-entry states, then (for
// pipelined shapes) the fp32 state hand-off buffer.  A forward-only workspace holds the factors and
// the hand-off buffer right after them.
struct FwdWs {
    size_t yh, qg, kt, p, tm, u, gam, states, total;
    size_t pipe_bytes;   // hand-off buffer (0: shape not pipelined)
    size_t infer_total;  // forward-only workspace
};
static size_t pipe_train_off(const FwdWs& L) { return L.total - L.pipe_bytes; }
static size_t pipe_infer_off(const FwdWs& L) { return L.states; }
static FwdWs fwd_ws_layout(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt) {
    const size_t es = gdr2_dtype_size(dt);
    const size_t ncc = (size_t)B * H * gdr2_num_chunks(T);
    const size_t C = GDR2_CHUNK;
    FwdWs w;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off += round_up(bytes, 256); return o; };
    w.yh = take(ncc * C * dk * es);
    w.qg = take(ncc * C * dk * es);
    w.kt = take(ncc * C * dk * es);
    w.p = take(ncc * C * C * es);
    w.tm = take(ncc * C * C * es);
    w.u = take(ncc * C * dv * es);
    w.gam = take(ncc * dk * 4);
    w.states = take(ncc * dv * dk * es);
    w.pipe_bytes = pipelined(B, T, H, dk, dv, dt) ? round_up((size_t)B * H * dk * dv * 4, 256) : 0;
    w.total = off + w.pipe_bytes;
    w.infer_total = w.states + w.pipe_bytes;
    return w;
}

static gdr2::WyBufs wy_bufs(const FwdWs& L, void* base) {
    char* b = (char*)base;
    gdr2::WyBufs w;
    w.Yh = b + L.yh;
    w.Qg = b + L.qg;
    w.Kt = b + L.kt;
    w.P = b + L.p;
    w.Tm = b + L.tm;
    w.U = b + L.u;
    w.gam = (float*)(b + L.gam);
    return w;
}

// Shared shape / dtype checks of the two chunked passes.  Each bound is tested before any product
// that depends on it, so that no size arithmetic here or in the layouts below can overflow: after
// it, B*H <= 2^30 chains, B*H*ceil(T/64) <= 2^30 chunk-heads, B*T*H <= 2^50 head-tokens.
static gdr2_status check_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                 gdr2_dtype dt) {
    if (dt != GDR2_F32 && dt != GDR2_BF16) return GDR2_E_DTYPE;
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return GDR2_E_SHAPE;
    if (!dims_ok(dk) || !dims_ok(dv)) return GDR2_E_UNSUPPORTED;
    if (T > ((int64_t)1 << 40) || !prod_le(B, H, (int64_t)1 << 30)) return GDR2_E_SHAPE;
    const int64_t BH = B * H;
    if (!prod_le(BH, dv / 16, (int64_t)1 << 30)) return GDR2_E_SHAPE;
    if (!prod_le(BH, gdr2_num_chunks(T), (int64_t)1 << 30)) return GDR2_E_SHAPE;
    if (!prod_le(BH, T, (int64_t)1 << 50)) return GDR2_E_SHAPE;
    return GDR2_OK;
}

size_t gdr2_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt) {
    if (check_chunked(B, T, H, dk, dv, dt) != GDR2_OK) return 0;
    return fwd_ws_layout(B, T, H, dk, dv, dt).total;
}

size_t gdr2_fwd_infer_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      gdr2_dtype dt) {
    if (check_chunked(B, T, H, dk, dv, dt) != GDR2_OK) return 0;
    return fwd_ws_layout(B, T, H, dk, dv, dt).infer_total;  // the factors (+ hand-off buffer)
}

// Backward workspace: the per-chunk exit-state gradients, then (pipelined shapes) the fp32
// hand-off buffer of the state-gradient carry.
static size_t bwd_dsx_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt) {
    return round_up((size_t)B * H * gdr2_num_chunks(T) * dk * dv * gdr2_dtype_size(dt), 256);
}
size_t gdr2_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt) {
    if (check_chunked(B, T, H, dk, dv, dt) != GDR2_OK) return 0;
    const size_t pipe = pipelined(B, T, H, dk, dv, dt) ? round_up((size_t)B * H * dk * dv * 4, 256) : 0;
    return bwd_dsx_bytes(B, T, H, dk, dv, dt) + pipe;
}

size_t gdr2_bwd_recompute_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                          gdr2_dtype dt) {
    if (check_chunked(B, T, H, dk, dv, dt) != GDR2_OK) return 0;
    return fwd_ws_layout(B, T, H, dk, dv, dt).total + gdr2_bwd_workspace_bytes(B, T, H, dk, dv, dt);
}

static gdr2::FwdParams fwd_params(int64_t B, int64_t T, int64_t H, int64_t dv, const void* q,
                                  const void* k, const void* v, const float* la, const void* b,
                                  const void* w, const float* S0, void* o, float* S_T,
                                  const FwdWs& L, void* ws, int dvs, unsigned gates = 0) {
    gdr2::FwdParams p;
    p.gates = (int)gates;
    p.prologue = 0;
    p.pro = prologue_of(nullptr);
    p.B = (int)B;
    p.H = (int)H;
    p.NS = (int)(dv / dvs);
    p.NC = (int)gdr2_num_chunks(T);
    p.c0 = 0;          // every chunk (a pipelined call narrows the range per launch)
    p.ncr = p.NC;
    p.T = T;
    p.DV = dv;
    p.q = q; p.k = k; p.v = v; p.b = b; p.w = w;
    p.la = la;
    p.S0 = S0;
    p.o = o;
    p.ST = S_T;
    p.states = ws ? (char*)ws + L.states : nullptr;
    p.wy = wy_bufs(L, ws);
    p.stream = L.states >= gdr2::kStreamFactorBytes;  // L.states = bytes of the factor tiles
    return p;
}

// Validation shared by the forward phases.  `need_inputs` / `need_out` select which pointers a
// phase requires; every pointer given must be aligned and every output disjoint from the inputs.
// `with_states`: the workspace also holds the chunk-entry states (training); without them it holds
// only the factors (forward-only calls).  `caller_ws` false: the factors go to the library's own
// scratch, so no workspace argument is checked.
static gdr2_status check_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dt, const void* q, const void* k, const void* v,
                             const float* la, const void* b, const void* w, const float* S0,
                             void* o, float* S_T, void* ws, size_t ws_bytes, bool need_inputs,
                             bool need_out, unsigned gates = 0, bool with_states = true,
                             bool caller_ws = true) {
    gdr2_status st = check_chunked(B, T, H, dk, dv, dt);
    if (st != GDR2_OK) return st;
    if (!gates_ok(gates)) return GDR2_E_UNSUPPORTED;
    const bool have_tokens = B > 0 && H > 0 && T > 0;
    if (have_tokens && need_inputs && (!q || !k || !v || !la || !b || !w)) return GDR2_E_NULL;
    if (have_tokens && need_out && !o) return GDR2_E_NULL;
    const void* ptrs[] = {q, k, v, la, b, w, S0, o, S_T, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDR2_E_ALIGN;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    const size_t ws_need = with_states ? L.total : L.infer_total;
    if (caller_ws && have_tokens && (!ws || ws_bytes < ws_need)) return GDR2_E_WORKSPACE;
    const size_t es = gdr2_dtype_size(dt);
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv;
    const size_t ns = (size_t)B * H * dk * dv;
    const GateSizes gs = gate_sizes(gates, (size_t)B * T * H, dk, dv);
    const Range ins[] = {{q, nk * es}, {k, nk * es}, {v, nv * es}, {la, gs.na * 4},
                         {b, gs.nb * es}, {w, gs.nw * es}, {S0, ns * 4}};
    const Range outs[] = {{o, nv * es}, {S_T, ns * 4}, {ws, have_tokens && caller_ws ? ws_need : 0}};
    if (any_alias(outs, 3, ins, 7)) return GDR2_E_ALIAS;
    return GDR2_OK;
}

gdr2_status gdr2_fwd_factors_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                                const void* q, const void* k,
                                const void* v, const float* log_alpha, const void* b,
                                const void* w, void* workspace, size_t workspace_bytes,
                                void* stream) {
    gdr2_status st = check_fwd(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, nullptr, nullptr,
                               nullptr, workspace, workspace_bytes, true, false, gates);
    if (st == GDR2_OK && !prologue_ok(pro)) st = GDR2_E_VALUE;
    if (st != GDR2_OK || B == 0 || H == 0 || T == 0) return st;
    const int bf = dt == GDR2_BF16;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    gdr2::FwdParams p = fwd_params(B, T, H, dv, q, k, v, log_alpha, b, w, nullptr, nullptr,
                                   nullptr, L, workspace, 16, gates);
    p.prologue = pro != nullptr;
    p.pro = prologue_of(pro);
    hipError_t e = gdr2::wy_dispatch(bf, (int)dk, (int)dv, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_fwd_factors(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dt, const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return gdr2_fwd_factors_ex(B, T, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b, w,
                               workspace, workspace_bytes, stream);
}

// The state carry after validation: o (may be NULL), S_T (may be NULL) and, with `with_states`,
// the chunk-entry states in the workspace's states region.
static gdr2_status launch_carry(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt, const float* S0, void* o, float* S_T,
                                void* workspace, bool with_states, void* stream) {
    const int bf = dt == GDR2_BF16;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    const int dvs = gdr2::carry_slice_width(bf, (int)dk, (int)dv, B * H);
    gdr2::FwdParams p = fwd_params(B, T, H, dv, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, S0, o, S_T, L, T > 0 ? workspace : nullptr, dvs);
    if (!with_states) p.states = nullptr;
    hipError_t e = gdr2::carry_fwd_dispatch(bf, (int)dk, dvs, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_fwd_carry(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dt, const float* S0, void* o, float* S_T, void* workspace,
                           size_t workspace_bytes, void* stream) {
    gdr2_status st = check_fwd(B, T, H, dk, dv, dt, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, S0, o, S_T, workspace, workspace_bytes, false, true);
    if (st != GDR2_OK || B == 0 || H == 0) return st;
    return launch_carry(B, T, H, dk, dv, dt, S0, o, S_T, workspace, true, stream);
}

// Factor kernel and state carry of a validated forward (B, H > 0).  `with_states`: training
// workspace (chunk-entry states kept) or forward-only workspace.  `allow_pipe`: the chunk ranges
// may be pipelined over a second stream (not for the no-allocation entry point).
static gdr2_status fwd_launch(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                              const void* q, const void* k, const void* v, const float* la,
                              const void* b, const void* w, const float* S0, void* o, float* S_T,
                              void* ws, bool with_states, bool allow_pipe, void* stream) {
    if (T == 0) return launch_carry(B, T, H, dk, dv, dt, S0, o, S_T, ws, with_states, stream);
    const int bf = dt == GDR2_BF16;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    hipStream_t m = (hipStream_t)stream;
    gdr2::FwdParams pw = fwd_params(B, T, H, dv, q, k, v, la, b, w, nullptr, nullptr, nullptr, L,
                                    ws, 16, gates);
    pw.prologue = pro != nullptr;
    pw.pro = prologue_of(pro);
    Pipe* P = (allow_pipe && L.pipe_bytes) ? pipe_of_device() : nullptr;
    if (!P) {
        if (gdr2::wy_dispatch(bf, (int)dk, (int)dv, pw, m) != hipSuccess) return GDR2_E_HIP;
        return launch_carry(B, T, H, dk, dv, dt, S0, o, S_T, ws, with_states, stream);
    }
    std::lock_guard<std::mutex> g(P->mu);
    hipStream_t s = P->side;
    const int64_t NC = gdr2_num_chunks(T);
    const int np = pipe_pieces(B * H, NC);
    float* hand = (float*)((char*)ws + (with_states ? pipe_train_off(L) : pipe_infer_off(L)));
    const int dvs = gdr2::carry_slice_width(bf, (int)dk, (int)dv, B * H);
    gdr2::FwdParams pc = fwd_params(B, T, H, dv, nullptr, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, S0, o, S_T, L, ws, dvs);
    if (!with_states) pc.states = nullptr;
    // factors of range 0 on the caller's stream (the whole chip); the side stream starts after
    // them, so that the factors of ranges 1.. share the chip only with the carry, each announced
    // by an event
    bool ok = true;
    for (int r = 0; ok && r < np; ++r) {
        pw.c0 = pipe_bound(NC, np, r);
        pw.ncr = pipe_bound(NC, np, r + 1) - pw.c0;
        ok = gdr2::wy_dispatch(bf, (int)dk, (int)dv, pw, r == 0 ? m : s) == hipSuccess;
        if (ok && r == 0)
            ok = hipEventRecord(P->ev[0], m) == hipSuccess && hipStreamWaitEvent(s, P->ev[0], 0) == hipSuccess;
        if (ok && r > 0) ok = hipEventRecord(P->ev[r], s) == hipSuccess;
    }
    // the carry walks the ranges on the caller's stream, its fp32 state handed over in `hand`
    for (int r = 0; ok && r < np; ++r) {
        if (r > 0) ok = hipStreamWaitEvent(m, P->ev[r], 0) == hipSuccess;
        pc.c0 = pipe_bound(NC, np, r);
        pc.ncr = pipe_bound(NC, np, r + 1) - pc.c0;
        pc.S0 = r == 0 ? S0 : hand;
        pc.ST = r == np - 1 ? S_T : hand;
        if (ok) ok = gdr2::carry_fwd_dispatch(bf, (int)dk, dvs, pc, m) == hipSuccess;
    }
    return ok ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_fwd_infer_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                              const void* q, const void* k, const void* v,
                              const float* log_alpha, const void* b, const void* w,
                              const float* S0, void* o, float* S_T, void* workspace,
                              size_t workspace_bytes, void* stream) {
    gdr2_status st = check_fwd(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, S0, o, S_T,
                               workspace, workspace_bytes, true, true, gates, false);
    if (st == GDR2_OK && !prologue_ok(pro)) st = GDR2_E_VALUE;
    if (st != GDR2_OK || B == 0 || H == 0) return st;
    return fwd_launch(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w, S0, o, S_T,
                      workspace, false, true, stream);
}

size_t gdr2_fwd_infer_noalloc_max_bytes(void) { return gdr2::kNoAllocScratchBytes; }

gdr2_status gdr2_fwd_infer_noalloc_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                                      const void* q, const void* k, const void* v,
                                      const float* log_alpha, const void* b, const void* w,
                                      const float* S0, void* o, float* S_T, void* stream) {
    gdr2_status st = check_fwd(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, S0, o, S_T, nullptr,
                               0, true, true, gates, false, false);
    if (st == GDR2_OK && !prologue_ok(pro)) st = GDR2_E_VALUE;
    if (st != GDR2_OK) return st;
    const size_t need = fwd_ws_layout(B, T, H, dk, dv, dt).states;
    if (need > gdr2::kNoAllocScratchBytes) return GDR2_E_TOO_LARGE;
    if (B == 0 || H == 0) return GDR2_OK;
    // the factors go to this device's static scratch (library memory: it cannot overlap the
    // caller's buffers); the launches are those of gdr2_fwd_infer_ex, never pipelined (that would
    // create the second stream and need the hand-off buffer)
    void* scr = nullptr;
    if (gdr2::noalloc_scratch(&scr) != hipSuccess) return GDR2_E_HIP;
    return fwd_launch(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w, S0, o, S_T, scr,
                      false, false, stream);
}

gdr2_status gdr2_fwd_infer(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dt, const void* q, const void* k, const void* v,
                           const float* log_alpha, const void* b, const void* w, const float* S0,
                           void* o, float* S_T, void* workspace, size_t workspace_bytes,
                           void* stream) {
    return gdr2_fwd_infer_ex(B, T, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b, w, S0, o,
                             S_T, workspace, workspace_bytes, stream);
}

gdr2_status gdr2_fwd_chunked_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                                const void* q, const void* k,
                                const void* v, const float* log_alpha, const void* b,
                                const void* w, const float* S0, void* o, float* S_T,
                                void* workspace, size_t workspace_bytes, void* stream) {
    gdr2_status st = check_fwd(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, S0, o, S_T,
                               workspace, workspace_bytes, true, true, gates);
    if (st == GDR2_OK && !prologue_ok(pro)) st = GDR2_E_VALUE;
    if (st != GDR2_OK || B == 0 || H == 0) return st;
    return fwd_launch(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w, S0, o, S_T,
                      workspace, true, true, stream);
}

gdr2_status gdr2_fwd_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dt, const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const float* S0, void* o, float* S_T, void* workspace,
                             size_t workspace_bytes, void* stream) {
    return gdr2_fwd_chunked_ex(B, T, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b, w, S0, o,
                               S_T, workspace, workspace_bytes, stream);
}

// Validation shared by the backward phases.
static gdr2_status check_bwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dt, const void* q, const void* k, const void* v,
                             const float* la, const void* b, const void* w, const void* fws,
                             size_t fws_bytes, const void* dO, const float* dS_T, void* dq,
                             void* dk_, void* dv_, float* dla, void* db, void* dw, float* dS0,
                             const void* ws, size_t ws_bytes, bool need_inputs, bool need_grads,
                             unsigned gates = 0) {
    gdr2_status st = check_chunked(B, T, H, dk, dv, dt);
    if (st != GDR2_OK) return st;
    if (!gates_ok(gates)) return GDR2_E_UNSUPPORTED;
    const bool have_tokens = B > 0 && H > 0 && T > 0;
    if (have_tokens && (!fws || !dO)) return GDR2_E_NULL;
    if (have_tokens && need_inputs && (!q || !k || !v || !la || !b || !w)) return GDR2_E_NULL;
    if (have_tokens && need_grads && (!dq || !dk_ || !dv_ || !dla || !db || !dw)) return GDR2_E_NULL;
    const void* ptrs[] = {q, k, v, la, b, w, fws, dO, dS_T, dq, dk_, dv_, dla, db, dw, dS0, ws};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDR2_E_ALIGN;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    const size_t need = gdr2_bwd_workspace_bytes(B, T, H, dk, dv, dt);
    if (have_tokens && (fws_bytes < L.total || !ws || ws_bytes < need)) return GDR2_E_WORKSPACE;
    const size_t es = gdr2_dtype_size(dt);
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv;
    const size_t ns = (size_t)B * H * dk * dv;
    const GateSizes gs = gate_sizes(gates, (size_t)B * T * H, dk, dv);
    const Range ins[] = {{q, nk * es},      {k, nk * es},      {v, nv * es},
                         {la, gs.na * 4},   {b, gs.nb * es},   {w, gs.nw * es},
                         {fws, have_tokens ? L.total : 0}, {dO, nv * es}, {dS_T, ns * 4}};
    // the state phase writes the workspace; the gradient phase reads it (then it is an input)
    const Range outs[] = {{dq, nk * es},     {dk_, nk * es},    {dv_, nv * es},
                          {dla, gs.na * 4},  {db, gs.nb * es},  {dw, gs.nw * es},
                          {dS0, ns * 4},     {ws, have_tokens ? need : 0}};
    if (any_alias(outs, 8, ins, 9)) return GDR2_E_ALIAS;
    return GDR2_OK;
}

static gdr2::BwdParams bwd_params(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                  gdr2_dtype dt, const void* q, const void* k, const void* v,
                                  const float* la, const void* b, const void* w, const void* fws,
                                  const void* dO, const float* dS_T, void* dq, void* dk_,
                                  void* dv_, float* dla, void* db, void* dw, float* dS0,
                                  const void* ws, unsigned gates = 0) {
    const int bf = dt == GDR2_BF16;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    gdr2::BwdParams p;
    p.gates = (int)gates;
    p.prologue = 0;
    p.pro = prologue_of(nullptr);
    p.B = (int)B; p.H = (int)H; p.NC = (int)gdr2_num_chunks(T); p.T = T; p.DV = dv;
    p.c0 = 0;
    p.ncr = p.NC;
    p.NS = (int)(dv / gdr2::carry_slice_width(bf, (int)dk, (int)dv, B * H));
    p.q = q; p.k = k; p.v = v; p.b = b; p.w = w; p.la = la;
    void* f = const_cast<void*>(fws);
    p.states = f ? (const char*)f + L.states : nullptr;
    p.wy = wy_bufs(L, f);
    p.dO = dO; p.dST = dS_T; p.dSx = const_cast<void*>(ws); p.dS0 = dS0;
    p.dq = dq; p.dk = dk_; p.dv = dv_; p.db = db; p.dw = dw; p.dla = dla;
    return p;
}

// State-gradient carry and chunk gradients of a validated backward (B, H > 0; for T = 0 only the
// pass-through of the state gradient).  Pipelined shapes run the chunk-gradient kernel of each
// chunk range on the second stream as soon as the state-gradient carry, walking the ranges
// backwards on the caller's stream, has produced that range's dS'.
static gdr2_status bwd_launch(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                              const void* q, const void* k, const void* v, const float* la,
                              const void* b, const void* w, const void* fws, const void* dO,
                              const float* dS_T, void* dq, void* dk_, void* dv_, float* dla,
                              void* db, void* dw, float* dS0, void* bws, bool allow_pipe,
                              void* stream) {
    const int bf = dt == GDR2_BF16;
    hipStream_t m = (hipStream_t)stream;
    gdr2::BwdParams pd = bwd_params(B, T, H, dk, dv, dt, nullptr, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, fws, dO, dS_T, nullptr, nullptr, nullptr,
                                    nullptr, nullptr, nullptr, dS0, bws);
    const int dvs = (int)(dv / pd.NS);
    if (T == 0)
        return gdr2::dstate_dispatch(bf, (int)dk, dvs, pd, m) == hipSuccess ? GDR2_OK : GDR2_E_HIP;
    gdr2::BwdParams pg = bwd_params(B, T, H, dk, dv, dt, q, k, v, la, b, w, fws, dO, nullptr, dq,
                                    dk_, dv_, dla, db, dw, nullptr, bws, gates);
    pg.prologue = pro != nullptr;
    pg.pro = prologue_of(pro);
    Pipe* P = (allow_pipe && pipelined(B, T, H, dk, dv, dt)) ? pipe_of_device() : nullptr;
    if (!P) {
        if (gdr2::dstate_dispatch(bf, (int)dk, dvs, pd, m) != hipSuccess) return GDR2_E_HIP;
        return gdr2::bgrad_dispatch(bf, (int)dk, (int)dv, pg, m) == hipSuccess ? GDR2_OK : GDR2_E_HIP;
    }
    std::lock_guard<std::mutex> g(P->mu);
    hipStream_t s = P->side;
    const int64_t NC = gdr2_num_chunks(T);
    const int np = pipe_pieces(B * H, NC);
    float* hand = (float*)((char*)bws + bwd_dsx_bytes(B, T, H, dk, dv, dt));
    bool ok = hipEventRecord(P->ev[0], m) == hipSuccess && hipStreamWaitEvent(s, P->ev[0], 0) == hipSuccess;
    for (int r = np - 1; ok && r >= 0; --r) {
        const int c0 = pipe_bound(NC, np, r), ncr = pipe_bound(NC, np, r + 1) - c0;
        pd.c0 = pg.c0 = c0;
        pd.ncr = pg.ncr = ncr;
        pd.dST = r == np - 1 ? dS_T : hand;  // the fp32 state gradient handed between ranges
        pd.dS0 = r == 0 ? dS0 : hand;
        ok = gdr2::dstate_dispatch(bf, (int)dk, dvs, pd, m) == hipSuccess &&
             hipEventRecord(P->ev[1 + r], m) == hipSuccess &&
             hipStreamWaitEvent(s, P->ev[1 + r], 0) == hipSuccess &&
             gdr2::bgrad_dispatch(bf, (int)dk, (int)dv, pg, s) == hipSuccess;
    }
    // the caller's stream continues once the side stream's chunk gradients are done
    if (ok) ok = hipEventRecord(P->ev[np + 1], s) == hipSuccess && hipStreamWaitEvent(m, P->ev[np + 1], 0) == hipSuccess;
    return ok ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_bwd_state(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dt, const void* fwd_workspace, size_t fwd_workspace_bytes,
                           const void* dO, const float* dS_T, float* dS0, void* workspace,
                           size_t workspace_bytes, void* stream) {
    gdr2_status st = check_bwd(B, T, H, dk, dv, dt, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, fwd_workspace, fwd_workspace_bytes, dO, dS_T, nullptr,
                               nullptr, nullptr, nullptr, nullptr, nullptr, dS0, workspace,
                               workspace_bytes, false, false);
    if (st != GDR2_OK || B == 0 || H == 0) return st;
    const int bf = dt == GDR2_BF16;
    gdr2::BwdParams p = bwd_params(B, T, H, dk, dv, dt, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, nullptr, fwd_workspace, dO, dS_T, nullptr, nullptr,
                                   nullptr, nullptr, nullptr, nullptr, dS0, workspace);
    hipError_t e = gdr2::dstate_dispatch(bf, (int)dk, (int)(dv / p.NS), p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_bwd_grads_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                              const void* q, const void* k,
                              const void* v, const float* log_alpha, const void* b, const void* w,
                              const void* fwd_workspace, size_t fwd_workspace_bytes,
                              const void* dO, void* dq, void* dk_, void* dv_, float* dlog_alpha,
                              void* db, void* dw, const void* workspace, size_t workspace_bytes,
                              void* stream) {
    gdr2_status st = check_bwd(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, fwd_workspace,
                               fwd_workspace_bytes, dO, nullptr, dq, dk_, dv_, dlog_alpha, db, dw,
                               nullptr, workspace, workspace_bytes, true, true, gates);
    if (st == GDR2_OK && !prologue_ok(pro)) st = GDR2_E_VALUE;
    if (st != GDR2_OK || B == 0 || H == 0 || T == 0) return st;
    const int bf = dt == GDR2_BF16;
    gdr2::BwdParams p = bwd_params(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, fwd_workspace,
                                   dO, nullptr, dq, dk_, dv_, dlog_alpha, db, dw, nullptr,
                                   workspace, gates);
    p.prologue = pro != nullptr;
    p.pro = prologue_of(pro);
    hipError_t e = gdr2::bgrad_dispatch(bf, (int)dk, (int)dv, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_bwd_grads(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dt, const void* q, const void* k, const void* v,
                           const float* log_alpha, const void* b, const void* w,
                           const void* fwd_workspace, size_t fwd_workspace_bytes, const void* dO,
                           void* dq, void* dk_, void* dv_, float* dlog_alpha, void* db, void* dw,
                           const void* workspace, size_t workspace_bytes, void* stream) {
    return gdr2_bwd_grads_ex(B, T, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b, w,
                             fwd_workspace, fwd_workspace_bytes, dO, dq, dk_, dv_, dlog_alpha, db,
                             dw, workspace, workspace_bytes, stream);
}

gdr2_status gdr2_bwd_chunked_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt, unsigned gates, const gdr2_prologue* pro,
                                const void* q, const void* k,
                                const void* v, const float* log_alpha, const void* b,
                                const void* w, const void* fwd_workspace,
                                size_t fwd_workspace_bytes, const void* dO, const float* dS_T,
                                void* dq, void* dk_, void* dv_, float* dlog_alpha, void* db,
                                void* dw, float* dS0, void* workspace, size_t workspace_bytes,
                                void* stream) {
    gdr2_status st = check_bwd(B, T, H, dk, dv, dt, q, k, v, log_alpha, b, w, fwd_workspace,
                               fwd_workspace_bytes, dO, dS_T, dq, dk_, dv_, dlog_alpha, db, dw,
                               dS0, workspace, workspace_bytes, true, true, gates);
    if (st == GDR2_OK && !prologue_ok(pro)) st = GDR2_E_VALUE;
    if (st != GDR2_OK || B == 0 || H == 0) return st;
    return bwd_launch(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w, fwd_workspace,
                      dO, dS_T, dq, dk_, dv_, dlog_alpha, db, dw, dS0, workspace, true, stream);
}

gdr2_status gdr2_bwd_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dt, const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const void* fwd_workspace, size_t fwd_workspace_bytes,
                             const void* dO, const float* dS_T, void* dq, void* dk_, void* dv_,
                             float* dlog_alpha, void* db, void* dw, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return gdr2_bwd_chunked_ex(B, T, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b, w,
                               fwd_workspace, fwd_workspace_bytes, dO, dS_T, dq, dk_, dv_,
                               dlog_alpha, db, dw, dS0, workspace, workspace_bytes, stream);
}

gdr2_status gdr2_bwd_chunked_recompute_ex(int64_t B, int64_t T, int64_t H, int64_t dk,
                                          int64_t dv, gdr2_dtype dt, unsigned gates,
                                          const gdr2_prologue* pro, const void* q, const void* k,
                                          const void* v, const float* log_alpha, const void* b,
                                          const void* w, const float* S0, const void* dO,
                                          const float* dS_T, void* dq, void* dk_, void* dv_,
                                          float* dlog_alpha, void* db, void* dw, float* dS0,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    gdr2_status st = check_chunked(B, T, H, dk, dv, dt);
    if (st != GDR2_OK) return st;
    if (!gates_ok(gates)) return GDR2_E_UNSUPPORTED;
    if (!prologue_ok(pro)) return GDR2_E_VALUE;
    const bool have_tokens = B > 0 && H > 0 && T > 0;
    if (have_tokens && (!q || !k || !v || !log_alpha || !b || !w || !dO)) return GDR2_E_NULL;
    if (have_tokens && (!dq || !dk_ || !dv_ || !dlog_alpha || !db || !dw)) return GDR2_E_NULL;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S0, dO, dS_T, dq, dk_, dv_, dlog_alpha, db, dw,
                          dS0, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDR2_E_ALIGN;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    const size_t need = gdr2_bwd_recompute_workspace_bytes(B, T, H, dk, dv, dt);
    if (have_tokens && (!workspace || workspace_bytes < need)) return GDR2_E_WORKSPACE;
    const size_t es = gdr2_dtype_size(dt);
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv;
    const size_t ns = (size_t)B * H * dk * dv;
    const GateSizes gs = gate_sizes(gates, (size_t)B * T * H, dk, dv);
    const Range ins[] = {{q, nk * es},      {k, nk * es},      {v, nv * es},
                         {log_alpha, gs.na * 4}, {b, gs.nb * es}, {w, gs.nw * es},
                         {S0, ns * 4},      {dO, nv * es},     {dS_T, ns * 4}};
    const Range outs[] = {{dq, nk * es},     {dk_, nk * es},    {dv_, nv * es},
                          {dlog_alpha, gs.na * 4}, {db, gs.nb * es}, {dw, gs.nw * es},
                          {dS0, ns * 4},     {workspace, have_tokens ? need : 0}};
    if (any_alias(outs, 8, ins, 9)) return GDR2_E_ALIAS;
    if (B == 0 || H == 0) return GDR2_OK;
    // the forward's factors and chunk-entry states into the first part of the workspace (o and
    // S_T are not formed), then the backward with the rest of it
    char* fws = (char*)workspace;
    char* bws = have_tokens ? fws + L.total : nullptr;
    if (T == 0) {  // nothing to recompute: the state gradient passes straight through
        return gdr2_bwd_state(B, T, H, dk, dv, dt, nullptr, 0, dO, dS_T, dS0, nullptr, 0, stream);
    }
    st = fwd_launch(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w, S0, nullptr, nullptr,
                    fws, true, true, stream);
    if (st != GDR2_OK) return st;
    return bwd_launch(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w, fws, dO, dS_T, dq,
                      dk_, dv_, dlog_alpha, db, dw, dS0, bws, true, stream);
}

gdr2_status gdr2_bwd_chunked_recompute(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                       gdr2_dtype dt, const void* q, const void* k, const void* v,
                                       const float* log_alpha, const void* b, const void* w,
                                       const float* S0, const void* dO, const float* dS_T,
                                       void* dq, void* dk_, void* dv_, float* dlog_alpha,
                                       void* db, void* dw, float* dS0, void* workspace,
                                       size_t workspace_bytes, void* stream) {
    return gdr2_bwd_chunked_recompute_ex(B, T, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b,
                                         w, S0, dO, dS_T, dq, dk_, dv_, dlog_alpha, db, dw, dS0,
                                         workspace, workspace_bytes, stream);
}

gdr2_status gdr2_decode_step_ex(int64_t N, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt,
                                unsigned gates, const gdr2_prologue* pro, const void* q,
                                const void* k, const void* v,
                                const float* log_alpha, const void* b, const void* w,
                                const float* S_in, float* S_out, void* o, void* stream) {
    if (dt != GDR2_F32 && dt != GDR2_BF16) return GDR2_E_DTYPE;
    if (N < 0 || H < 0 || dk < 0 || dv < 0) return GDR2_E_SHAPE;
    if (!dims_ok(dk) || !dims_ok(dv) || !gates_ok(gates)) return GDR2_E_UNSUPPORTED;
    if (!prologue_ok(pro)) return GDR2_E_VALUE;
    if (!prod_le(N, H, ((int64_t)1 << 31) - 1)) return GDR2_E_SHAPE;
    if (N == 0 || H == 0) return GDR2_OK;
    if (!q || !k || !v || !log_alpha || !b || !w || !S_out || !o) return GDR2_E_NULL;
    const void* ptrs[] = {q, k, v, log_alpha, b, w, S_in, S_out, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDR2_E_ALIGN;
    const size_t es = gdr2_dtype_size(dt);
    const size_t nk = (size_t)N * H * dk, nv = (size_t)N * H * dv, ns = (size_t)N * H * dk * dv;
    const GateSizes gs = gate_sizes(gates, (size_t)N * H, dk, dv);
    const Range ins[] = {{q, nk * es}, {k, nk * es}, {v, nv * es}, {log_alpha, gs.na * 4},
                         {b, gs.nb * es}, {w, gs.nw * es}};
    const Range outs[] = {{S_out, ns * 4}, {o, nv * es}};
    if (any_alias(outs, 2, ins, 6)) return GDR2_E_ALIAS;
    // S_in may be S_out exactly; any other overlap with an output is an error
    if (S_in && S_in != S_out && (overlap({S_in, ns * 4}, outs[0]) || overlap({S_in, ns * 4}, outs[1])))
        return GDR2_E_ALIAS;
    if (S_in && S_in == S_out && overlap({S_in, ns * 4}, outs[1])) return GDR2_E_ALIAS;
    gdr2::DecodeParams p;
    p.N = N; p.H = H; p.gates = (int)gates;
    p.prologue = pro != nullptr;
    p.pro = prologue_of(pro);
    p.q = q; p.k = k; p.v = v; p.b = b; p.w = w; p.la = log_alpha;
    p.S_in = S_in; p.S_out = S_out; p.o = o;
    hipError_t e = gdr2::decode_dispatch(dt == GDR2_BF16, (int)dk, (int)dv, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt,
                             const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const float* S_in, float* S_out, void* o, void* stream) {
    return gdr2_decode_step_ex(N, H, dk, dv, dt, 0u, nullptr, q, k, v, log_alpha, b, w, S_in,
                               S_out, o, stream);
}

// ------------------------------------------------------------------ output epilogue
static gdr2_status check_epi(int64_t rows, int64_t dv, gdr2_dtype dt, float eps) {
    if (dt != GDR2_F32 && dt != GDR2_BF16) return GDR2_E_DTYPE;
    // one workgroup per 128 rows, and a launch takes at most 2^31 - 1 workgroups
    if (rows < 0 || dv < 0 || rows > ((int64_t)1 << 37)) return GDR2_E_SHAPE;
    if (!dims_ok(dv)) return GDR2_E_UNSUPPORTED;
    if (!(eps > 0.f) || !(eps < 1e30f)) return GDR2_E_VALUE;
    return GDR2_OK;
}

size_t gdr2_out_gate_bwd_workspace_bytes(int64_t rows, int64_t dv) {
    if (rows <= 0 || dv <= 0) return 0;
    return (size_t)gdr2::epi_blocks(rows) * dv * sizeof(float);
}

gdr2_status gdr2_out_gate_fwd(int64_t rows, int64_t dv, gdr2_dtype dt, const void* o,
                              const void* g, const float* weight, float eps, void* y,
                              void* stream) {
    gdr2_status st = check_epi(rows, dv, dt, eps);
    if (st != GDR2_OK || rows == 0) return st;
    if (!o || !g || !weight || !y) return GDR2_E_NULL;
    const void* ptrs[] = {o, g, weight, y};
    for (const void* p : ptrs)
        if (!aligned16(p)) return GDR2_E_ALIGN;
    const size_t n = (size_t)rows * dv * gdr2_dtype_size(dt);
    const Range ins[] = {{o, n}, {g, n}, {weight, (size_t)dv * 4}};
    const Range outs[] = {{y, n}};
    if (any_alias(outs, 1, ins, 3)) return GDR2_E_ALIAS;
    gdr2::EpiParams p{};
    p.rows = rows; p.eps = eps; p.o = o; p.g = g; p.weight = weight; p.y = y;
    hipError_t e = gdr2::epi_dispatch(dt == GDR2_BF16, (int)dv, false, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

gdr2_status gdr2_out_gate_bwd(int64_t rows, int64_t dv, gdr2_dtype dt, const void* o,
                              const void* g, const float* weight, float eps, const void* dy,
                              void* do_, void* dg, float* dweight, void* workspace,
                              size_t workspace_bytes, void* stream) {
    gdr2_status st = check_epi(rows, dv, dt, eps);
    if (st != GDR2_OK) return st;
    if (!dweight) return GDR2_E_NULL;
    if (rows > 0 && (!o || !g || !weight || !dy || !do_ || !dg)) return GDR2_E_NULL;
    const void* ptrs[] = {o, g, weight, dy, do_, dg, dweight, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDR2_E_ALIGN;
    const size_t need = gdr2_out_gate_bwd_workspace_bytes(rows, dv);
    if (rows > 0 && (!workspace || workspace_bytes < need)) return GDR2_E_WORKSPACE;
    const size_t n = (size_t)rows * dv * gdr2_dtype_size(dt);
    const Range ins[] = {{o, n}, {g, n}, {weight, (size_t)dv * 4}, {dy, n}};
    const Range outs[] = {{do_, n}, {dg, n}, {dweight, (size_t)dv * 4}, {workspace, need}};
    if (any_alias(outs, 4, ins, 4)) return GDR2_E_ALIAS;
    gdr2::EpiParams p{};  // (no rows: only the weight gradient, zero, is written)
    p.rows = rows; p.eps = eps; p.o = o; p.g = g; p.weight = weight; p.dy = dy;
    p.dox = do_; p.dg = dg; p.dweight = dweight; p.dw_part = (float*)workspace;
    hipError_t e = gdr2::epi_dispatch(dt == GDR2_BF16, (int)dv, true, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
}

}  // extern "C"
