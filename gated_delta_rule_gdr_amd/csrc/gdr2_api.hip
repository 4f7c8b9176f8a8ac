// gdr2_api.hip -- the C ABI declared in include/gdr2.h: host-side validation, then kernel launch.
// Nothing here touches device memory before every check has passed.
#include "gdr2.h"

#include <hip/hip_runtime.h>

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
    }
    return "unknown status";
}

int gdr2_abi_version(void) { return GDR2_ABI_VERSION; }

// Layout of the forward workspace: per-chunk WY factors, then the chunk-entry states.
struct FwdWs {
    size_t yh, qg, kt, p, tm, u, gam, states, total;
};
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
    w.total = off;
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

size_t gdr2_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0 || gdr2_dtype_size(dt) == 0) return 0;
    return fwd_ws_layout(B, T, H, dk, dv, dt).total;
}

size_t gdr2_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dt) {
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0 || gdr2_dtype_size(dt) == 0) return 0;
    return round_up((size_t)B * H * gdr2_num_chunks(T) * dk * dv * gdr2_dtype_size(dt), 256);
}

// Shared shape / dtype checks of the two chunked passes.
static gdr2_status check_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                 gdr2_dtype dt) {
    if (dt != GDR2_F32 && dt != GDR2_BF16) return GDR2_E_DTYPE;
    if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return GDR2_E_SHAPE;
    if (!dims_ok(dk) || !dims_ok(dv)) return GDR2_E_UNSUPPORTED;
    if (B * H * (dv / 16) > (int64_t)1 << 30) return GDR2_E_SHAPE;
    if (B * H * gdr2_num_chunks(T) > (int64_t)1 << 30) return GDR2_E_SHAPE;
    if (T > ((int64_t)1 << 40) || B * T * H > ((int64_t)1 << 50)) return GDR2_E_SHAPE;
    return GDR2_OK;
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
    p.T = T;
    p.DV = dv;
    p.q = q; p.k = k; p.v = v; p.b = b; p.w = w;
    p.la = la;
    p.S0 = S0;
    p.o = o;
    p.ST = S_T;
    p.states = ws ? (char*)ws + L.states : nullptr;
    p.wy = wy_bufs(L, ws);
    return p;
}

// Validation shared by the forward phases.  `need_inputs` / `need_out` select which pointers a
// phase requires; every pointer given must be aligned and every output disjoint from the inputs.
static gdr2_status check_fwd(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dt, const void* q, const void* k, const void* v,
                             const float* la, const void* b, const void* w, const float* S0,
                             void* o, float* S_T, void* ws, size_t ws_bytes, bool need_inputs,
                             bool need_out, unsigned gates = 0) {
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
    if (have_tokens && (!ws || ws_bytes < L.total)) return GDR2_E_WORKSPACE;
    const size_t es = gdr2_dtype_size(dt);
    const size_t nk = (size_t)B * T * H * dk, nv = (size_t)B * T * H * dv;
    const size_t ns = (size_t)B * H * dk * dv;
    const GateSizes gs = gate_sizes(gates, (size_t)B * T * H, dk, dv);
    const Range ins[] = {{q, nk * es}, {k, nk * es}, {v, nv * es}, {la, gs.na * 4},
                         {b, gs.nb * es}, {w, gs.nw * es}, {S0, ns * 4}};
    const Range outs[] = {{o, nv * es}, {S_T, ns * 4}, {ws, have_tokens ? L.total : 0}};
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

gdr2_status gdr2_fwd_carry(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dt, const float* S0, void* o, float* S_T, void* workspace,
                           size_t workspace_bytes, void* stream) {
    gdr2_status st = check_fwd(B, T, H, dk, dv, dt, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, S0, o, S_T, workspace, workspace_bytes, false, true);
    if (st != GDR2_OK || B == 0 || H == 0) return st;
    const int bf = dt == GDR2_BF16;
    const FwdWs L = fwd_ws_layout(B, T, H, dk, dv, dt);
    const int dvs = gdr2::carry_slice_width(bf, (int)dk, (int)dv, B * H);
    gdr2::FwdParams p = fwd_params(B, T, H, dv, nullptr, nullptr, nullptr, nullptr, nullptr,
                                   nullptr, S0, o, S_T, L, T > 0 ? workspace : nullptr, dvs);
    hipError_t e = gdr2::carry_fwd_dispatch(bf, (int)dk, dvs, p, (hipStream_t)stream);
    return e == hipSuccess ? GDR2_OK : GDR2_E_HIP;
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
    if (T > 0) {
        st = gdr2_fwd_factors_ex(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w,
                                 workspace, workspace_bytes, stream);
        if (st != GDR2_OK) return st;
    }
    return gdr2_fwd_carry(B, T, H, dk, dv, dt, S0, o, S_T, workspace, workspace_bytes, stream);
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
    p.NS = (int)(dv / gdr2::carry_slice_width(bf, (int)dk, (int)dv, B * H));
    p.q = q; p.k = k; p.v = v; p.b = b; p.w = w; p.la = la;
    void* f = const_cast<void*>(fws);
    p.states = f ? (const char*)f + L.states : nullptr;
    p.wy = wy_bufs(L, f);
    p.dO = dO; p.dST = dS_T; p.dSx = const_cast<void*>(ws); p.dS0 = dS0;
    p.dq = dq; p.dk = dk_; p.dv = dv_; p.db = db; p.dw = dw; p.dla = dla;
    return p;
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
    st = gdr2_bwd_state(B, T, H, dk, dv, dt, fwd_workspace, fwd_workspace_bytes, dO, dS_T, dS0,
                        workspace, workspace_bytes, stream);
    if (st != GDR2_OK || T == 0) return st;
    return gdr2_bwd_grads_ex(B, T, H, dk, dv, dt, gates, pro, q, k, v, log_alpha, b, w,
                             fwd_workspace, fwd_workspace_bytes, dO, dq, dk_, dv_, dlog_alpha, db,
                             dw, workspace, workspace_bytes, stream);
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

gdr2_status gdr2_decode_step_ex(int64_t N, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dt,
                                unsigned gates, const gdr2_prologue* pro, const void* q,
                                const void* k, const void* v,
                                const float* log_alpha, const void* b, const void* w,
                                const float* S_in, float* S_out, void* o, void* stream) {
    if (dt != GDR2_F32 && dt != GDR2_BF16) return GDR2_E_DTYPE;
    if (N < 0 || H < 0 || dk < 0 || dv < 0) return GDR2_E_SHAPE;
    if (!dims_ok(dk) || !dims_ok(dv) || !gates_ok(gates)) return GDR2_E_UNSUPPORTED;
    if (!prologue_ok(pro)) return GDR2_E_VALUE;
    if (N * H > ((int64_t)1 << 31) - 1) return GDR2_E_SHAPE;
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
