/* Host driver for the fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * Calls every entry point of oracle/gdr2_oracle.c on small seeded inputs -- ragged token counts
 * around the checkpoint length, odd head sizes, with and without S0 and dS_T -- and checks what
 * holds by construction: every output is finite, T one-token decode steps reproduce the forward
 * exactly (both run the same token step), and the KDA rule with beta = b = w matches GDR-2. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void gdr2o_forward(long B, long T, long H, long dk, long dv, const double* q, const double* k,
                   const double* v, const double* la, const double* b, const double* w,
                   const double* S0, double* o, double* ST);
void gdr2o_backward(long B, long T, long H, long dk, long dv, const double* q, const double* k,
                    const double* v, const double* la, const double* b, const double* w,
                    const double* S0, const double* dO, const double* dST, double* dq, double* dk_,
                    double* dv_, double* dla, double* db, double* dw, double* dS0);
void gdr2o_decode_step(long N, long H, long dk, long dv, const double* q, const double* k,
                       const double* v, const double* la, const double* b, const double* w,
                       const double* S_in, double* S_out, double* o);
void gdr2o_kda_forward(long B, long T, long H, long dk, long dv, int scalar_decay, const double* q,
                       const double* k, const double* v, const double* la, const double* beta,
                       const double* S0, double* o, double* ST);

static unsigned long long g_state = 88172645463325252ull;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
    g_state ^= g_state << 13;
    g_state ^= g_state >> 7;
    g_state ^= g_state << 17;
    return (double)(g_state >> 11) / 9007199254740992.0;
}
static double* arr(size_t n, double lo, double hi) {
    double* x = (double*)malloc(sizeof(double) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) x[i] = lo + (hi - lo) * urand();
    return x;
}
static int finite_all(const double* x, size_t n) {
    for (size_t i = 0; i < n; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

static int g_fail = 0;
#define CHECK(c)                                                     \
    do {                                                             \
        if (!(c)) {                                                  \
            printf("FAIL line %d: %s\n", __LINE__, #c);              \
            ++g_fail;                                                \
        }                                                            \
    } while (0)

static void run_case(long B, long T, long H, long dk, long dv, int with_s0, int with_dst) {
    const size_t nk = (size_t)(B * T * H * dk), nv = (size_t)(B * T * H * dv), ns = (size_t)(B * H * dk * dv);
    double *q = arr(nk, -1, 1), *k = arr(nk, -1, 1), *v = arr(nv, -1, 1), *la = arr(nk, -3, 0);
    double *b = arr(nk, 0, 1), *w = arr(nv, 0, 1), *dO = arr(nv, -1, 1);
    double *S0 = with_s0 ? arr(ns, -0.1, 0.1) : NULL, *dST = with_dst ? arr(ns, -1, 1) : NULL;
    double *o = arr(nv, 0, 0), *ST = arr(ns, 0, 0);
    gdr2o_forward(B, T, H, dk, dv, q, k, v, la, b, w, S0, o, ST);
    CHECK(finite_all(o, nv) && finite_all(ST, ns));
    double *dq = arr(nk, 0, 0), *dk_ = arr(nk, 0, 0), *dv_ = arr(nv, 0, 0), *dla = arr(nk, 0, 0);
    double *db = arr(nk, 0, 0), *dw = arr(nv, 0, 0), *dS0 = arr(ns, 0, 0);
    gdr2o_backward(B, T, H, dk, dv, q, k, v, la, b, w, S0, dO, dST, dq, dk_, dv_, dla, db, dw, dS0);
    CHECK(finite_all(dq, nk) && finite_all(dk_, nk) && finite_all(dv_, nv) && finite_all(dla, nk));
    CHECK(finite_all(db, nk) && finite_all(dw, nv) && finite_all(dS0, ns));
    /* T decode steps from S0 over the same tokens: identical outputs and final state */
    double *S = arr(ns, 0, 0), *ot = arr((size_t)(B * H * dv), 0, 0);
    double *qt = arr((size_t)(B * H * dk), 0, 0), *kt = arr((size_t)(B * H * dk), 0, 0);
    double *lt = arr((size_t)(B * H * dk), 0, 0), *bt = arr((size_t)(B * H * dk), 0, 0);
    double *vt = arr((size_t)(B * H * dv), 0, 0), *wt = arr((size_t)(B * H * dv), 0, 0);
    if (S0) memcpy(S, S0, sizeof(double) * ns);
    int same = 1;
    for (long t = 0; t < T; ++t) {
        for (long bb = 0; bb < B; ++bb)
            for (long h = 0; h < H; ++h) {
                const size_t src_k = (size_t)(((bb * T + t) * H + h) * dk), dst_k = (size_t)((bb * H + h) * dk);
                const size_t src_v = (size_t)(((bb * T + t) * H + h) * dv), dst_v = (size_t)((bb * H + h) * dv);
                memcpy(qt + dst_k, q + src_k, sizeof(double) * dk);
                memcpy(kt + dst_k, k + src_k, sizeof(double) * dk);
                memcpy(lt + dst_k, la + src_k, sizeof(double) * dk);
                memcpy(bt + dst_k, b + src_k, sizeof(double) * dk);
                memcpy(vt + dst_v, v + src_v, sizeof(double) * dv);
                memcpy(wt + dst_v, w + src_v, sizeof(double) * dv);
            }
        gdr2o_decode_step(B, H, dk, dv, qt, kt, vt, lt, bt, wt, (t == 0 && !S0) ? NULL : S, S, ot);
        for (long bb = 0; bb < B; ++bb)
            for (long h = 0; h < H; ++h)
                if (memcmp(ot + (bb * H + h) * dv, o + ((bb * T + t) * H + h) * dv, sizeof(double) * dv)) same = 0;
    }
    if (T > 0) CHECK(same && memcmp(S, ST, sizeof(double) * ns) == 0);
    /* KDA with beta: GDR-2 with b = w = beta broadcast (same recurrence, independent code) */
    double* beta = arr((size_t)(B * T * H), 0, 1);
    for (size_t i = 0; i < (size_t)(B * T * H); ++i) {
        for (long c = 0; c < dk; ++c) b[i * dk + c] = beta[i];
        for (long c = 0; c < dv; ++c) w[i * dv + c] = beta[i];
    }
    double *o2 = arr(nv, 0, 0), *ST2 = arr(ns, 0, 0), *o3 = arr(nv, 0, 0), *ST3 = arr(ns, 0, 0);
    gdr2o_forward(B, T, H, dk, dv, q, k, v, la, b, w, S0, o2, ST2);
    gdr2o_kda_forward(B, T, H, dk, dv, 0, q, k, v, la, beta, S0, o3, ST3);
    double err = 0, mag = 0;
    for (size_t i = 0; i < nv; ++i) { err = fmax(err, fabs(o2[i] - o3[i])); mag = fmax(mag, fabs(o2[i])); }
    CHECK(err <= 1e-12 * (mag + 1));
    gdr2o_kda_forward(B, T, H, dk, dv, 1, q, k, v, la, beta, NULL, o3, NULL);
    CHECK(finite_all(o3, nv));
    free(q); free(k); free(v); free(la); free(b); free(w); free(dO); free(S0); free(dST); free(o); free(ST);
    free(dq); free(dk_); free(dv_); free(dla); free(db); free(dw); free(dS0); free(S); free(ot);
    free(qt); free(kt); free(lt); free(bt); free(vt); free(wt); free(beta); free(o2); free(ST2); free(o3); free(ST3);
}

int main(void) {
    const long Ts[] = {0, 1, 5, 63, 64, 65, 130};
    for (int i = 0; i < 7; ++i) {
        run_case(2, Ts[i], 2, 3, 2, i & 1, (i >> 1) & 1);
        run_case(1, Ts[i], 3, 4, 5, !(i & 1), 1);
    }
    run_case(1, 70, 1, 16, 8, 1, 1);
    printf("%s: %d failures\n", g_fail ? "FAIL" : "ok", g_fail);
    return g_fail ? 1 : 0;
}
