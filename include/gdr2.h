/*
 * gdr2.h -- C ABI of the MI355X (gfx950) Gated Delta Rule-2 library (libgdr2.so).
 *
 * The operation (per batch b, head h, with state S in R^{d_k x d_v}) is the Gated Delta Rule-2
 * update printed in the forum summary "Gated DeltaNet-2: Decoupling Erase and Write Gates in
 * Linear Attention for Better Memory Editing" (zhichai.net, English), section "Gated Delta Rule-2":
 *
 *     S_t = (I - k_t (b_t . k_t)^T) Diag(alpha_t) S_{t-1} + k_t (w_t . v_t)^T
 *
 * with the channel-wise decay applied before the edit, the erase gate b_t in [0,1]^{d_k} on the
 * key side and the write gate w_t in [0,1]^{d_v} on the value side (ainews.random.gg article on
 * Gated DeltaNet-2, section "Gated Delta Rule-2: two gates instead of one"), and the read-out
 * o_t = S_t^T q_t on the updated state (no query scale; callers pre-scale q if they want one).
 * The decay is passed as log(alpha_t), natural log, one value per key channel.
 *
 * Conventions shared by every entry point
 *   - Tensors are dense, row-major, and live in DEVICE memory owned by the caller.  No call
 *     allocates or frees device memory, and caller memory is never freed.  Kept between calls,
 *     per device: the second stream and its events of the long-sequence split below (created on
 *     first use) and the static scratch of gdr2_fwd_infer_noalloc_ex.  No result depends on an
 *     earlier call.
 *   - Token tensors: q, k, log_alpha, b : [B][T][H][d_k];  v, w, o, dO : [B][T][H][d_v].
 *     States: [B][H][d_k][d_v], fp32.
 *   - dtype selects the element type of q, k, v, b, w, o and of dq, dk, dv, db, dw:
 *     GDR2_BF16 (bfloat16) or GDR2_F32.  log_alpha, dlog_alpha and every state are fp32.
 *   - Every pointer must be 16-byte aligned.  Outputs must not overlap inputs or each other
 *     (decode's S_in == S_out is the one allowed, exact, alias).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).  All
 *     validation happens on the host before any launch: on any error nothing is launched and
 *     no output is written.  Launch failures return GDR2_E_HIP; faults during execution
 *     surface at the caller's next synchronisation.  No C++ exception crosses this ABI.
 *   - Results are bitwise deterministic run to run (no floating-point atomics).
 *   - Supported sizes: d_k, d_v in {64, 128}.
 *     B, H >= 1 and T >= 0 (T = 0 produces no tokens; S_T then equals S0).  Larger problems are
 *     rejected with GDR2_E_SHAPE before any size arithmetic could overflow: the chunked passes
 *     accept T <= 2^40, B*H*ceil(T/64) <= 2^30 and B*T*H <= 2^50; decode accepts N*H < 2^31.
 *   - Decay range: any finite log_alpha <= 0, i.e. any alpha in (0, 1] per channel and token (the
 *     decay is a channel-wise diagonal gate: ainews.random.gg article, section "Gated Delta
 *     Rule-2: two gates instead of one").  The chunked kernels fold the cumulative decay into
 *     factors referenced to 16-token blocks; a chunk in which some channel decays by more than
 *     exp(-60) across one block takes a second path whose factors are all <= 1, so no decay drives
 *     a factor out of the fp32 range.
 *   - Long sequences at a small batch (bf16; at most 128 state-carry workgroups, i.e. B*H <= 16 at
 *     d_v = 128; at least two ranges of 128 chunks and 512 chunk-heads): gdr2_fwd_chunked(_ex),
 *     gdr2_fwd_infer(_ex), gdr2_bwd_chunked(_ex) and gdr2_bwd_chunked_recompute(_ex) split the
 *     chunks into up to four ranges and run the chunk-parallel kernel of the later ranges on a
 *     second stream (one per device, created by the library on first use, default priority)
 *     beside the sequential state carry, joined back into `stream` with events before the call's
 *     work ends; the results are bitwise those of the unsplit phase entry points.  For these
 *     shapes the workspace queries include an fp32 B*H*d_k*d_v buffer through which the carry
 *     hands its state from range to range.  Calls that split serialise their enqueueing per
 *     device (a lock), so they may be made from several host threads.
 */
#ifndef GDR2_H
#define GDR2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDR2_ABI_VERSION 4
#define GDR2_CHUNK 64 /* tokens per chunk of the chunked passes */

typedef enum gdr2_status {
    GDR2_OK = 0,
    GDR2_E_NULL = 1,        /* a required pointer is NULL */
    GDR2_E_SHAPE = 2,       /* a size is negative, or too large for 32-bit launch indexing */
    GDR2_E_DTYPE = 3,       /* dtype is not GDR2_F32 / GDR2_BF16 */
    GDR2_E_UNSUPPORTED = 4, /* head sizes / dtype combination not built */
    GDR2_E_ALIGN = 5,       /* a pointer is not 16-byte aligned */
    GDR2_E_ALIAS = 6,       /* an output overlaps an input or another output */
    GDR2_E_WORKSPACE = 7,   /* workspace missing or smaller than the size its query returns */
    GDR2_E_HIP = 8,         /* the HIP runtime refused the launch */
    GDR2_E_VALUE = 9,       /* a scalar argument is out of range (e.g. eps <= 0) */
    GDR2_E_TOO_LARGE = 10   /* the problem exceeds the no-allocation entry point's static scratch */
} gdr2_status;

typedef enum gdr2_dtype { GDR2_F32 = 0, GDR2_BF16 = 1 } gdr2_dtype;

/*
 * Gate shapes for the *_ex entry points (bit mask; 0 = every gate channel-wise, as in the plain
 * entry points).  A set bit makes that gate one value per (batch, token, head) -- [B][T][H], or
 * [N][H] for decode -- broadcast over its channels, and makes its gradient the sum over those
 * channels, in the same [B][T][H] shape:
 *   GDR2_ERASE_SCALAR  b is a scalar per head: the ablation arm that keeps only the write gate
 *                      channel-wise (forum summary "Gated DeltaNet-2: Decoupling Erase and Write
 *                      Gates ..." on zhichai.net, section "Ablation: the erase gate matters more")
 *   GDR2_WRITE_SCALAR  w is a scalar per head: the arm of the same ablation that keeps only the
 *                      erase gate channel-wise
 *   GDR2_DECAY_SCALAR  log_alpha is a scalar per head (the scalar decay of Gated DeltaNet)
 * With b = w (both scalar) the update is KDA's; adding GDR2_DECAY_SCALAR gives Gated DeltaNet's
 * (same summary, section "Gated Delta Rule-2": the two reductions).
 */
typedef enum gdr2_gates {
    GDR2_GATES_CHANNEL = 0,
    GDR2_ERASE_SCALAR = 1,
    GDR2_WRITE_SCALAR = 2,
    GDR2_DECAY_SCALAR = 4
} gdr2_gates;

/*
 * Fused prologue for the *_ex entry points (NULL = off).  With it, q, k, log_alpha, b and w are
 * the pre-activations of the block's branches and the library applies, inside its kernels, what
 * the ainews.random.gg article on Gated DeltaNet-2 (section "Block design and hybrid model", and
 * "Gated Delta Rule-2: two gates instead of one" for the sigmoid gates) puts between the
 * projections and the mixer:
 *     q <- q / sqrt(sum_i q_i^2 + norm_eps),   k <- k / sqrt(sum_i k_i^2 + norm_eps)
 *     b <- sigmoid(b),   w <- sigmoid(w),   log_alpha <- -decay_scale * softplus(log_alpha)
 * and the backward returns dq, dk, dlog_alpha, db and dw with respect to those pre-activations
 * (v and dv are unchanged).  Both parameters must be > 0 and finite (else GDR2_E_VALUE).
 */
typedef struct gdr2_prologue {
    float decay_scale;
    float norm_eps;
} gdr2_prologue;

/* Bytes of one element of `dtype` (4 or 2), 0 for an unknown dtype. */
size_t gdr2_dtype_size(gdr2_dtype dtype);

/* Number of chunks, ceil(T / GDR2_CHUNK). */
int64_t gdr2_num_chunks(int64_t T);

/*
 * Chunked forward: o_t = S_t^T q_t for all tokens, optionally the final state.  Implements the
 * chunkwise WY form in which the cumulative channel-wise decay of a chunk is absorbed into the two
 * factors of each rank-one erase (ainews.random.gg article on Gated DeltaNet-2, section "Chunkwise
 * training and gate-aware backward"): a chunk-parallel kernel builds each chunk's WY factors, then
 * a state-carry kernel walks the chunks.
 *
 *   q, k, b         [B][T][H][dk]  dtype          (inputs)
 *   v, w            [B][T][H][dv]  dtype          (inputs)
 *   log_alpha       [B][T][H][dk]  fp32           (input, natural log of the decay)
 *   S0              [B][H][dk][dv] fp32 or NULL   (input, initial state; NULL = zero)
 *   o               [B][T][H][dv]  dtype          (output)
 *   S_T             [B][H][dk][dv] fp32 or NULL   (output, final state; NULL = not wanted)
 *   workspace       device memory of at least gdr2_fwd_workspace_bytes() bytes (required when
 *                   T > 0).  On return it holds the per-chunk WY factors and the state entering
 *                   every chunk; gdr2_bwd_chunked reads them, so keep it unchanged between the
 *                   two calls when training.
 */
gdr2_status gdr2_fwd_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dtype, const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const float* S0, void* o, float* S_T, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Bytes of device workspace gdr2_fwd_chunked needs (per token and head about
 * (4*dk + 2*64 + dv) elements of dtype plus the chunk-entry states, dk*dv/64 elements; plus the
 * fp32 hand-off buffer for the split long-sequence shapes above); 0 for sizes the chunked passes
 * reject. */
size_t gdr2_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dtype);

/*
 * Forward-only chunked forward (inference prefill, where no backward follows): o and S_T exactly
 * as gdr2_fwd_chunked computes them, bit for bit, without storing the chunk-entry states that only
 * the backward reads (dk*dv/64 elements of dtype per token and head: 512 bytes at d = 128 in
 * bf16).  Its workspace holds only the per-chunk factors -- gdr2_fwd_infer_workspace_bytes() bytes,
 * device memory, no larger than the training forward's -- and cannot be passed to
 * gdr2_bwd_chunked; gdr2_bwd_chunked_recompute is the backward that needs no forward workspace.
 * Arguments and errors as gdr2_fwd_chunked(_ex).  Decoding can continue from S_T
 * (gdr2_decode_step), constant-memory decoding after the prefill (forum summary on zhichai.net,
 * section "The Memory Dilemma").
 */
size_t gdr2_fwd_infer_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      gdr2_dtype dtype);
gdr2_status gdr2_fwd_infer(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dtype, const void* q, const void* k, const void* v,
                           const float* log_alpha, const void* b, const void* w, const float* S0,
                           void* o, float* S_T, void* workspace, size_t workspace_bytes,
                           void* stream);
gdr2_status gdr2_fwd_infer_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              gdr2_dtype dtype, unsigned gates, const gdr2_prologue* pro,
                              const void* q, const void* k, const void* v,
                              const float* log_alpha, const void* b, const void* w,
                              const float* S0, void* o, float* S_T, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of device workspace gdr2_bwd_chunked needs (the per-chunk state gradients; plus the fp32
 * hand-off buffer for the split long-sequence shapes). */
size_t gdr2_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dtype);

/*
 * Gate-aware backward (vector-Jacobian product) of gdr2_fwd_chunked for the loss
 * L = <dO, o> + <dS_T, S_T>.  The erase gate b and the write gate w enter the gradient dot
 * products themselves rather than as one scalar factor (ainews.random.gg article, section
 * "Chunkwise training and gate-aware backward").
 *
 *   q, k, v, log_alpha, b, w   as passed to gdr2_fwd_chunked (same values)
 *   fwd_workspace   the workspace of the gdr2_fwd_chunked call on these inputs, unchanged since
 *                   (it holds the WY factors and the chunk-entry states, S0 included)
 *   dO              [B][T][H][dv]  dtype           (input)
 *   dS_T            [B][H][dk][dv] fp32 or NULL    (input; NULL = zero)
 *   dq, dk_, db     [B][T][H][dk]  dtype           (outputs)
 *   dv_, dw         [B][T][H][dv]  dtype           (outputs)
 *   dlog_alpha      [B][T][H][dk]  fp32            (output)
 *   dS0             [B][H][dk][dv] fp32 or NULL    (output; NULL = not wanted)
 *   workspace       device memory of at least gdr2_bwd_workspace_bytes() bytes
 */
gdr2_status gdr2_bwd_chunked(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dtype, const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const void* fwd_workspace, size_t fwd_workspace_bytes,
                             const void* dO, const float* dS_T, void* dq, void* dk_, void* dv_,
                             float* dlog_alpha, void* db, void* dw, float* dS0,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * No-allocation variant of gdr2_fwd_infer_ex, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * per-chunk factors go to a static device array of the library instead of a workspace argument.
 * The caller still passes every input and output.  The call allocates nothing and calls no
 * allocating routine; on its first call on a device it looks up that device's copy of the array
 * (hipGetSymbolAddress) and keeps the address.
 *   - Limit: the problem's factors -- gdr2_fwd_infer_workspace_bytes(B, T, H, dk, dv, dtype), less
 *     the hand-off buffer of the split long-sequence shapes, which this entry point never splits
 *     (that would create the second stream) -- must fit gdr2_fwd_infer_noalloc_max_bytes()
 *     (128 MiB: e.g. B*H*ceil(T/64) <= 1,600 chunk-heads at d = 128 in bf16); larger problems
 *     return GDR2_E_TOO_LARGE before any launch.
 *   - Every call on one device shares that device's array, which keeps the last call's contents
 *     (each call overwrites every byte it reads, so nothing needs clearing).  Calls that overlap
 *     in time on one device -- on different streams, or from different threads without
 *     synchronisation -- race on the array; order them on one stream.
 *   - Each device the library runs on holds its array (128 MiB) until the process ends.
 * Arguments, results (bit for bit) and every other error as gdr2_fwd_infer_ex.
 */
size_t gdr2_fwd_infer_noalloc_max_bytes(void);
gdr2_status gdr2_fwd_infer_noalloc_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                      gdr2_dtype dtype, unsigned gates, const gdr2_prologue* pro,
                                      const void* q, const void* k, const void* v,
                                      const float* log_alpha, const void* b, const void* w,
                                      const float* S0, void* o, float* S_T, void* stream);

/*
 * Gate-aware backward that needs no forward workspace: it recomputes the per-chunk factors and
 * the chunk-entry states from the inputs and S0 (the chunked forward without o), then runs the
 * backward of gdr2_bwd_chunked; the gradients equal gdr2_bwd_chunked's bit for bit.  For callers
 * that ran gdr2_fwd_infer, or that do not keep the forward workspace between the passes.
 *   S0              [B][H][dk][dv] fp32 or NULL (= 0): the initial state the forward used
 *   workspace       device memory of at least gdr2_bwd_recompute_workspace_bytes() bytes (the
 *                   training forward's workspace followed by the backward's)
 * Every other argument and every error as in gdr2_bwd_chunked(_ex).
 */
size_t gdr2_bwd_recompute_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                          gdr2_dtype dtype);
gdr2_status gdr2_bwd_chunked_recompute(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                       gdr2_dtype dtype, const void* q, const void* k,
                                       const void* v, const float* log_alpha, const void* b,
                                       const void* w, const float* S0, const void* dO,
                                       const float* dS_T, void* dq, void* dk_, void* dv_,
                                       float* dlog_alpha, void* db, void* dw, float* dS0,
                                       void* workspace, size_t workspace_bytes, void* stream);
gdr2_status gdr2_bwd_chunked_recompute_ex(int64_t B, int64_t T, int64_t H, int64_t dk,
                                          int64_t dv, gdr2_dtype dtype, unsigned gates,
                                          const gdr2_prologue* pro, const void* q, const void* k,
                                          const void* v, const float* log_alpha, const void* b,
                                          const void* w, const float* S0, const void* dO,
                                          const float* dS_T, void* dq, void* dk_, void* dv_,
                                          float* dlog_alpha, void* db, void* dw, float* dS0,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Phase entry points.  gdr2_fwd_chunked is gdr2_fwd_factors followed by gdr2_fwd_carry on the same
 * stream, gdr2_bwd_chunked is gdr2_bwd_state followed by gdr2_bwd_grads; the arguments mean the
 * same as there.  They exist so that callers can time, overlap or reuse the stages.
 *   gdr2_fwd_factors  chunk-parallel: writes each chunk's WY factors into `workspace`
 *   gdr2_fwd_carry    sequential over chunks: o, S_T and the chunk-entry states from the factors
 *   gdr2_bwd_state    sequential over chunks in reverse: the state gradient entering every
 *                     chunk's exit (kept in `workspace`) and dS0
 *   gdr2_bwd_grads    chunk-parallel: dq, dk, dv, dlog_alpha, db, dw from both workspaces
 */
gdr2_status gdr2_fwd_factors(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                             gdr2_dtype dtype, const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             void* workspace, size_t workspace_bytes, void* stream);
gdr2_status gdr2_fwd_carry(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dtype, const float* S0, void* o, float* S_T,
                           void* workspace, size_t workspace_bytes, void* stream);
gdr2_status gdr2_bwd_state(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dtype, const void* fwd_workspace, size_t fwd_workspace_bytes,
                           const void* dO, const float* dS_T, float* dS0, void* workspace,
                           size_t workspace_bytes, void* stream);
gdr2_status gdr2_bwd_grads(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                           gdr2_dtype dtype, const void* q, const void* k, const void* v,
                           const float* log_alpha, const void* b, const void* w,
                           const void* fwd_workspace, size_t fwd_workspace_bytes, const void* dO,
                           void* dq, void* dk_, void* dv_, float* dlog_alpha, void* db, void* dw,
                           const void* workspace, size_t workspace_bytes, void* stream);

/*
 * One recurrent token for N independent sequences x H heads (constant-memory decoding; forum
 * summary, section "The Memory Dilemma").  The state stays in HBM and is updated in place when
 * S_in == S_out.
 *
 *   q, k, b         [N][H][dk]  dtype
 *   v, w            [N][H][dv]  dtype
 *   log_alpha       [N][H][dk]  fp32
 *   S_in            [N][H][dk][dv] fp32 or NULL (= zero state); may equal S_out
 *   S_out           [N][H][dk][dv] fp32 (required)
 *   o               [N][H][dv]  dtype (output)
 */
gdr2_status gdr2_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dtype,
                             const void* q, const void* k, const void* v,
                             const float* log_alpha, const void* b, const void* w,
                             const float* S_in, float* S_out, void* o, void* stream);

/*
 * The same entry points with the gate shapes of `gates` (a gdr2_gates bit mask; any other bit
 * returns GDR2_E_UNSUPPORTED) and the optional fused prologue `pro` (NULL = off).  Every argument
 * means what it means in the plain entry point, except that b / w / log_alpha and their gradients
 * db / dw / dlog_alpha have the [B][T][H] ([N][H] for decode) shape when their bit is set, and
 * that with `pro` the inputs and their gradients are pre-activations.  With gates = 0 and
 * pro = NULL each equals the plain call.
 */
gdr2_status gdr2_fwd_chunked_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dtype, unsigned gates, const gdr2_prologue* pro,
                                const void* q, const void* k,
                                const void* v, const float* log_alpha, const void* b,
                                const void* w, const float* S0, void* o, float* S_T,
                                void* workspace, size_t workspace_bytes, void* stream);
gdr2_status gdr2_bwd_chunked_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dtype, unsigned gates, const gdr2_prologue* pro,
                                const void* q, const void* k,
                                const void* v, const float* log_alpha, const void* b,
                                const void* w, const void* fwd_workspace,
                                size_t fwd_workspace_bytes, const void* dO, const float* dS_T,
                                void* dq, void* dk_, void* dv_, float* dlog_alpha, void* db,
                                void* dw, float* dS0, void* workspace, size_t workspace_bytes,
                                void* stream);
gdr2_status gdr2_fwd_factors_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                                gdr2_dtype dtype, unsigned gates, const gdr2_prologue* pro,
                                const void* q, const void* k,
                                const void* v, const float* log_alpha, const void* b,
                                const void* w, void* workspace, size_t workspace_bytes,
                                void* stream);
gdr2_status gdr2_bwd_grads_ex(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv,
                              gdr2_dtype dtype, unsigned gates, const gdr2_prologue* pro,
                              const void* q, const void* k,
                              const void* v, const float* log_alpha, const void* b, const void* w,
                              const void* fwd_workspace, size_t fwd_workspace_bytes,
                              const void* dO, void* dq, void* dk_, void* dv_, float* dlog_alpha,
                              void* db, void* dw, const void* workspace, size_t workspace_bytes,
                              void* stream);
gdr2_status gdr2_decode_step_ex(int64_t N, int64_t H, int64_t dk, int64_t dv, gdr2_dtype dtype,
                                unsigned gates, const gdr2_prologue* pro, const void* q,
                                const void* k, const void* v,
                                const float* log_alpha, const void* b, const void* w,
                                const float* S_in, float* S_out, void* o, void* stream);

/*
 * Output epilogue of the block (ainews.random.gg article on Gated DeltaNet-2, section "Block design
 * and hybrid model": the mixer output is RMS-normalised and multiplied by a SiLU output gate before
 * the output projection).  For every row (one token of one head; rows = B*T*H) of dv channels:
 *     y_j = o_j / sqrt(mean_i o_i^2 + eps) * weight_j * silu(g_j),   silu(x) = x / (1 + exp(-x))
 * with one weight vector shared by all heads.
 *   o, g, y         [rows][dv]  dtype       (o: the mixer output, g: gate pre-activation; y: output)
 *   weight          [dv]        fp32
 *   eps             > 0, finite (else GDR2_E_VALUE)
 * The backward takes dy [rows][dv] and writes do_, dg [rows][dv] (dtype) and dweight [dv] (fp32,
 * the sum over all rows, reduced in a fixed order: bitwise deterministic); it needs a workspace
 * of gdr2_out_gate_bwd_workspace_bytes(rows, dv) bytes.  dv in {64, 128}; rows <= 2^37
 * (GDR2_E_SHAPE above).
 */
gdr2_status gdr2_out_gate_fwd(int64_t rows, int64_t dv, gdr2_dtype dtype, const void* o,
                              const void* g, const float* weight, float eps, void* y,
                              void* stream);
size_t gdr2_out_gate_bwd_workspace_bytes(int64_t rows, int64_t dv);
gdr2_status gdr2_out_gate_bwd(int64_t rows, int64_t dv, gdr2_dtype dtype, const void* o,
                              const void* g, const float* weight, float eps, const void* dy,
                              void* do_, void* dg, float* dweight, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Static description of a status code. */
const char* gdr2_status_string(gdr2_status s);

/* GDR2_ABI_VERSION of the loaded library. */
int gdr2_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDR2_H */
