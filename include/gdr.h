/*
 * gdr.h -- C ABI of the MI355X (gfx950) gated delta-rule operator library
 * (libgdr.so).
 *
 * The operator (KDA blog "线性注意力架构演进与Kimi Delta Attention创新实践",
 * section 2.1, with "=" and "+" restored where the page's extraction lost them):
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t
 *
 * S is a dk x dv matrix per (sequence, head); the read-out uses the state after
 * the token's write.  One family, three gate kinds (linear-attention comparison
 * explainer "线性注意力架构：机制、权衡与跨层路由", core method 1):
 *   GDR_GATE_NONE     DeltaNet             alpha == 1
 *   GDR_GATE_SCALAR   Gated DeltaNet       one alpha per token and head
 *   GDR_GATE_CHANNEL  Kimi Delta Attention one alpha per token, head, key channel
 * The normaliser Z_t of the explainer's unified notation is 1 for this family.
 *
 * Optional Cross-Layer Value Routing (CLVR) epilogue (explainer, cross-layer
 * routing section; abstract on the paper page): the layer's written value v_t
 * is added into the aligned hidden (residual) stream, with a per-channel scale
 * lam standing in for the paper's zero-initialised routing projection:
 *     h[b,t,h*dv+j] += lam[h*dv+j] * v[b,t,h,j]
 * or, with desc->route == GDR_ROUTE_ERROR, the error-routing variant CLER-H
 * (popular article on the study, cross-layer section), which adds the write
 * error of the delta rule instead of the value:
 *     h[b,t,h*dv+j] += lam[h*dv+j] * e[b,t,h,j],
 *     e_t = v_t - (Diag(alpha_t) S_{t-1})^T k_t      (so that u_t = beta_t e_t
 *                                                     is what the step writes)
 * The chunked kernels obtain e_t as u_t / beta_t, so CLER-H requires every
 * beta != 0 (beta in (0, 1], the sigmoid range the pages use); beta == 0 gives
 * Inf/NaN in h and in the gradients (rejected in the debug mode below).
 *
 * Conventions shared by every entry point
 *   - Every function is extern "C", never throws, never aborts, and never
 *     allocates device memory.  The caller owns every buffer.
 *   - Pointers are device pointers unless stated otherwise, and must be
 *     16-byte aligned.  All tensors are dense row-major:
 *       q, k        [B, T, H, dk]          v, o   [B, T, H, dv]
 *       beta        [B, T, H]    fp32
 *       alpha       NONE: NULL; SCALAR: [B, T, H] fp32; CHANNEL: [B, T, H, dk]
 *                   fp32; every value in (0, 1] (the chunked kernels work with
 *                   log2(alpha); alpha == 0 is outside the domain); logits
 *                   with a prologue (gdr_prologue)
 *       S0, ST      [B, H, dk, dv] fp32
 *       h_clvr      [B, T, H*dv] in the input dtype
 *       clvr_scale  [H*dv] fp32
 *   - v1 supports dk == dv in {64, 128} and chunk size 64.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream) and
 *     the call returns at once.  Host-side validation runs before any launch;
 *     on a non-OK status nothing has been launched and no output was touched.
 *     A launch failure returns GDR_ERR_DEVICE; asynchronous device faults
 *     surface at the caller's next synchronisation.
 *   - Precision: fp32 state and fp32 accumulation throughout.  For bf16 inputs
 *     the matrix-core operands of the chunked path are rounded to fp16 (one
 *     pass), and so are the chunk-start states and state gradients the
 *     backward keeps.  Every such value must stay below 65504 in magnitude:
 *     q, k, v, S0, dO, dST, dh themselves, and what grows from them -- the
 *     state (about |v| times a few for unit-norm keys) and the state gradient
 *     (a sum of scale * q do^T over the decay horizon).  Measured on MI355X
 *     at d = 128 with unit-norm q, k: v scaled to N(0, 1000^2) and dO scaled
 *     by 256 (a loss scale) at T = 2048 without decay stay within the 2e-3
 *     bar; a larger loss scale on long sequences without decay can overflow
 *     the fp16 state-gradient snapshots (Inf in the gradients).  Unscale the
 *     loss scale into dO beforehand, or use fp32 inputs, whose operands stay
 *     fp32.
 *   - NaN and Inf propagate; in the normal mode no input is checked.
 *   - Debug mode: with the environment variable GDR_VALIDATE=1 (read at every
 *     call) each entry point, after its host checks, checks its inputs on the
 *     device and synchronises `stream` to read the result; a violation
 *     returns GDR_ERR_INVALID_ARG, names the tensor and the first offending
 *     element in gdr_last_error(), and launches nothing else, so every output
 *     is untouched.  Rules: every float input finite; alpha in (0, 1] for
 *     the chunked calls (with a prologue: finite logits) and in [0, 1] for the
 *     decode step; beta != 0 on the error route (without a prologue); for
 *     bf16 inputs, |x| < 65504 for q, k (without a prologue), v, S0, dO, dST
 *     and dh.  Valid inputs give the same results bit for bit as the normal
 *     mode.  The check cannot run under stream capture (it synchronises):
 *     there it returns GDR_ERR_INVALID_ARG.  Concurrent validated calls on one
 *     device are serialised by a lock.
 */
#ifndef GDR_H
#define GDR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID_ARG = 1, /* NULL/misaligned pointer, bad size, bad enum, aliasing */
    GDR_ERR_UNSUPPORTED = 2, /* a valid request this version does not implement */
    GDR_ERR_WORKSPACE = 3,   /* ws_bytes below gdr_workspace_size() or ws NULL */
    GDR_ERR_DEVICE = 4       /* the HIP runtime reported an error at launch */
} gdr_status;

typedef enum { GDR_GATE_NONE = 0, GDR_GATE_SCALAR = 1, GDR_GATE_CHANNEL = 2 } gdr_gate;

typedef enum { GDR_BF16 = 0, GDR_FP32 = 1 } gdr_dtype;

/* What the hidden-stream epilogue (h_clvr) adds per token: the written value
 * v_t (CLVR) or the write error e_t (CLER-H). */
typedef enum { GDR_ROUTE_VALUE = 0, GDR_ROUTE_ERROR = 1 } gdr_route;

/* Fused prologue of the chunked calls (KDA blog sections 2.1 and 7.1: q and k
 * are L2-normalised after their projections; the gates come out of sigmoids,
 * the forget gate's logit biased to -3 so that it forgets ~5 % per token at
 * initialisation).  With a prologue, q and k are passed unnormalised and beta
 * and alpha as logits b and a; the operator uses
 *     q_hat = q / max(|q|_2, 1e-6)   (per token and head; k likewise)
 *     beta  = sigmoid(b)
 *     alpha = sigmoid(a)                       GDR_PROLOGUE_ALPHA_SIGMOID
 *     alpha = exp(-softplus(a)) = 1 - sigmoid(a)   GDR_PROLOGUE_ALPHA_FORGET
 * and the backward returns dq, dk, dbeta, dalpha with respect to the raw
 * q, k and the logits.  Any finite logit is in the domain.  The decode step
 * takes activated inputs. */
typedef enum {
    GDR_PROLOGUE_NONE = 0,
    GDR_PROLOGUE_ALPHA_SIGMOID = 1,
    GDR_PROLOGUE_ALPHA_FORGET = 2
} gdr_prologue;

typedef struct {
    int64_t B, T, H, dk, dv; /* batch, tokens, heads, key and value widths */
    int32_t gate;            /* gdr_gate */
    int32_t in_dtype;        /* gdr_dtype of q, k, v, dO and h_clvr */
    int32_t out_dtype;       /* gdr_dtype of o, dq, dk, dv */
    float scale;             /* o = scale * S^T q ; 1.0 is the pages' equation */
    int32_t chunk;           /* 0 selects the default (64); only 64 is supported */
    int32_t route;           /* gdr_route of the h_clvr epilogue; 0 (VALUE) when unused */
    int32_t prologue;        /* gdr_prologue; 0 (NONE): q, k, beta, alpha used as passed */
} gdr_desc;

/* Bytes of device workspace the chunked calls need for `desc`.
 * op = 0: gdr_forward_chunked, op = 1: gdr_backward.  Returns 0 for an invalid
 * descriptor (gdr_last_error() then says why).  Host function, no GPU access. */
size_t gdr_workspace_size(const gdr_desc* desc, int op);

/* Chunked forward over B sequences of T tokens.
 *
 * The sequence is cut into chunks of 64 tokens (the chunkwise recurrent form of
 * the KDA blog, section 6.1: every chunk carries its own start state).  Inside a
 * chunk the rank-1 updates are gathered into one triangular solve and dense
 * matrix-core products (the "UT transform" the blog's section 6.2 names), with
 * the cumulative decay kept in log space (section 7.1); the chunks are then
 * chained by a sequential state pass.
 *
 *   S0        initial state, NULL = zeros.  ST final state, NULL = not written;
 *             ST may alias S0.
 *   o         [B,T,H,dv] in out_dtype; must not alias an input.
 *   h_clvr    NULL = no epilogue; else updated in place (in_dtype) with
 *             lam * v (route VALUE) or lam * e (route ERROR).
 *   clvr_scale NULL = lam == 1.
 *   ws        device workspace of at least gdr_workspace_size(desc, 0) bytes;
 *             its contents on entry do not matter.
 */
gdr_status gdr_forward_chunked(const gdr_desc* desc, const void* q, const void* k,
                               const void* v, const float* beta, const float* alpha,
                               const float* S0, void* o, float* ST, void* h_clvr,
                               const float* clvr_scale, void* ws, size_t ws_bytes,
                               void* stream);

/* gdr_forward_chunked with the output-gate epilogue of KDA blog section 4.1
 * applied to o before it leaves the chip (the inference form of
 * gdr_forward_chunked followed by gdr_output_gate_forward on its o):
 *     y = sigmoid(g) * w * o / sqrt(mean_j o_j^2 + 1e-6)      (j over dv)
 *   g   [B,T,H,dv] in_dtype, the caller's low-rank projection output (required)
 *   w   [H*dv] fp32 norm weight, NULL = ones
 *   y   [B,T,H,dv] out_dtype, written in place of o (o itself is not kept); it
 *       must not overlap any input
 * Every other argument, the workspace size (gdr_workspace_size(desc, 0)) and
 * the error behaviour are those of gdr_forward_chunked; in the debug mode g and
 * w are checked to be finite.  y equals the two separate calls bit for bit.
 * bf16 inputs: the output kernel normalises and gates the rows it assembles on
 * chip, so o is neither written nor read back.  fp32 inputs: the state pass
 * writes o into y and the gate runs over y in place. */
gdr_status gdr_forward_chunked_gated(const gdr_desc* desc, const void* q, const void* k,
                                     const void* v, const float* beta, const float* alpha,
                                     const float* S0, const void* g, const float* w, void* y,
                                     float* ST, void* h_clvr, const float* clvr_scale, void* ws,
                                     size_t ws_bytes, void* stream);

/* Gradients of gdr_forward_chunked (reverse mode, chunked, recomputing the
 * forward's intermediates):
 *   dO        [B,T,H,dv] in_dtype, upstream gradient of o.
 *   dST       NULL = zero gradient on the final state.
 *   dh_clvr   NULL = no epilogue term; else [B,T,H*dv] in_dtype, the gradient
 *             arriving at the hidden stream after the epilogue's add (for
 *             route ERROR it reaches every input through e_t).
 *   dq, dk    [B,T,H,dk], dv [B,T,H,dv] in out_dtype.
 *   dbeta     [B,T,H] fp32.
 *   dalpha    alpha's shape, fp32, derivative w.r.t. alpha itself; must be NULL
 *             iff the gate is NONE.  The kernels form the gradient with
 *             respect to ln(alpha) (the decay enters through its cumulative
 *             logarithm) and divide by alpha: alpha * dalpha is held to the
 *             same relative bar as every other output, and the absolute error
 *             of dalpha grows like 1 / alpha where alpha is small (measured
 *             raw relative errors are listed with the parity results).
 *   dS0       [B,H,dk,dv] fp32, NULL = not written.
 *   dclvr_scale [H*dv] fp32, NULL = not written (requires dh_clvr).
 *   ws        at least gdr_workspace_size(desc, 1) bytes.
 * fp32 inputs at dk = dv = 128 run the two gradient stages as two kernels
 * (neither fits one workgroup's LDS with fp32 operands).
 */
gdr_status gdr_backward(const gdr_desc* desc, const void* q, const void* k, const void* v,
                        const float* beta, const float* alpha, const float* S0,
                        const void* dO, const float* dST, const void* dh_clvr,
                        const float* clvr_scale, void* dq, void* dk, void* dv, float* dbeta,
                        float* dalpha, float* dS0, float* dclvr_scale, void* ws,
                        size_t ws_bytes, void* stream);

/* Training pair: a forward that keeps its intermediates, and the backward that
 * uses them instead of recomputing them (the per-chunk operands of the
 * intra-chunk transform and the chunk-start states and U of the state pass).
 *
 * gdr_forward_train computes exactly what gdr_forward_chunked computes (same
 * arguments, same results bit for bit) and in addition leaves in `ws` the
 * intermediates gdr_backward_saved reads.  Its workspace has the backward's
 * size, gdr_workspace_size(desc, 1).
 *
 * gdr_backward_saved takes the arguments of gdr_backward and returns the same
 * gradients bit for bit.  Its `ws` must be the workspace of the preceding
 * gdr_forward_train call on the same stream, with the same desc, q, k, v, beta,
 * alpha and S0, none of them modified in between (the library cannot check
 * this; other contents give wrong gradients, never an out-of-bounds access).
 */
gdr_status gdr_forward_train(const gdr_desc* desc, const void* q, const void* k,
                             const void* v, const float* beta, const float* alpha,
                             const float* S0, void* o, float* ST, void* h_clvr,
                             const float* clvr_scale, void* ws, size_t ws_bytes,
                             void* stream);

gdr_status gdr_backward_saved(const gdr_desc* desc, const void* q, const void* k,
                              const void* v, const float* beta, const float* alpha,
                              const float* S0, const void* dO, const float* dST,
                              const void* dh_clvr, const float* clvr_scale, void* dq,
                              void* dk, void* dv, float* dbeta, float* dalpha, float* dS0,
                              float* dclvr_scale, void* ws, size_t ws_bytes, void* stream);

/* Allocation-free chunked forward, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same arguments, checks and results (bit for bit) as
 * gdr_forward_chunked, without ws / ws_bytes: the workspace is a fixed device
 * array inside the library of GDR_NOALLOC_SCRATCH_BYTES (256 MiB), one per
 * GPU, held until the process ends.  A descriptor whose
 * gdr_workspace_size(desc, 0) exceeds it returns GDR_ERR_WORKSPACE (at
 * d = 128 with bf16 inputs the limit is about 2,100 chunk-heads, e.g. B = 1,
 * H = 16, T = 8192).  The call allocates nothing.  Every call on a GPU shares
 * that GPU's array: calls that overlap in time on one GPU (different streams,
 * or threads without ordering) race and give wrong results; order them on one
 * stream or with events. */
#define GDR_NOALLOC_SCRATCH_BYTES (256ull * 1024ull * 1024ull)
size_t gdr_noalloc_scratch_bytes(void);
gdr_status gdr_forward_chunked_noalloc(const gdr_desc* desc, const void* q, const void* k,
                                       const void* v, const float* beta, const float* alpha,
                                       const float* S0, void* o, float* ST, void* h_clvr,
                                       const float* clvr_scale, void* stream);

/* One decode step for N independent sequences, state updated in place
 * (inference with a fixed-size state, KDA blog section 6.1):
 *   p = S^T (alpha*k), r = S^T (alpha*q), u = beta (v - p),
 *   o = scale (r + u (k.q)),  S <- Diag(alpha) S + k u^T,
 * which is exactly one step of the recurrence above.
 *   q, k [N,H,dk] and v [N,H,dv] in in_dtype; beta [N,H] fp32;
 *   alpha NULL (NONE), [N,H] (SCALAR) or [N,H,dk] (CHANNEL) fp32;
 *   S [N,H,dk,dv] fp32 in/out; o [N,H,dv] in out_dtype (must not alias S).
 * No workspace. */
gdr_status gdr_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, int32_t gate,
                           int32_t in_dtype, int32_t out_dtype, float scale, const void* q,
                           const void* k, const void* v, const float* beta,
                           const float* alpha, float* S, void* o, void* stream);

/* Output-gate epilogue, the elementwise tail of the gated output of KDA blog
 * section 4.1 (o_t = W_o(Sigmoid(W_up W_down x_t) * RMSNorm(KDA(...)))); the
 * projections are GEMMs outside this library and g is the caller's low-rank
 * projection output.  Per token and head:
 *     y = sigmoid(g) * w * o / sqrt(mean_j o_j^2 + 1e-6)      (j over dv)
 *   o, y      [B,T,H,dv] in out_dtype (the operator's output); y may be o itself
 *   g         [B,T,H,dv] in in_dtype
 *   w         [H*dv] fp32 norm weight, NULL = ones
 * Only B, T, H, dv, in_dtype and out_dtype of desc are used (dk must equal dv).
 * No workspace. */
gdr_status gdr_output_gate_forward(const gdr_desc* desc, const void* o, const void* g, const float* w,
                                   void* y, void* stream);

/* Bytes of workspace gdr_output_gate_backward needs (the partial sums of dw). */
size_t gdr_output_gate_workspace_size(const gdr_desc* desc);

/* Backward of gdr_output_gate_forward, from dy [B,T,H,dv] (out_dtype):
 *   dO   [B,T,H,dv] in in_dtype: the gradient of o, in the dtype gdr_backward
 *        takes as its dO
 *   dg   [B,T,H,dv] in in_dtype
 *   dw   [H*dv] fp32, NULL = not computed (then ws may be NULL)
 * Outputs must not overlap the inputs or each other. */
gdr_status gdr_output_gate_backward(const gdr_desc* desc, const void* o, const void* g, const float* w,
                                    const void* dy, void* dO, void* dg, float* dw, void* ws, size_t ws_bytes,
                                    void* stream);

/* Gated DeltaNet-2: separate erase and write gates (popular article on the
 * study, its Gated DeltaNet-2 paragraph, which describes the mechanism in words
 * only: erasing and writing decoupled, each steered by its own gate computed
 * from the token, the erase gate choosing the regions of the memory to clear,
 * the write gate the regions to write; equal gates fall back to Kimi Delta
 * Attention).  Reading implemented, with the regions taken as key channels:
 *     S_t = (I - (e_t*k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t*k_t) v_t^T
 *     o_t = scale * S_t^T q_t                          (* elementwise)
 *   erase, write  [B, T, H, dk] fp32 (any finite values; gates in [0, 1])
 *   q, k, v, alpha, S0, ST, o as for gdr_forward_chunked; e = w = beta 1
 *   computes what gdr_forward_chunked computes.
 * desc->route and desc->prologue must be 0 (no hidden-stream epilogue: the
 * article leaves open what routing the written value means here), else
 * GDR_ERR_UNSUPPORTED.  For bf16 inputs the chunk products and the state
 * pass take fp16 operands with fp32 accumulation and an fp32 state (as
 * gdr_forward_chunked); fp32 inputs run in fp32 throughout.  Forward only (no
 * backward in this version).
 * ws: at least gdr_gdn2_workspace_size(desc) bytes (240.5 KiB per chunk-head
 * of 64 tokens at dk = dv = 128, plus one fp32 [dk][dv] state per (batch,
 * head) handed between the chunk ranges of a cut state pass). */
size_t gdr_gdn2_workspace_size(const gdr_desc* desc);
gdr_status gdr_gdn2_forward_chunked(const gdr_desc* desc, const void* q, const void* k, const void* v,
                                    const float* erase, const float* write, const float* alpha,
                                    const float* S0, void* o, float* ST, void* ws, size_t ws_bytes,
                                    void* stream);

/* One Gated DeltaNet-2 step for N sequences, S [N,H,dk,dv] fp32 in place:
 *   p = S^T (alpha*k), r = S^T (alpha*q),
 *   S <- Diag(alpha) S - (e*k) p^T + (w*k) v^T,
 *   o = scale (r - (q.(e*k)) p + (q.(w*k)) v),
 * exactly one step of the recurrence above; erase, write [N,H,dk] fp32, the
 * other arguments as for gdr_decode_step.  No workspace. */
gdr_status gdr_gdn2_decode_step(int64_t N, int64_t H, int64_t dk, int64_t dv, int32_t gate,
                                int32_t in_dtype, int32_t out_dtype, float scale, const void* q,
                                const void* k, const void* v, const float* erase, const float* write,
                                const float* alpha, float* S, void* o, void* stream);

/* Static text for a status code. */
const char* gdr_status_string(gdr_status status);

/* Thread-local detail for the last non-OK status returned on this thread. */
const char* gdr_last_error(void);

/* Library ABI version (major * 10000 + minor * 100 + patch). */
int32_t gdr_version(void);

/* Per-kernel timing (a measurement aid, off by default).
 * gdr_profile_begin() makes every later launch on this process record a HIP
 * event pair on the launch stream around each kernel (at most 65536 launches;
 * later ones are not recorded).  gdr_profile_end() waits for the recorded
 * events, fills up to `max` entries of `out` with, per kernel name, the number
 * of launches and their summed duration in milliseconds, returns the number of
 * entries, and turns recording off.  Not thread-safe: profile from one thread.
 * Returns -1 (gdr_last_error() says why) if the HIP runtime fails. */
typedef struct {
    char name[32];
    int64_t launches;
    double total_ms;
} gdr_kernel_time;

int32_t gdr_profile_begin(void);
int32_t gdr_profile_end(gdr_kernel_time* out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
