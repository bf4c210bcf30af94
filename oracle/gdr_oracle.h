/*
 * gdr_oracle.h -- fp64 reference ("oracle") for the gated delta-rule operator.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never links, loads or calls it, and it shares no code, header or constant
 * with the GPU path.
 *
 * What it computes (the plain definition, token by token, no chunking):
 *   Kimi Delta Attention blog ("线性注意力架构演进与Kimi Delta Attention创新实践"),
 *   section 2.1: the state update
 *       S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 *   and the read-out o_t = S_t^T q_t (read after the write, decay applied first).
 *   The three gate kinds are the family named by the linear-attention comparison
 *   explainer ("线性注意力架构：机制、权衡与跨层路由", core method 1): DeltaNet
 *   (alpha == 1), Gated DeltaNet (one alpha per token and head) and Kimi Delta
 *   Attention (one alpha per token, head and key channel).
 *
 * Layouts (row-major, contiguous, all double):
 *   q, k   [B, T, H, dk]      v, o   [B, T, H, dv]      beta [B, T, H]
 *   alpha  NONE: ignored (may be NULL); SCALAR: [B, T, H]; CHANNEL: [B, T, H, dk]
 *   S0, ST, dS0, dST  [B, H, dk, dv]
 * A NULL S0 means a zero initial state; a NULL ST is not written.
 *
 * Return value: 0 on success, -1 on a bad argument (negative size, NULL
 * required pointer, unknown gate), -2 when memory could not be allocated.
 */
#ifndef GDR_ORACLE_H
#define GDR_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_GATE_NONE = 0, ORACLE_GATE_SCALAR = 1, ORACLE_GATE_CHANNEL = 2 };

/* Forward recurrence over all tokens.  o = scale * S_t^T q_t.
 * nthreads <= 0 means one thread; work is split over the B*H independent slabs. */
int oracle_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                   double scale, const double* q, const double* k, const double* v,
                   const double* beta, const double* alpha, const double* S0,
                   double* o, double* ST, int nthreads);

/* Reverse-mode derivative of oracle_forward (adjoint of the token loop, with
 * state checkpoints every ceil(sqrt(T)) tokens and recomputation in between).
 * dO [B,T,H,dv]; dST NULL means zero.  Outputs dq, dk, dv, dbeta have the
 * shapes of their inputs; dalpha has alpha's shape (NULL allowed, and ignored,
 * for the NONE gate); dS0 may be NULL.  The derivative w.r.t. alpha is taken
 * with respect to alpha itself (not log alpha). */
int oracle_backward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                    double scale, const double* q, const double* k, const double* v,
                    const double* beta, const double* alpha, const double* S0,
                    const double* dO, const double* dST,
                    double* dq, double* dk_out, double* dv_out, double* dbeta,
                    double* dalpha, double* dS0, int nthreads);

/* oracle_forward that also writes every token's write error
 *     e_t = v_t - (Diag(alpha_t) S_{t-1})^T k_t        E [B, T, H, dv]
 * the correction the delta rule writes (u_t = beta_t e_t), which the
 * error-routing epilogue CLER-H sends into the hidden stream (popular article on
 * the study, cross-layer section).  E must not be NULL. */
int oracle_forward_errors(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                          double scale, const double* q, const double* k, const double* v,
                          const double* beta, const double* alpha, const double* S0, double* o,
                          double* ST, double* E, int nthreads);

/* oracle_backward with a gradient dE [B, T, H, dv] arriving at the write errors
 * e_t as well (NULL means zero, which is oracle_backward). */
int oracle_backward_errors(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate,
                           double scale, const double* q, const double* k, const double* v,
                           const double* beta, const double* alpha, const double* S0,
                           const double* dO, const double* dST, const double* dE, double* dq,
                           double* dk_out, double* dv_out, double* dbeta, double* dalpha,
                           double* dS0, int nthreads);

/* One recurrence step for N independent sequences (decode): S is [N,H,dk,dv]
 * and is updated in place; q,k [N,H,dk], v,o [N,H,dv], beta [N,H],
 * alpha [N,H] (SCALAR) or [N,H,dk] (CHANNEL). */
int oracle_decode(int64_t N, int64_t H, int64_t dk, int64_t dv, int gate, double scale,
                  const double* q, const double* k, const double* v, const double* beta,
                  const double* alpha, double* S, double* o, int nthreads);

/* Cross-Layer Value Routing epilogue (linear-attention comparison explainer,
 * cross-layer routing section; the abstract's "forward the write value"):
 * the written value v_t of this layer is added into the hidden stream,
 * h_out[b,t,h*dv+j] = h_in[b,t,h*dv+j] + lam[h*dv+j] * v[b,t,h,j].
 * lam NULL means lam == 1.  h_in and h_out may alias. */
int oracle_clvr_forward(int64_t B, int64_t T, int64_t H, int64_t dv, const double* h_in,
                        const double* v, const double* lam, double* h_out);

/* Derivative of the CLVR epilogue: dv_acc[b,t,h,j] += lam[h*dv+j] * dh[b,t,h*dv+j]
 * (dv_acc may be NULL), dlam[h*dv+j] = sum_{b,t} dh * v (dlam may be NULL). */
int oracle_clvr_backward(int64_t B, int64_t T, int64_t H, int64_t dv, const double* dh,
                         const double* v, const double* lam, double* dv_acc, double* dlam);

/* Gated DeltaNet-2 (popular article on the study, its Gated DeltaNet-2
 * paragraph: separate erase and write gates).  Reading (see the C file):
 *     S_t = (I - (e_t * k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t * k_t) v_t^T
 *     o_t = scale * S_t^T q_t
 * with the erase gate e and the write gate w [B, T, H, dk] (elementwise *);
 * alpha, S0, ST as for oracle_forward.  e = w = beta (broadcast over dk) is
 * oracle_forward's recurrence. */
int oracle_gdn2_forward(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv, int gate, double scale,
                        const double* q, const double* k, const double* v, const double* erase,
                        const double* write, const double* alpha, const double* S0, double* o, double* ST,
                        int nthreads);

/* One Gated DeltaNet-2 step for N sequences, S [N,H,dk,dv] updated in place;
 * erase, write [N,H,dk]. */
int oracle_gdn2_decode(int64_t N, int64_t H, int64_t dk, int64_t dv, int gate, double scale, const double* q,
                       const double* k, const double* v, const double* erase, const double* write,
                       const double* alpha, double* S, double* o, int nthreads);

#ifdef __cplusplus
}
#endif

#endif /* GDR_ORACLE_H */
