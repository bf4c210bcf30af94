// gdr_cler.hpp -- per-piece arithmetic of the error-routing epilogue (CLER-H).
//
// CLER-H (popular article on the study, cross-layer section) adds the write
// error of the delta rule, e_t = v_t - (Diag(alpha_t) S_{t-1})^T k_t, into the
// hidden stream: h[t, h*dv + j] += lam[h*dv + j] * e_t[j].  The chunked form
// keeps u_t = beta_t e_t (the rows of U), so e_t = u_t / beta_t; beta == 0 is
// outside the domain.
//
// The saved U is in fragment order: piece p (eight consecutive columns of one
// row) is lane p % 64 of fragment p / 64 = (row tile, 32-column step).  The
// kernels below walk the pieces of a chunk, which keeps the U reads contiguous
// and lets 256 threads cover whole 128-byte lines of the hidden rows.
#pragma once

#include "gdr_common.hpp"

namespace gdr {

template <int D>
__device__ __forceinline__ void frag_piece(int p, int& pos, int& j) {
    const int f = p >> 6, l = p & 63;
    pos = 16 * (f / (D / 32)) + (l & 15);
    j = 32 * (f % (D / 32)) + 8 * (l >> 4);
}

// h[0..7] += lam[0..7] * u[0..7] / beta for one piece of a hidden row.
template <typename InT>
__device__ __forceinline__ void cler_add8(InT* hrow, const float (&u)[8], const float (&lm)[8], float beta) {
    float hv[8];
    load8f(hrow, hv);
    const float ib = 1.f / beta;
#pragma unroll
    for (int e = 0; e < 8; ++e) hv[e] = __builtin_fmaf(lm[e], u[e] * ib, hv[e]);
    store8f(hrow, hv);
}

}  // namespace gdr
