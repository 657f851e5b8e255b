// One row of an input state matrix from a raw token vector (LDU fill with a
// determinant-correcting scalar; "Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points).  The mean is shared with the scans that
// start from raw token vectors, so both compute the same e_k.
//
// For X = the token vector viewed row-major n-by-n (in LDS or registers):
//   e_k = exp(X_kk - mean_j X_jj),  M_ij = sum_{k <= min(i, j)} L_ik e_k U_kj,
// with L_ik = X_ik (k < i), L_ii = 1, U_kj = X_kj (k < j), U_kk = 1.
#pragma once

#include <hip/hip_runtime.h>

namespace mru {

// mean_j X_jj, summed in index order.  Contraction is off so that the final
// scaling never fuses into a caller's subtraction: every caller gets the same
// rounded mean, whatever the surrounding code.
template <int N>
__device__ inline float ldu_mean(const float* X) {
#pragma clang fp contract(off)
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) sum += X[k * N + k];
    return sum * (1.0f / N);
}

// The same mean from the diagonal already gathered, d[k] = X_kk: the same sum
// in the same order, so the same rounded value.
template <int N>
__device__ inline float ldu_mean_diag(const float (&d)[N]) {
#pragma clang fp contract(off)
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) sum += d[k];
    return sum * (1.0f / N);
}

// acc[j] = M_ij for j = 0..N-1, given e[k] = exp(X_kk - mean); n = 4, 8 (the
// matrix-core build covers n = 16, 32).  The k loop is fully unrolled, so U's
// zero pattern is resolved at compile time.
template <int N, class E>
__device__ inline void ldu_row(const float* X, int i, const E& e, float (&acc)[N]) {
    static_assert(N == 4 || N == 8, "vector-ALU rows for n = 4, 8");
#pragma unroll
    for (int j = 0; j < N; ++j) acc[j] = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const float ek = e(k);
        const float coef = (k < i) ? X[i * N + k] * ek : ((k == i) ? ek : 0.f);
#pragma unroll
        for (int j = k; j < N; ++j) {
            const float u = (j == k) ? 1.f : X[k * N + j];
            acc[j] = fmaf(coef, u, acc[j]);
        }
    }
}

}  // namespace mru
