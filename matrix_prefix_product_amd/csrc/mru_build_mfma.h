// Per-token routines of the matrix-core (n = 16, 32) input build and its
// gradient, shared by the build kernels and the scans that form input matrices
// on chip, so that every path computes the same bits.  The LDU fill with a
// determinant-correcting scalar is from "Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points.  Wave64; the lanes of a DPP row (16
// lanes) hold one row of an accumulator tile of v_mfma_f32_16x16x4f32
// (A[i][k] in lane i + 16k, B[k][j] in lane j + 16k, D[i][j] in lane
// j + 16(i/4), register i%4).
#pragma once

#include <hip/hip_runtime.h>

#include "mru_mfma.h"

namespace mru {

// Sum over each row of 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror); every lane of the row gets the same bits (each
// step adds two values in either order).
__device__ inline float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// The same butterfly in fp64 (each step moves both 32-bit halves).
template <int CTRL>
__device__ inline double dpp_f64(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp(0, int(b), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, int(b >> 32), CTRL, 0xF, 0xF, false);
    return __longlong_as_double(static_cast<long long>(static_cast<unsigned>(lo)) |
                                (static_cast<long long>(hi) << 32));
}

__device__ inline double row16_sum_f64(double v) {
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    return v;
}

// e_k = exp(X_kk - mean_j X_jj) in fp64 for the token staged at xs (row stride
// n + 4): the diagonal summed in fp64 over each 16-lane row (every lane gets
// the same bits), scaled exactly by 1/n; lanes 0..n-1 write e_l to ed and, for
// the gradient's fp32 arithmetic, e_l rounded to fp32 to ef.
template <int N>
__device__ inline void token_e_f64(const float* xs, double* ed, float* ef) {
    constexpr int NT = N / 16;
    constexpr int LS = N + 4;
    const int l = threadIdx.x & 63;
    double dsum = 0.0;  // X_kk for k = l%16 (+ 16, n = 32)
#pragma unroll
    for (int t = 0; t < NT; ++t) dsum += double(xs[((l & 15) + 16 * t) * (LS + 1)]);
    const double mean = row16_sum_f64(dsum) * (1.0 / N);
    const int k = l & (N - 1);
    const double ek = exp(double(xs[k * (LS + 1)]) - mean);
    if (l < N) {
        ed[l] = ek;
        ef[l] = float(ek);
    }
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

// One 16x16 tile of M = Lt W, with Lt the unit lower factor of X (Lt_rk = X_rk
// for k < r, 1 on the diagonal) and W = diag(e) U (W_kc = e_k X_kc for k < c,
// e_k on the diagonal), in fp64 on the matrix core (v_mfma_f64_16x16x4f64:
// A[i][k] in lane i + 16k, B[k][j] in lane j + 16k, D[i][j] in lane
// j + 16(i%4), register i/4).  Rows come from the 16-row block RB through
// row(i), columns from the 16-column block CB through col(j); the k-tiles
// T <= min(RB, CB) are summed in ascending order (the others are zero).
//   TR false: D[i][j] = M[row(i)][col(j)]  (A entries from Lt, B from W)
//   TR true:  D[i][j] = M[row(j)][col(i)]  (A entries from W, B from Lt)
// Both sum the same fp64 products in the same k order, so every entry of M has
// the same bits whichever layout a caller asks for.  xs: X with row stride
// n + 4; ed: e in fp64.
template <int N, bool TR, class Row, class Col>
__device__ inline f64x4 ldu_tile_f64(const float* xs, const double* ed, int RB, int CB,
                                     Row row, Col col) {
    constexpr int LS = N + 4;
    const int l = threadIdx.x & 63;
    const int r = row(l & 15);  // the Lt row this lane supplies
    const int c = col(l & 15);  // the W column this lane supplies
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    const int tmax = RB < CB ? RB : CB;
#pragma unroll
    for (int T = 0; T < N / 16; ++T) {
        if (T > tmax) break;
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
            const int k = 16 * T + 4 * s4 + (l >> 4);
            const double lt = k < r ? double(xs[r * LS + k]) : (k == r ? 1.0 : 0.0);
            const double ek = ed[k];
            const double w = c > k ? ek * double(xs[k * LS + c]) : (c == k ? ek : 0.0);
            if constexpr (TR) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(w, lt, acc, 0, 0, 0);
            else acc = __builtin_amdgcn_mfma_f64_16x16x4f64(lt, w, acc, 0, 0, 0);
        }
    }
    return acc;
}

// One token's n-by-n result staged row-major in LDS (row stride n + 4) is
// written with 16-byte stores, 1 KiB of whole rows per wave instruction: a
// tile's accumulator holds column pieces, and writing those directly leaves
// every 128-byte row of an n = 32 matrix in two halves written at different
// times, which doubled the HBM write traffic.
template <int N>
__device__ inline void store_rows_from_lds(float* __restrict__ out, const float* ms) {
    constexpr int LS = N + 4;
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < N * N / 256; ++q) {
        const int f = q * 64 + l;        // float4 index within the token
        const int row = f / (N / 4);
        const int c = 4 * (f % (N / 4));
        reinterpret_cast<float4*>(out)[f] = *reinterpret_cast<const float4*>(ms + row * LS + c);
    }
}

// Gradient through the build for one token staged in LDS (row stride n + 4):
// xs = X (the token viewed n-by-n), gs = G = dL/dM, es = e (e_k =
// exp(X_kk - mean_j X_jj)); part is 4 floats of LDS.  With H = G U^T and
// (L^T G) as fp32 16x16x4 products (only the k-tiles where the triangular factor
// is nonzero), every lane holds entries (i, j) of both in the accumulator layout
// and writes into ds (row stride n + 4)
//   dX_ij = e_j H_ij (i > j),  e_i (L^T G)_ij (i < j),  e_i g_i - mean_k e_k g_k (i = j),
// g_i = sum_j (L^T G)_ij U_ij: a 16-lane DPP sum per accumulator row, and the
// mean over the four lane rows through part, added in a fixed order.  Contains
// one barrier; the caller orders ds's later reads with another.
template <int N>
__device__ inline void build_vjp_token(const float* xs, const float* gs, const float* es,
                                       float* part, float* ds) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    constexpr int NT = N / 16;
    constexpr int LS = N + 4;
    const int l = threadIdx.x & 63;
    const int m = l >> 4;  // lane row: accumulator rows 4m .. 4m+3 of each tile
    f4 h[NT][NT], u[NT][NT];  // H and L^T G, accumulator layout
    float eg = 0.f;           // sum over this lane row's diagonal entries of e_i g_i
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            const int i = 16 * I + (l & 15);  // A-operand row
            const int j = 16 * J + (l & 15);  // B-operand column
            f4 ah = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int K = J; K < NT; ++K)  // H = G U^T: U[j][k] = 0 for k < j
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int k = 16 * K + 4 * s4 + m;
                    const float a = gs[i * LS + k];
                    const float b = k > j ? xs[j * LS + k] : (k == j ? 1.f : 0.f);
                    ah = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, ah, 0, 0, 0);
                }
#pragma unroll
            for (int K = I; K < NT; ++K)  // L^T G: L[k][i] = 0 for k < i
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int k = 16 * K + 4 * s4 + m;
                    const float a = k > i ? xs[k * LS + i] : (k == i ? 1.f : 0.f);
                    const float b = gs[k * LS + j];
                    au = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, au, 0, 0, 0);
                }
            h[I][J] = ah;
            u[I][J] = au;
        }
    // g_i for this lane row's rows i = 16I + 4m + r
    float g[NT][4];
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * I + 4 * m + r;
            float p = 0.f;
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                const int j = 16 * J + (l & 15);
                const float uij = j > i ? xs[i * LS + j] : (j == i ? 1.f : 0.f);
                p = fmaf(u[I][J][r], uij, p);
            }
            g[I][r] = row16_sum(p);
            eg += es[i] * g[I][r];
        }
    if ((l & 15) == 0) part[m] = eg;
    wave_lds_sync();
    const float meaneg = (((part[0] + part[1]) + part[2]) + part[3]) * (1.0f / N);
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J < NT; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * I + 4 * m + r;
                const int j = 16 * J + (l & 15);
                float v;
                if (i > j) v = es[j] * h[I][J][r];
                else if (i < j) v = es[i] * u[I][J][r];
                else v = es[i] * g[I][r] - meaneg;
                ds[i * LS + j] = v;
            }
}

}  // namespace mru
