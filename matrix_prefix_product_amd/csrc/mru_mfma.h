// Tile arithmetic on the CDNA matrix cores for n = 16 and n = 32 (fp64), shared
// by the scans and the orthogonal-input builds.
//
// An n-by-n matrix is held as (n/16)^2 tiles of 16x16, each in the accumulator
// layout of v_mfma_f64_16x16x4_f64; a 16x16x16 tile product is 4 MFMAs.  Read
// as a B operand, an accumulator tile is the B layout of the same tile once the
// k index of each k-block is permuted (block b, lane group kk holds k = 4b+kk),
// so the result of one product feeds the next with no lane shuffles, provided
// the left operand's entries are loaded with the same permutation.  Layout of
// v_mfma_f64_16x16x4_f64 on gfx950 (checked on the device by the scans' parity
// pins):
//   A[i][k] lane i+16k,  B[k][j] lane j+16k,  D[i][j] lane j+16(i%4), reg i/4.
// The accumulator interleaves rows across lane groups, so a tile's row index
// is relabelled with pi(i) = 4(i%4) + i/4 (a fixed permutation applied to both
// the rows of X and the rows of A, which leaves the algebra unchanged).  In
// actual indices every lane then holds 4 contiguous entries of one row per
// tile, and only the row index of each A-operand entry is permuted (tacol).
#pragma once

#include <hip/hip_runtime.h>

#include "mru_device.h"

namespace mru {

typedef double d4 __attribute__((ext_vector_type(4)));


// Lane geometry of one 16x16 tile (actual indices).
__device__ inline int tcol(int l) { return l & 15; }                     // column of X held
__device__ inline int trow(int l, int r) { return 4 * (l >> 4) + r; }   // row of entry r / k of block r
__device__ inline int tacol(int l) { return 4 * (l & 3) + ((l & 15) >> 2); }  // row of A entries

template <int N>
struct Mf {
    static constexpr int NT = N / 16;  // tiles per dimension
    static constexpr int NN = N * N;
    using acc_t = double;
    struct vec_t {
        d4 t[NT][NT];  // tile (I, J): X[16I + trow][16J + tcol]
    };
    // A-operand entries a[I][K][b] of one step (tile (I, K), k-block b)
    struct aop_t {
        double v[NT][NT][4];
    };
};

__device__ inline d4 mfma(double a, double b, d4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// X <- A X + C.  a holds this lane's A entries; X's accumulator entry b of tile
// (K, J) is the matching B entry of k-block b.
template <int N>
__device__ inline typename Mf<N>::vec_t chain_step(const typename Mf<N>::aop_t& a,
                                                   const typename Mf<N>::vec_t& X,
                                                   const typename Mf<N>::vec_t& C) {
    constexpr int NT = Mf<N>::NT;
    typename Mf<N>::vec_t out;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            d4 acc = C.t[I][J];
#pragma unroll
            for (int K = 0; K < NT; ++K)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc = mfma(a.v[I][K][b], X.t[K][J][b], acc);
            out.t[I][J] = acc;
        }
    return out;
}

// chain_step that calls between(k) after its k-th product (k = 0, 1, ...),
// with a scheduling barrier on each side.  Instructions issue in order and a
// product that needs the previous one's accumulator waits for it, so work
// placed after the last product would only start once all of them have been
// issued; placed between them (LDS traffic of the next token's operand, the
// previous prefix's store, loads) it runs while they execute.
template <int N, class Between>
__device__ inline typename Mf<N>::vec_t chain_step_with(const typename Mf<N>::aop_t& a,
                                                        const typename Mf<N>::vec_t& X,
                                                        const typename Mf<N>::vec_t& C,
                                                        Between&& between) {
    constexpr int NT = Mf<N>::NT;
    typename Mf<N>::vec_t out;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            d4 acc = C.t[I][J];
#pragma unroll
            for (int K = 0; K < NT; ++K)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    acc = mfma(a.v[I][K][b], X.t[K][J][b], acc);
                    __builtin_amdgcn_sched_barrier(0);
                    between(((I * NT + J) * NT + K) * 4 + b);
                    __builtin_amdgcn_sched_barrier(0);
                }
            out.t[I][J] = acc;
        }
    return out;
}

template <int N>
__device__ inline typename Mf<N>::vec_t vzero() {
    typename Mf<N>::vec_t v;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) v.t[I][J] = d4{0.0, 0.0, 0.0, 0.0};
    return v;
}

template <int N>
__device__ inline typename Mf<N>::vec_t videntity(int l) {
    typename Mf<N>::vec_t v;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                v.t[I][J][r] = (16 * I + trow(l, r) == 16 * J + tcol(l)) ? 1.0 : 0.0;
    return v;
}

// The accumulator holds X = Y^T; store / load Y row-major at p.  Lane entries
// of tile (I, J) are Y[16J + tcol][16I + trow(l, 0..3)], 4 contiguous values.
// The same fp32 stores, non-temporal (the nt bit): for outputs that are streamed
// once and not read back by the kernel.
template <int N>
__device__ inline void store_acc_rows_nt(float* p, const typename Mf<N>::vec_t& X) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) {
            float* q = p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0);
            const d4 x = X.t[I][J];
            const f4v v = {float(x[0]), float(x[1]), float(x[2]), float(x[3])};
            __builtin_nontemporal_store(v, reinterpret_cast<f4v*>(q));
        }
}

template <int N, class T>
__device__ inline void store_acc_rows(T* p, const typename Mf<N>::vec_t& X) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) {
            T* q = p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0);
            const d4 x = X.t[I][J];
            if constexpr (sizeof(T) == 4) {
                *reinterpret_cast<float4*>(q) = make_float4(float(x[0]), float(x[1]), float(x[2]), float(x[3]));
            } else {
                *reinterpret_cast<double2*>(q) = make_double2(x[0], x[1]);
                *reinterpret_cast<double2*>(q + 2) = make_double2(x[2], x[3]);
            }
        }
}

template <int N, class T>
__device__ inline typename Mf<N>::vec_t load_acc_rows(const T* p) {
    const int l = threadIdx.x & 63;
    typename Mf<N>::vec_t X;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) {
            const T* q = p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0);
            if constexpr (sizeof(T) == 4) {
                const float4 v = *reinterpret_cast<const float4*>(q);
                X.t[I][J] = d4{v.x, v.y, v.z, v.w};
            } else {
                const double2 v0 = *reinterpret_cast<const double2*>(q);
                const double2 v1 = *reinterpret_cast<const double2*>(q + 2);
                X.t[I][J] = d4{v0.x, v0.y, v1.x, v1.y};
            }
        }
    return X;
}

// A operand for X <- Y^T X (right multiplication of the untransposed state by
// Y, row-major at p): a[I][K][b] = Y[16K + trow(l, b)][16I + tacol(l)].
template <int N, class T>
__device__ inline void load_a_transposed(typename Mf<N>::aop_t& a, const T* p) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int K = 0; K < Mf<N>::NT; ++K)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                a.v[I][K][b] = double(p[(16 * K + trow(l, b)) * N + 16 * I + tacol(l)]);
}

// A operand for X <- Y X (left multiplication of the state by Y, row-major at
// p): a[I][K][b] = Y[16I + tacol(l)][16K + trow(l, b)], 4 contiguous values.
template <int N, class T>
__device__ inline void load_a_direct(typename Mf<N>::aop_t& a, const T* p) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int K = 0; K < Mf<N>::NT; ++K) {
            const T* q = p + (16 * I + tacol(l)) * N + 16 * K + trow(l, 0);
#pragma unroll
            for (int b = 0; b < 4; ++b) a.v[I][K][b] = double(q[b]);
        }
}

}  // namespace mru
