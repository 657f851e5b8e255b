// Orthogonal input state matrices ("Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points: orthogonal constraints through the Cayley
// map or the matrix exponential).  With X the row-major n-by-n view of a token
// vector and A = (X - X^T) / 2 its skew-symmetric part:
//   Cayley:       M = (I - A)^{-1} (I + A)
//   exponential:  M = exp(A)
// Both are orthogonal with det M = 1, so a scan of them keeps |P_t|_F = sqrt(n).
//
// On the vector ALUs (Cayley for every n, the exponential for n = 4, 8) a
// chain of n lanes works on one token, lane i owning row i, in fp64 (the
// vector fp64 rate equals the fp32 one on CDNA4, and fp64 keeps the only
// rounding of the result the final one to fp32).  Rows of the other lanes come
// through LDS.  The exponential for n = 16, 32 runs on the matrix cores
// (build_expm_mfma_kernel below), also in fp64.
//   Cayley: Gauss-Jordan elimination on [I - A | I + A].  No pivoting is needed:
//     the symmetric part of I - A is I, so every leading block is nonsingular.
//   Exponential: scaling and squaring.  A is scaled by 2^-s (exact) so that its
//     largest row sum is at most 1/2, exp of the scaled matrix is summed by
//     Horner's rule to degree 12 (remainder below 1e-14), then squared s times.
//     s is the token's own; the wave runs the largest s among its tokens with
//     each token's squarings gated to its own count, so a token's result never
//     depends on the tokens it shares a wave with.
#include "mru_device.h"
#include "mru_kernels.h"
#include "mru_mfma.h"

namespace mru {
namespace {

constexpr int kTaylorDegree = 12;

template <int N>
struct Orth {
    static constexpr int NN = N * N;
    static constexpr int TPW = 64 / N;          // tokens per wave
    static constexpr int XS = TPW * NN;         // staged floats per wave
    static constexpr int ES = N + 1;            // LDS row stride of a token's matrix (doubles)
};

template <int N>
__device__ inline double group_max_d(double v) {
#pragma unroll
    for (int m = 1; m < N; m <<= 1) v = fmax(v, __shfl_xor(v, m, 64));
    return v;
}

template <int N, int METHOD>
__global__ __launch_bounds__(64) void build_orth_kernel(const float* __restrict__ x,
                                                        float* __restrict__ M, int64_t ntok) {
    using O = Orth<N>;
    __shared__ __align__(16) float xs[O::XS];
    __shared__ double ms[O::TPW * N * O::ES];
    __shared__ double as[METHOD == 1 ? O::TPW * N * O::ES : 2];  // rows of the scaled A
    const int lane = threadIdx.x & 63;
    const int tk = lane / N;  // token of the wave
    const int i = lane % N;   // row
    double* mine = ms + tk * N * O::ES;
    const int64_t groups = (ntok + O::TPW - 1) / O::TPW;
    for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
        const int64_t tok0 = grp * O::TPW;
        const int64_t tok = tok0 + tk;
        const bool live = tok < ntok;
        // stage the wave's tokens (float4 per lane per step; zeros past the end)
        __syncthreads();
#pragma unroll
        for (int q = 0; q < O::XS / 256; ++q) {
            const int f = q * 64 + lane;  // float4 index within the wave's tokens
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (tok0 + (f * 4) / O::NN < ntok)
                v = reinterpret_cast<const float4*>(x + tok0 * O::NN)[f];
            reinterpret_cast<float4*>(xs)[f] = v;
        }
        __syncthreads();
        const float* X = xs + tk * O::NN;
        double a[N];  // row i of A
#pragma unroll
        for (int j = 0; j < N; ++j) a[j] = 0.5 * (double(X[i * N + j]) - double(X[j * N + i]));

        double r[N];  // row i of the result
        if constexpr (METHOD == 0) {
            double lft[N];
#pragma unroll
            for (int j = 0; j < N; ++j) {
                lft[j] = (j == i ? 1.0 : 0.0) - a[j];
                r[j] = (j == i ? 1.0 : 0.0) + a[j];
            }
            // pivot row k (normalised) goes to the token's LDS rows 0 (left) and 1 (right)
#pragma unroll
            for (int k = 0; k < N; ++k) {
                // read column k before branching: inside "i == k" the compiler
                // would rewrite lft[k] as lft[i], a lane-dependent index that
                // moves the whole row to scratch memory
                const double lk = lft[k];
                __syncthreads();
                if (i == k) {
                    const double inv = 1.0 / lk;
#pragma unroll
                    for (int j = 0; j < N; ++j) {
                        lft[j] *= inv;
                        r[j] *= inv;
                        mine[j] = lft[j];
                        mine[O::ES + j] = r[j];
                    }
                }
                __syncthreads();
                if (i != k) {
                    const double f = lk;
#pragma unroll
                    for (int j = 0; j < N; ++j) {
                        lft[j] = fma(-f, mine[j], lft[j]);
                        r[j] = fma(-f, mine[O::ES + j], r[j]);
                    }
                }
            }
        } else {
            // scale: largest absolute row sum of A to at most 1/2
            double rs = 0.0;
#pragma unroll
            for (int j = 0; j < N; ++j) rs += fabs(a[j]);
            const double nrm = group_max_d<N>(rs);
            const int s = nrm > 0.5 ? frexp_exp(nrm) + 1 : 0;  // nrm < 2^e, so nrm 2^-s <= 1/2
            const int s_wave = __builtin_amdgcn_readfirstlane(group_max<64>(s));
            double* arow = as + (tk * N + i) * O::ES;  // the lane's row of A, read back per k
#pragma unroll
            for (int j = 0; j < N; ++j) arow[j] = ldexp(a[j], -s);
            // Horner: E = I + (A E) / d, ..., E = I + (A E) / 1, starting from E = I
#pragma unroll
            for (int j = 0; j < N; ++j) r[j] = (j == i) ? 1.0 : 0.0;
#pragma unroll 1
            for (int d = kTaylorDegree; d >= 1; --d) {
                __syncthreads();
#pragma unroll
                for (int j = 0; j < N; ++j) mine[i * O::ES + j] = r[j];
                __syncthreads();
                // row i of A E, accumulated in place of r (already in LDS)
#pragma unroll
                for (int j = 0; j < N; ++j) r[j] = 0.0;
#pragma unroll
                for (int k = 0; k < N; ++k) {
                    const double c = arow[k];
#pragma unroll
                    for (int j = 0; j < N; ++j) r[j] = fma(c, mine[k * O::ES + j], r[j]);
                }
                const double inv = 1.0 / double(d);
#pragma unroll
                for (int j = 0; j < N; ++j) r[j] = fma(r[j], inv, (j == i) ? 1.0 : 0.0);
            }
#pragma unroll 1
            for (int q = 0; q < s_wave; ++q) {
                __syncthreads();
#pragma unroll
                for (int j = 0; j < N; ++j) mine[i * O::ES + j] = r[j];
                __syncthreads();
                if (q < s) {  // row i of E E; the coefficients are this lane's row, in LDS
#pragma unroll
                    for (int j = 0; j < N; ++j) r[j] = 0.0;
#pragma unroll
                    for (int k = 0; k < N; ++k) {
                        const double c = mine[i * O::ES + k];
#pragma unroll
                        for (int j = 0; j < N; ++j) r[j] = fma(c, mine[k * O::ES + j], r[j]);
                    }
                }
            }
        }
        if (live) {
            float4* out = reinterpret_cast<float4*>(M + tok * O::NN + i * N);
#pragma unroll
            for (int c = 0; c < N / 4; ++c)
                out[c] = make_float4(float(r[4 * c]), float(r[4 * c + 1]), float(r[4 * c + 2]),
                                     float(r[4 * c + 3]));
        }
    }
}

// Cayley map by columns (n = 8, 16, 32): lane j of a token's 2n lanes owns
// column j of the augmented matrix [I - A | I + A].  Gauss-Jordan without
// pivoting, as above, with the same arithmetic on every entry (the pivot row
// scaled by the reciprocal of the pivot, then one fused multiply-add per entry
// and step, steps in order), so the result is bitwise that of the row kernel.
// But a step needs only the pivot column (n values held by one lane; each
// lane's own pivot-row entry is in its registers), and it reaches the other
// lanes without LDS: for n = 8 a token is one 16-lane row and a DPP row
// broadcast moves each value; for n = 16, 32 a wave works on one token (for
// n = 16 the upper 32 lanes idle) and readlane puts the pivot column in scalar
// registers, which the multiply-adds read directly.  Lanes n..2n-1 end up
// holding the columns of M.  (n = 4 keeps the row kernel: two 8-lane tokens
// per row need two masked broadcasts per value, which measured slower.)
template <int B, int E, class F>
__device__ inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// Value of v in lane k of the lane's token (k a compile-time constant).
template <int N, int k>
__device__ inline double bcast_col(double v) {
    const int lo = __double2loint(v), hi = __double2hiint(v);
    int rlo, rhi;
    if constexpr (N == 8) {
        rlo = __builtin_amdgcn_update_dpp(0, lo, 0x150 + k, 0xF, 0xF, false);  // row_newbcast:k
        rhi = __builtin_amdgcn_update_dpp(0, hi, 0x150 + k, 0xF, 0xF, false);
    } else {  // one token per wave, starting at lane 0
        rlo = __builtin_amdgcn_readlane(lo, k);
        rhi = __builtin_amdgcn_readlane(hi, k);
    }
    return __hiloint2double(rhi, rlo);
}

template <int N>
__global__ __launch_bounds__(64) void build_cayley_cols_kernel(const float* __restrict__ x,
                                                               float* __restrict__ M, int64_t ntok) {
    static_assert(N == 8 || N == 16 || N == 32, "column kernel for n = 8, 16, 32");
    constexpr int NN = N * N;
    constexpr int W = 2 * N;                    // lanes per token
    constexpr int TPW = N == 8 ? 64 / W : 1;    // tokens per wave
    constexpr int XS = TPW * NN;                // staged floats per wave
    __shared__ __align__(16) float xs[XS];
    const int lane = threadIdx.x & 63;
    const int tk = TPW > 1 ? lane / W : 0;      // token of the wave
    const int j = lane % W;                     // column of [I - A | I + A]
    const int jc = j % N;                       // column of A
    const double sgn = j < N ? -1.0 : 1.0;
    const bool owner = TPW > 1 || lane < W;     // lanes 32-63 idle for n = 16
    const int64_t groups = (ntok + TPW - 1) / TPW;
    for (int64_t grp = blockIdx.x; grp < groups; grp += gridDim.x) {
        const int64_t tok0 = grp * TPW;
        const int64_t tok = tok0 + tk;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < XS / 256; ++q) {
            const int f = q * 64 + lane;  // float4 index within the wave's tokens
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (tok0 + (f * 4) / NN < ntok) v = reinterpret_cast<const float4*>(x + tok0 * NN)[f];
            reinterpret_cast<float4*>(xs)[f] = v;
        }
        __syncthreads();
        const float* X = xs + tk * NN;
        double col[N];  // column j: I -/+ A
#pragma unroll
        for (int i = 0; i < N; ++i)
            col[i] = (i == jc ? 1.0 : 0.0) + sgn * (0.5 * (double(X[i * N + jc]) - double(X[jc * N + i])));
        static_for<0, N>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const double piv = bcast_col<N, k>(col[k]);  // pivot, from column k
            const double r = col[k] * (1.0 / piv);       // this column's pivot-row entry
            static_for<0, N>([&](auto ic) {
                constexpr int i = decltype(ic)::value;
                if constexpr (i != k) {
                    const double m = bcast_col<N, k>(col[i]);  // pivot column, row i
                    col[i] = fma(-m, r, col[i]);
                }
            });
            col[k] = r;
        });
        if (owner && j >= N && tok < ntok) {
#pragma unroll
            for (int i = 0; i < N; ++i) M[tok * NN + i * N + jc] = float(col[i]);
        }
    }
}

template <int N>
hipError_t run_cayley_cols(const float* x, float* M, int64_t ntok, hipStream_t stream) {
    constexpr int TPW = N == 8 ? 64 / (2 * N) : 1;
    const int64_t groups = (ntok + TPW - 1) / TPW;
    const unsigned blocks = unsigned(groups < 16384 ? groups : 16384);
    hipLaunchKernelGGL((build_cayley_cols_kernel<N>), dim3(blocks), dim3(64), 0, stream, x, M, ntok);
    return hipGetLastError();
}

// Exponential for n = 16 and 32 on the matrix cores: the same scaling and
// squaring (Horner's rule to degree 12, then s squarings), one token per wave,
// every product a chain of fp64 16x16x4 MFMAs in the tile layout of
// mru_mfma.h.  The accumulator holds E = exp(-A), which is exp(A)^T because A
// is skew-symmetric, so that writing the accumulator's rows the way the scans
// write P stores exp(A) row-major.  The Horner products take -A as their left
// operand (formed once per token from the staged X); a squaring takes E
// itself, through one LDS transpose.
template <int N>
__global__ __launch_bounds__(64) void build_expm_mfma_kernel(const float* __restrict__ x,
                                                             float* __restrict__ M, int64_t ntok) {
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
    constexpr int NT = F::NT;
    constexpr int NN = N * N;
    __shared__ __align__(16) float xs[NN];
    __shared__ __align__(16) double es[NN];
    const int l = threadIdx.x & 63;
    for (int64_t tok = blockIdx.x; tok < ntok; tok += gridDim.x) {
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NN / 256; ++q)
            reinterpret_cast<float4*>(xs)[q * 64 + l] =
                reinterpret_cast<const float4*>(x + tok * NN)[q * 64 + l];
        __syncthreads();
        // s from the largest absolute row sum of A (lane i < n sums row i)
        double rs = 0.0;
        if (l < N) {
#pragma unroll
            for (int j = 0; j < N; ++j) rs += fabs(0.5 * (double(xs[l * N + j]) - double(xs[j * N + l])));
        }
        const double nrm = group_max_d<64>(rs);
        const int s = nrm > 0.5 ? frexp_exp(nrm) + 1 : 0;  // nrm < 2^e, so nrm 2^-s <= 1/2
        // left operand: -A 2^-s, entry (16I + tacol, 16K + trow(b)) of tile (I, K)
        typename F::aop_t a;
#pragma unroll
        for (int I = 0; I < NT; ++I)
#pragma unroll
            for (int K = 0; K < NT; ++K)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int r = 16 * I + tacol(l), c = 16 * K + trow(l, b);
                    a.v[I][K][b] = ldexp(0.5 * (double(xs[c * N + r]) - double(xs[r * N + c])), -s);
                }
        // Horner: E = I + (-A E) / d for d = 12 .. 1, from E = I
        vec_t E = videntity<N>(l);
#pragma unroll 1
        for (int d = kTaylorDegree; d >= 1; --d) {
            const vec_t AE = chain_step<N>(a, E, vzero<N>());
            const double inv = 1.0 / double(d);
#pragma unroll
            for (int I = 0; I < NT; ++I)
#pragma unroll
                for (int J = 0; J < NT; ++J)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        E.t[I][J][r] = fma(AE.t[I][J][r], inv,
                                           (16 * I + trow(l, r) == 16 * J + tcol(l)) ? 1.0 : 0.0);
        }
#pragma unroll 1
        for (int q = 0; q < s; ++q) {
            typename F::aop_t ae;
            __syncthreads();
            store_acc_rows<N, double>(es, E);  // E^T row-major
            __syncthreads();
            load_a_transposed<N, double>(ae, es);  // E as the left operand
            E = chain_step<N>(ae, E, vzero<N>());
        }
        store_acc_rows<N, float>(M + tok * NN, E);  // E^T = exp(A), row-major
    }
}

template <int N>
hipError_t run_expm_mfma(const float* x, float* M, int64_t ntok, hipStream_t stream) {
    const unsigned blocks = unsigned(ntok < 16384 ? ntok : 16384);
    hipLaunchKernelGGL((build_expm_mfma_kernel<N>), dim3(blocks), dim3(64), 0, stream, x, M, ntok);
    return hipGetLastError();
}

template <int N, int METHOD>
hipError_t run_orth(const float* x, float* M, int64_t ntok, hipStream_t stream) {
    const int64_t groups = (ntok + Orth<N>::TPW - 1) / Orth<N>::TPW;
    const unsigned blocks = unsigned(groups < 16384 ? groups : 16384);
    hipLaunchKernelGGL((build_orth_kernel<N, METHOD>), dim3(blocks), dim3(64), 0, stream, x, M, ntok);
    return hipGetLastError();
}

template <int METHOD>
hipError_t run_orth_n(const float* x, float* M, int64_t ntok, int n, hipStream_t stream) {
    if constexpr (METHOD == 0) {  // Cayley
        switch (n) {
            case 4: return run_orth<4, 0>(x, M, ntok, stream);
            case 8: return run_cayley_cols<8>(x, M, ntok, stream);
            case 16: return run_cayley_cols<16>(x, M, ntok, stream);
            case 32: return run_cayley_cols<32>(x, M, ntok, stream);
            default: return hipErrorInvalidValue;
        }
    } else {  // exponential
        switch (n) {
            case 4: return run_orth<4, 1>(x, M, ntok, stream);
            case 8: return run_orth<8, 1>(x, M, ntok, stream);
            case 16: return run_expm_mfma<16>(x, M, ntok, stream);
            case 32: return run_expm_mfma<32>(x, M, ntok, stream);
            default: return hipErrorInvalidValue;
        }
    }
}

}  // namespace

hipError_t launch_build_orth(const float* x, float* M, int64_t ntok, int n, int method,
                             hipStream_t stream) {
    if (method == 0) return run_orth_n<0>(x, M, ntok, n, stream);
    if (method == 1) return run_orth_n<1>(x, M, ntok, n, stream);
    return hipErrorInvalidValue;
}

}  // namespace mru
