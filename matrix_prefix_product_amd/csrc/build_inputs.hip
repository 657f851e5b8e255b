// Input state matrices from raw token vectors: LDU fill with a
// determinant-correcting scalar ("Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points).
//
// For a token vector viewed row-major as X (n-by-n):
//   L = I + strictly-lower(X),  U = I + strictly-upper(X),  D = diag(exp X_ii),
//   c = |det(L D U)|^(-1/n) = exp(-mean_i X_ii)     (det L = det U = 1),
//   M = c L D U = L diag(e) U  with  e_k = exp(X_kk - mean_i X_ii),
// so  M_ij = sum_{k <= min(i, j)} L_ik e_k U_kj.
// Elementwise over tokens: a group of n/R lanes builds one token, each lane R
// rows of M, from the token staged in LDS.  HBM-bound (8 n^2 bytes per token).
#include "mru_device.h"
#include "mru_kernels.h"

namespace mru {
namespace {

constexpr int kBuildThreads = 128;

template <int N, int R>
__global__ __launch_bounds__(kBuildThreads) void build_kernel(const float* __restrict__ x,
                                                              float* __restrict__ M,
                                                              int64_t ntok) {
    constexpr int NN = N * N;
    constexpr int LPC = N / R;                   // lanes per token
    constexpr int TPI = kBuildThreads / LPC;     // tokens per block iteration
    constexpr int XS = NN + 4;                   // LDS stride per token (16 B skew)
    __shared__ float sx[TPI * XS];
    __shared__ float se[TPI * N];
    const int tid = threadIdx.x;
    const int tk = tid / LPC;
    const int li = tid % LPC;
    const float* xt = sx + tk * XS;
    for (int64_t tok0 = int64_t(blockIdx.x) * TPI; tok0 < ntok; tok0 += int64_t(gridDim.x) * TPI) {
        __syncthreads();
        for (int f = tid; f < TPI * NN / 4; f += kBuildThreads) {
            const int t = f / (NN / 4);
            const int q = f % (NN / 4);
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (tok0 + t < ntok) v = reinterpret_cast<const float4*>(x + (tok0 + t) * NN)[q];
            *reinterpret_cast<float4*>(sx + t * XS + 4 * q) = v;
        }
        __syncthreads();
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) sum += xt[k * N + k];
        const float mean = sum * (1.0f / N);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = li * R + r;
            se[tk * N + i] = expf(xt[i * N + i] - mean);
        }
        __syncthreads();
        float acc[R][N];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < N; ++j) acc[r][j] = 0.f;
        if constexpr (N <= 16) {
            // fully unrolled: the zero pattern of U is resolved at compile time
#pragma unroll
            for (int k = 0; k < N; ++k) {
                const float ek = se[tk * N + k];
                float coef[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int i = li * R + r;
                    coef[r] = (k < i) ? xt[i * N + k] * ek : ((k == i) ? ek : 0.f);
                }
#pragma unroll
                for (int j = k; j < N; ++j) {
                    const float u = (j == k) ? 1.f : xt[k * N + j];
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r][j] = fmaf(coef[r], u, acc[r][j]);
                }
            }
        } else {
            // k loop kept rolled (register pressure); U's zeros are masked
#pragma unroll 2
            for (int k = 0; k < N; ++k) {
                const float ek = se[tk * N + k];
                float coef[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int i = li * R + r;
                    coef[r] = (k < i) ? xt[i * N + k] * ek : ((k == i) ? ek : 0.f);
                }
#pragma unroll
                for (int j = 0; j < N; ++j) {
                    const float u = (j > k) ? xt[k * N + j] : ((j == k) ? 1.f : 0.f);
#pragma unroll
                    for (int r = 0; r < R; ++r) acc[r][j] = fmaf(coef[r], u, acc[r][j]);
                }
            }
        }
        const int64_t tok = tok0 + tk;
        if (tok < ntok) {
            float* dst = M + tok * NN + li * R * N;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < N / 4; ++q)
                    reinterpret_cast<float4*>(dst + r * N)[q] =
                        make_float4(acc[r][4 * q], acc[r][4 * q + 1], acc[r][4 * q + 2], acc[r][4 * q + 3]);
        }
    }
}

template <int N, int R>
hipError_t run_build(const float* x, float* M, int64_t ntok, hipStream_t stream) {
    constexpr int TPI = kBuildThreads / (N / R);
    int64_t blocks = (ntok + TPI - 1) / TPI;
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL((build_kernel<N, R>), dim3(unsigned(blocks)), dim3(kBuildThreads), 0,
                       stream, x, M, ntok);
    return hipGetLastError();
}

}  // namespace

// Rows per lane for each n (overridable at build time for tuning sweeps).
#ifndef MRU_BUILD_R4
#define MRU_BUILD_R4 1
#endif
#ifndef MRU_BUILD_R8
#define MRU_BUILD_R8 1
#endif
#ifndef MRU_BUILD_R16
#define MRU_BUILD_R16 2
#endif
#ifndef MRU_BUILD_R32
#define MRU_BUILD_R32 2
#endif

hipError_t launch_build(const float* x, float* M, int64_t ntok, int n, hipStream_t stream) {
    switch (n) {
        case 4: return run_build<4, MRU_BUILD_R4>(x, M, ntok, stream);
        case 8: return run_build<8, MRU_BUILD_R8>(x, M, ntok, stream);
        case 16: return run_build<16, MRU_BUILD_R16>(x, M, ntok, stream);
        case 32: return run_build<32, MRU_BUILD_R32>(x, M, ntok, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mru
