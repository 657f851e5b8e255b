// Input state matrices from raw token vectors: LDU fill with a
// determinant-correcting scalar ("Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points).
//
// For a token vector viewed row-major as X (n-by-n):
//   L = I + strictly-lower(X),  U = I + strictly-upper(X),  D = diag(exp X_ii),
//   c = |det(L D U)|^(-1/n) = exp(-mean_i X_ii)     (det L = det U = 1),
//   M = c L D U = L diag(e) U  with  e_k = exp(X_kk - mean_i X_ii),
// so  M_ij = sum_{k <= min(i, j)} L_ik e_k U_kj.
// Elementwise over tokens.  n = 4, 8: a group of n/R lanes builds one token,
// each lane R rows of M, from the token staged in LDS; n = 16, 32: one wave per
// token on the matrix cores (build_mfma_kernel).  HBM-bound (8 n^2 bytes per
// token).
#include <type_traits>

#include "mru_build.h"
#include "mru_build_mfma.h"
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
        const float mean = ldu_mean<N>(xt);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = li * R + r;
            se[tk * N + i] = expf(xt[i * N + i] - mean);
        }
        __syncthreads();
        float acc[R][N];
#pragma unroll
        for (int r = 0; r < R; ++r)
            ldu_row<N>(xt, li * R + r, [&](int k) { return se[tk * N + k]; }, acc[r]);
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

// Gradient through the LDU build (training through the input construction).
// For G = dL/dM, e_k = exp(X_kk - mean X) and H = G U^T:
//   dX_ij = e_j H_ij                     (i > j, through L)
//   dX_ij = e_i (L^T G)_ij               (i < j, through U)
//   dX_kk = e_k g_k - mean_j e_j g_j     (through e; X_kk also enters the mean)
// with g_k = (L^T G U^T)_kk = sum_r L_rk H_rk.  One lane per row of dX; the
// column sums for g go through LDS.  n = 4, 8 (n = 16, 32: build_bwd_mfma_kernel).
template <int N>
__global__ __launch_bounds__(kBuildThreads) void build_bwd_kernel(const float* __restrict__ x,
                                                                  const float* __restrict__ dM,
                                                                  float* __restrict__ dx,
                                                                  int64_t ntok) {
    static_assert(N == 4 || N == 8, "vector-ALU build backward for n = 4, 8");
    constexpr int NN = N * N;
    constexpr int TPI = kBuildThreads / N;  // tokens per block iteration
    constexpr int XS = NN + 4;
    __shared__ float sx[TPI * XS];
    __shared__ float sg[TPI * XS];
    __shared__ float sc[TPI * XS];
    __shared__ float se[TPI * N];
    __shared__ float seg[TPI * N];
    const int tid = threadIdx.x;
    const int tk = tid / N;
    const int i = tid % N;  // row of dX owned by this lane
    const float* xt = sx + tk * XS;
    const float* gt = sg + tk * XS;
    float* ct = sc + tk * XS;
    // The next iteration's x and dM are loaded into registers while this one
    // computes; loads are unconditional (tokens past the end read the last
    // token and are never stored), so the compiler can wait for them without
    // waiting for the stores issued after them.
    constexpr int LDQ = TPI * NN / 4 / kBuildThreads;  // float4 per thread and array
    static_assert(TPI * NN / 4 == LDQ * kBuildThreads, "tiles must cover the block");
    float4 px[LDQ], pg[LDQ];
    auto fetch = [&](int64_t tok0) {
#pragma unroll
        for (int k = 0; k < LDQ; ++k) {
            const int f = tid + k * kBuildThreads;
            const int64_t tok = min(tok0 + f / (NN / 4), ntok - 1);
            const float4 vx = reinterpret_cast<const float4*>(x + tok * NN)[f % (NN / 4)];
            const float4 vg = reinterpret_cast<const float4*>(dM + tok * NN)[f % (NN / 4)];
            px[k] = make_float4(vx.x, vx.y, vx.z, vx.w);
            pg[k] = make_float4(vg.x, vg.y, vg.z, vg.w);
        }
    };
    const int64_t step = int64_t(gridDim.x) * TPI;
    // FULL: all TPI tokens of the iteration exist, so the stores are unconditional.
    auto iteration = [&](int64_t tok0, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < LDQ; ++k) {
            const int f = tid + k * kBuildThreads;
            const int t = f / (NN / 4);
            const int q = f % (NN / 4);
            *reinterpret_cast<float4*>(sx + t * XS + 4 * q) = px[k];
            *reinterpret_cast<float4*>(sg + t * XS + 4 * q) = pg[k];
        }
        __syncthreads();
        fetch(tok0 + step);
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) sum += xt[k * N + k];
        const float mean = sum * (1.0f / N);
        se[tk * N + i] = expf(xt[i * N + i] - mean);
        __syncthreads();
        // H row i: H_ij = sum_{m >= j} G_im U_jm (U_jj = 1)
        float h[N];
        {
            float grow[N];
#pragma unroll
            for (int m = 0; m < N; ++m) grow[m] = gt[i * N + m];
#pragma unroll
            for (int j = 0; j < N; ++j) {
                float acc = grow[j];
#pragma unroll
                for (int m = j + 1; m < N; ++m) acc = fmaf(grow[m], xt[j * N + m], acc);
                h[j] = acc;
            }
        }
        // row i's terms of g_k = sum_r L_rk H_rk (L_ik = X_ik for k < i, L_ii = 1)
#pragma unroll
        for (int k = 0; k < N; ++k) ct[i * N + k] = (k < i) ? xt[i * N + k] * h[k] : ((k == i) ? h[k] : 0.f);
        // (L^T G) row i: sum_{m >= i} L_mi G_mj
        float u[N];
#pragma unroll
        for (int j = 0; j < N; ++j) u[j] = 0.f;
#pragma unroll
        for (int m = 0; m < N; ++m) {
            const float coef = (m > i) ? xt[m * N + i] : ((m == i) ? 1.f : 0.f);
#pragma unroll
            for (int j = 0; j < N; ++j) u[j] = fmaf(coef, gt[m * N + j], u[j]);
        }
        const float ei = se[tk * N + i];
        float out[N];
#pragma unroll
        for (int j = 0; j < N; ++j) out[j] = (j < i) ? se[tk * N + j] * h[j] : ((j > i) ? ei * u[j] : 0.f);
        __syncthreads();
        float gi = 0.f;
#pragma unroll
        for (int r = 0; r < N; ++r) gi += ct[r * N + i];
        seg[tk * N + i] = ei * gi;
        __syncthreads();
        float tot = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) tot += seg[tk * N + k];
        const float meaneg = tot * (1.0f / N);
#pragma unroll
        for (int j = 0; j < N; ++j)
            if (j == i) out[j] = seg[tk * N + i] - meaneg;
        const int64_t tok = tok0 + tk;
        if (FULL || tok < ntok) {
            float* dst = dx + tok * NN + i * N;
#pragma unroll
            for (int q = 0; q < N / 4; ++q)
                reinterpret_cast<float4*>(dst)[q] = make_float4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
        }
    };
    const std::integral_constant<bool, true> full;
    const std::integral_constant<bool, false> partial;
    int64_t tok0 = int64_t(blockIdx.x) * TPI;
    if (tok0 >= ntok) return;
    fetch(tok0);
    if (tok0 + TPI <= ntok) {
        // the first full iteration is peeled, so that the loop is entered only
        // from a full iteration
        iteration(tok0, full);
        for (tok0 += step; tok0 + TPI <= ntok; tok0 += step) iteration(tok0, full);
    }
    if (tok0 < ntok) iteration(tok0, partial);
}

template <int N>
hipError_t run_build_bwd(const float* x, const float* dM, float* dx, int64_t ntok, hipStream_t stream) {
    constexpr int TPI = kBuildThreads / N;
    int64_t blocks = (ntok + TPI - 1) / TPI;
    if (blocks > 256 * 16) blocks = 256 * 16;
    hipLaunchKernelGGL((build_bwd_kernel<N>), dim3(unsigned(blocks)), dim3(kBuildThreads), 0, stream,
                       x, dM, dx, ntok);
    return hipGetLastError();
}

// n = 16, 32 on the matrix cores.  M = Lt W, Lt the unit lower factor and
// W = diag(e) U, as fp64 16x16x4 products (ldu_tile_f64) with e in fp64, so
// each entry is the exact product up to fp64 rounding and is rounded to fp32
// once: M is the correctly rounded LDU product (an fp32 accumulation here was
// three times the rounding error, mostly the fp32 exponential on the diagonal,
// and the gradient of a long scan amplifies exactly that input error).  One
// wave per token: the token is staged in LDS, its diagonal summed in fp64 over
// a 16-lane row with DPP, e formed by lanes 0..N-1, then every lane reads its
// operand entries of Lt and W; tile (I, J) sums the k-tiles K <= min(I, J).
template <int N>
__global__ __launch_bounds__(64) void build_mfma_kernel(const float* __restrict__ x,
                                                       float* __restrict__ M, int64_t ntok) {
    static_assert(N == 16 || N == 32, "matrix-core build for n = 16, 32");
    constexpr int NT = N / 16;
    constexpr int NN = N * N;
    constexpr int LS = N + 4;       // LDS row stride (floats)
    constexpr int NV = NN / 256;    // float4 pieces per lane and token
    __shared__ __align__(16) float xs[N * LS];
    __shared__ __align__(16) float ms[N * LS];  // the token's M, row-major, for whole-row stores
    __shared__ double ed[N];
    __shared__ float ef[N];
    // native vector type: an array of HIP's float4 (a union) kept across the
    // barrier was not promoted to registers and went through scratch memory
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int l = threadIdx.x;
    for (int64_t tok = blockIdx.x; tok < ntok; tok += gridDim.x) {
        f4 v[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) v[q] = reinterpret_cast<const f4*>(x + tok * NN)[q * 64 + l];
        __syncthreads();  // the previous token's reads are done
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int f = q * 64 + l;
            *reinterpret_cast<f4*>(xs + (f / (N / 4)) * LS + 4 * (f % (N / 4))) = v[q];
        }
        __syncthreads();
        token_e_f64<N>(xs, ed, ef);
        __syncthreads();
#pragma unroll
        for (int I = 0; I < NT; ++I)
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                // D[i][j] = M[16I + i][16J + j]: lane l, register r holds row 4r + l/16
                const f64x4 acc = ldu_tile_f64<N, false>(
                    xs, ed, I, J, [&](int i) { return 16 * I + i; }, [&](int j) { return 16 * J + j; });
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ms[(16 * I + 4 * r + (l >> 4)) * LS + 16 * J + (l & 15)] = float(acc[r]);
            }
        __syncthreads();
        store_rows_from_lds<N>(M + tok * NN, ms);
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

// Its gradient at n = 16, 32 on the matrix cores, one wave per token.  With
// G = dL/dM, H = G U^T and (L^T G) as fp32 16x16x4 products (only the k-tiles
// where the triangular factor is nonzero), every lane holds entries (i, j) of
// both in the accumulator layout and writes
//   dX_ij = e_j H_ij (i > j),  e_i (L^T G)_ij (i < j),  e_i g_i - mean_k e_k g_k (i = j),
// g_i = sum_j (L^T G)_ij U_ij: a 16-lane DPP sum per accumulator row (lanes of
// a DPP row hold one row of a tile), and the mean over the four lane rows
// through LDS, added in a fixed order.
template <int N>
__global__ __launch_bounds__(64) void build_bwd_mfma_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ dM,
                                                           float* __restrict__ dx, int64_t ntok) {
    static_assert(N == 16 || N == 32, "matrix-core build backward for n = 16, 32");
    constexpr int NN = N * N;
    constexpr int LS = N + 4;
    constexpr int NV = NN / 256;
    __shared__ __align__(16) float xs[N * LS];
    __shared__ __align__(16) float gs[N * LS];
    __shared__ __align__(16) float ds[N * LS];  // the token's dx, row-major, for whole-row stores
    __shared__ double ed[N];
    __shared__ float es[N];
    __shared__ float part[4];
    typedef float f4 __attribute__((ext_vector_type(4)));  // (registers, as above)
    const int l = threadIdx.x;
    for (int64_t tok = blockIdx.x; tok < ntok; tok += gridDim.x) {
        f4 vx[NV], vg[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            vx[q] = reinterpret_cast<const f4*>(x + tok * NN)[q * 64 + l];
            vg[q] = reinterpret_cast<const f4*>(dM + tok * NN)[q * 64 + l];
        }
        __syncthreads();  // the previous token's reads are done
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int f = q * 64 + l;
            const int off = (f / (N / 4)) * LS + 4 * (f % (N / 4));
            *reinterpret_cast<f4*>(xs + off) = vx[q];
            *reinterpret_cast<f4*>(gs + off) = vg[q];
        }
        __syncthreads();
        token_e_f64<N>(xs, ed, es);  // e as the build forms it, rounded to fp32
        __syncthreads();
        build_vjp_token<N>(xs, gs, es, part, ds);
        __syncthreads();
        store_rows_from_lds<N>(dx + tok * NN, ds);
    }
}

template <int N>
hipError_t run_build_bwd_mfma(const float* x, const float* dM, float* dx, int64_t ntok,
                              hipStream_t stream) {
    int64_t blocks = ntok;
    if (blocks > 256 * 64) blocks = 256 * 64;
    hipLaunchKernelGGL((build_bwd_mfma_kernel<N>), dim3(unsigned(blocks)), dim3(64), 0, stream, x, dM,
                       dx, ntok);
    return hipGetLastError();
}

template <int N>
hipError_t run_build_mfma(const float* x, float* M, int64_t ntok, hipStream_t stream) {
    int64_t blocks = ntok;
    if (blocks > 256 * 64) blocks = 256 * 64;  // grid-stride beyond 64 waves per CU
    hipLaunchKernelGGL((build_mfma_kernel<N>), dim3(unsigned(blocks)), dim3(64), 0, stream, x, M, ntok);
    return hipGetLastError();
}

// The vector-ALU build (n = 4, 8) gives each lane one row of M (measured best).

hipError_t launch_build(const float* x, float* M, int64_t ntok, int n, hipStream_t stream) {
    switch (n) {
        case 4: return run_build<4, 1>(x, M, ntok, stream);
        case 8: return run_build<8, 1>(x, M, ntok, stream);
        case 16: return run_build_mfma<16>(x, M, ntok, stream);
        case 32: return run_build_mfma<32>(x, M, ntok, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_build_bwd(const float* x, const float* dM, float* dx, int64_t ntok, int n,
                            hipStream_t stream) {
    switch (n) {
        case 4: return run_build_bwd<4>(x, dM, dx, ntok, stream);
        case 8: return run_build_bwd<8>(x, dM, dx, ntok, stream);
        case 16: return run_build_bwd_mfma<16>(x, dM, dx, ntok, stream);
        case 32: return run_build_bwd_mfma<32>(x, dM, dx, ntok, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mru
