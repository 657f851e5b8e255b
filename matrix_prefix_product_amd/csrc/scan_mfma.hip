// Chunked look-back scans for n = 16 (fp64 running state) and n = 32 (fp32)
// on the CDNA matrix cores, one chain per wave.
//
// The chain keeps the TRANSPOSED state X = P^T in the MFMA accumulator layout
// and advances it as X_t = M_t^T X_{t-1}.  The accumulator layout, read as a B
// operand, is exactly the B layout of the same matrix once the k index of each
// k-block is permuted (block b, lane-row kk holds k = sigma(b, kk)), so the
// result of one step feeds the next step with no lane shuffles; the permutation
// is absorbed into which entries of M_t each lane loads (M_t comes from memory
// anyway).  Layouts used (gfx950, checked on the device by the parity pins):
//   v_mfma_f64_16x16x4_f64:  A[i][k] lane i+16k,  B[k][j] lane j+16k,
//                            D[i][j] lane j+16(i%4), reg i/4.
//   v_mfma_f32_32x32x2_f32:  A[i][k] lane i+32k,  B[k][j] lane j+32k,
//                            D[i][j] lane j+32((i/4)%2), reg 4(i/8)+i%4.
// For the f64 shape the accumulator interleaves rows across lane groups.  The
// chain relabels the state's row index with pi(i) = 4(i%4) + i/4 (a fixed
// permutation, applied to both the rows of X and the rows of A, so the algebra
// is unchanged); in actual indices every lane then again holds 4 contiguous
// entries of one row of P, and only the row index of each A-operand entry is
// permuted (Mf::acol).  Every P_t is written with 16-byte stores.
//
// Forward: "MRU Update: ...", section "What MRU Actually Does" (cumulative
// product, state times new input).  Backward: the gradient of
// sum_t <dP_t, P_t>, with G_t = Q_t^T = dP_t^T + M_{t+1} G_{t+1} advanced the
// same way and dM_t^T = G_t P_{t-1} taken through one LDS transpose of G_t.
#include "mru_device.h"
#include "mru_kernels.h"

namespace mru {
namespace {

typedef double d4 __attribute__((ext_vector_type(4)));
typedef float f16 __attribute__((ext_vector_type(16)));

template <int N>
struct Mf;

template <>
struct Mf<16> {
    using acc_t = double;
    using vec_t = d4;
    static constexpr int NR = 4;  // accumulator entries per lane
    static constexpr int NB = 4;  // k-blocks per 16x16x16 product
    // actual column of the state held by the lane; actual row of accumulator
    // entry r (also the k index of block b for this lane); actual row index of
    // the lane's A-operand entries
    __device__ static int col(int l) { return l & 15; }
    __device__ static int row(int l, int r) { return 4 * (l >> 4) + r; }
    __device__ static int acol(int l) { return 4 * (l & 3) + ((l & 15) >> 2); }
    __device__ static vec_t mfma(acc_t a, acc_t b, vec_t c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
};

template <>
struct Mf<32> {
    using acc_t = float;
    using vec_t = f16;
    static constexpr int NR = 16;
    static constexpr int NB = 16;
    __device__ static int col(int l) { return l & 31; }
    __device__ static int row(int l, int r) { return 8 * (r >> 2) + 4 * (l >> 5) + (r & 3); }
    __device__ static int acol(int l) { return l & 31; }
    __device__ static vec_t mfma(acc_t a, acc_t b, vec_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
};

// X <- A X + C for the transposed-state chain; a[b] is this lane's A-operand
// entry of k-block b, X's accumulator entry b is the matching B entry.
template <int N>
__device__ inline typename Mf<N>::vec_t chain_step(const typename Mf<N>::acc_t (&a)[Mf<N>::NB],
                                                   const typename Mf<N>::vec_t& X,
                                                   typename Mf<N>::vec_t acc) {
#pragma unroll
    for (int b = 0; b < Mf<N>::NB; ++b) acc = Mf<N>::mfma(a[b], X[b], acc);
    return acc;
}

template <int N>
__device__ inline typename Mf<N>::vec_t vzero() {
    typename Mf<N>::vec_t v;
#pragma unroll
    for (int r = 0; r < Mf<N>::NR; ++r) v[r] = 0;
    return v;
}

template <int N>
__device__ inline typename Mf<N>::vec_t videntity(int l) {
    typename Mf<N>::vec_t v;
#pragma unroll
    for (int r = 0; r < Mf<N>::NR; ++r) v[r] = (Mf<N>::row(l, r) == Mf<N>::col(l)) ? 1 : 0;
    return v;
}

// Accumulator entries r of a lane are row col(l), columns row(l, r) of the
// (untransposed) matrix; columns come in runs of 4.  Store / load that matrix
// row-major at `p`.
template <int N, class T>
__device__ inline void store_acc_rows(T* p, const typename Mf<N>::vec_t& X) {
    const int l = threadIdx.x & 63;
    const int c = Mf<N>::col(l);
#pragma unroll
    for (int r = 0; r < Mf<N>::NR; r += 4) {
        const int j = Mf<N>::row(l, r);
        if constexpr (sizeof(T) == 4) {
            *reinterpret_cast<float4*>(p + c * N + j) =
                make_float4(float(X[r]), float(X[r + 1]), float(X[r + 2]), float(X[r + 3]));
        } else {
            *reinterpret_cast<double2*>(p + c * N + j) = make_double2(X[r], X[r + 1]);
            *reinterpret_cast<double2*>(p + c * N + j + 2) = make_double2(X[r + 2], X[r + 3]);
        }
    }
}

template <int N, class T>
__device__ inline typename Mf<N>::vec_t load_acc_rows(const T* p) {
    const int l = threadIdx.x & 63;
    const int c = Mf<N>::col(l);
    typename Mf<N>::vec_t X;
#pragma unroll
    for (int r = 0; r < Mf<N>::NR; r += 4) {
        const int j = Mf<N>::row(l, r);
        if constexpr (sizeof(T) == 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + c * N + j);
            X[r] = v.x; X[r + 1] = v.y; X[r + 2] = v.z; X[r + 3] = v.w;
        } else {
            const double2 v0 = *reinterpret_cast<const double2*>(p + c * N + j);
            const double2 v1 = *reinterpret_cast<const double2*>(p + c * N + j + 2);
            X[r] = v0.x; X[r + 1] = v0.y; X[r + 2] = v1.x; X[r + 3] = v1.y;
        }
    }
    return X;
}

// A operand for X <- Y^T X, i.e. right multiplication of the untransposed
// state by Y (row-major at p): lane entry b = Y[row(l, b)][acol(l)].
template <int N, class T>
__device__ inline void load_a_transposed(typename Mf<N>::acc_t (&a)[Mf<N>::NB], const T* p) {
    const int l = threadIdx.x & 63;
    const int c = Mf<N>::acol(l);
#pragma unroll
    for (int b = 0; b < Mf<N>::NB; ++b) a[b] = typename Mf<N>::acc_t(p[Mf<N>::row(l, b) * N + c]);
}

// A operand for X <- Y X (left multiplication of the state by Y, row-major at
// p): lane entry b = Y[acol(l)][row(l, b)]; runs of 4 are contiguous.
template <int N, class T>
__device__ inline void load_a_direct(typename Mf<N>::acc_t (&a)[Mf<N>::NB], const T* p) {
    const int l = threadIdx.x & 63;
    const int c = Mf<N>::acol(l);
#pragma unroll
    for (int b = 0; b < Mf<N>::NB; b += 4) {
        const int j = Mf<N>::row(l, b);
        if constexpr (sizeof(T) == 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + c * N + j);
            a[b] = v.x; a[b + 1] = v.y; a[b + 2] = v.z; a[b + 3] = v.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) a[b + u] = typename Mf<N>::acc_t(p[c * N + j + u]);
        }
    }
}

struct Chunk {
    int64_t c;     // chunk index
    int64_t base;  // token index s*T + t0
    int64_t pos;   // k (forward) or nch-1-k (backward) within the sequence's chunk order
    int64_t t0;
    int len;
};

__device__ inline Chunk chunk_at(int64_t c, int64_t nch, int64_t K, int64_t T, bool reverse) {
    Chunk ch;
    ch.c = c;
    const int64_t s = c / nch;
    ch.pos = c - s * nch;
    const int64_t k = reverse ? nch - 1 - ch.pos : ch.pos;
    ch.t0 = k * K;
    ch.len = int(min(T, ch.t0 + K) - ch.t0);
    ch.base = s * T + ch.t0;
    return ch;
}

// ---------------------------------------------------------------------------- forward

template <int N, int PF, bool WRITE>
__device__ void fwd_sweep(typename Mf<N>::vec_t& X, const float* __restrict__ M,
                          float* __restrict__ P, int64_t base, int len) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    constexpr int NN = N * N;
    const int l = threadIdx.x & 63;
    const int ac = F::acol(l);
    int aoff[F::NB];
#pragma unroll
    for (int b = 0; b < F::NB; ++b) aoff[b] = F::row(l, b) * N + ac;
    float ring[PF][F::NB];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < len)
#pragma unroll
            for (int b = 0; b < F::NB; ++b) ring[p][b] = M[(base + p) * NN + aoff[b]];
    for (int t0 = 0; t0 < len; t0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int t = t0 + p;
            if (t < len) {
                acc_t a[F::NB];
#pragma unroll
                for (int b = 0; b < F::NB; ++b) a[b] = acc_t(ring[p][b]);
                if (t + PF < len)
#pragma unroll
                    for (int b = 0; b < F::NB; ++b)
                        ring[p][b] = M[(base + t + PF) * NN + aoff[b]];
                X = chain_step<N>(a, X, vzero<N>());
                if (WRITE) store_acc_rows<N, float>(P + (base + t) * NN, X);
            }
        }
    }
}

template <int N, int PF>
__global__ __launch_bounds__(64) void fwd_mfma_kernel(const float* __restrict__ M,
                                                      float* __restrict__ P, int64_t S, int64_t T,
                                                      int64_t K, int64_t nch, int64_t Z,
                                                      unsigned char* __restrict__ ws) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    using vec_t = typename F::vec_t;
    constexpr int NN = N * N;
    __shared__ acc_t xl[NN];
    const int l = threadIdx.x & 63;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    const int64_t cidx = multi ? int64_t(wave_ticket(&hdr->ticket)) : int64_t(blockIdx.x);
    if (cidx >= nchunks) return;
    const Chunk ch = chunk_at(cidx, nch, K, T, false);

    vec_t X = videntity<N>(l);
    if (!multi) {
        fwd_sweep<N, PF, true>(X, M, P, ch.base, ch.len);
        return;
    }
    const WsLayout L = ws_layout(nchunks, N, sizeof(acc_t), 2);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.flags_off);
    acc_t* agg = reinterpret_cast<acc_t*>(ws + L.slot_off[0]);
    acc_t* incl = reinterpret_cast<acc_t*>(ws + L.slot_off[1]);
    const int64_t c = ch.c;
    const int64_t k = ch.pos;
    const int64_t first = c - k % Z;

    // 1. chunk aggregate
    fwd_sweep<N, PF, false>(X, M, P, ch.base, ch.len);
    store_acc_rows<N, acc_t>(agg + c * NN, X);
    fence_release();
    if (l == 0) store_flag(&flags[c], kFlagAgg);

    // 2. Lt = (agg[first] ... agg[c-1])^T
    wait_range_nonempty(flags, first, c, hdr);
    fence_acquire();
    acc_t a[F::NB];
    X = videntity<N>(l);
    for (int64_t j = first; j < c; ++j) {
        load_a_transposed<N, acc_t>(a, agg + j * NN);
        X = chain_step<N>(a, X, vzero<N>());
    }

    // 3. carry^T = Lt * prefix^T, prefix from the previous super's last chunk
    if (k >= Z) {
        store_acc_rows<N, acc_t>(xl, X);  // L row-major
        wait_flag_eq(&flags[first - 1], kFlagPrefix, hdr);
        fence_acquire();
        __syncthreads();
        load_a_transposed<N, acc_t>(a, xl);
        X = chain_step<N>(a, load_acc_rows<N, acc_t>(incl + (first - 1) * NN), vzero<N>());
    }
    if (k % Z == Z - 1 && k + 1 < nch) {
        load_a_transposed<N, acc_t>(a, agg + c * NN);
        const vec_t inc = chain_step<N>(a, X, vzero<N>());
        store_acc_rows<N, acc_t>(incl + c * NN, inc);
        fence_release();
        if (l == 0) store_flag(&flags[c], kFlagPrefix);
    }

    // 4. re-run from the carry
    fwd_sweep<N, PF, true>(X, M, P, ch.base, ch.len);
}

// ---------------------------------------------------------------------------- backward

// Reverse sweep over the chunk (positions len-1 .. 0).
//   AGG:  G <- dP_t^T + M_{t+1} G from G = 0 and W <- M_{t+1} W from W = I.
//   GRAD: G <- dP_t^T + M_{t+1} G from the carry; dM_t^T = G_t P_{t-1}.
// At the last token of a sequence there is no M_{t+1}: G <- dP_t^T.
template <int N, int PF, bool GRAD>
__device__ void bwd_sweep(typename Mf<N>::vec_t& G, typename Mf<N>::vec_t& W,
                          const float* __restrict__ M, const float* __restrict__ P,
                          const float* __restrict__ dP, float* __restrict__ dM,
                          typename Mf<N>::acc_t* tr, int64_t base, int64_t t0, int len,
                          int64_t T) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    using vec_t = typename F::vec_t;
    constexpr int NN = N * N;
    constexpr int TS = N + 1;  // LDS row stride of the transpose buffer
    const int l = threadIdx.x & 63;
    const int c = F::col(l);
    const int ac = F::acol(l);
    int poff[F::NB];
#pragma unroll
    for (int b = 0; b < F::NB; ++b) poff[b] = F::row(l, b) * N + c;

    // ring of prefetched operands: M_{t+1} and dP_t (runs of 4 in row c), P_{t-1}
    float rm[PF][F::NB], rr[PF][F::NR], rp[PF][GRAD ? F::NB : 1];
    auto fetch = [&](int slot, int i) {
        const int pos = len - 1 - i;
        const int64_t tok = base + pos;
        const int64_t tseq = t0 + pos;
        if (tseq + 1 < T) {
#pragma unroll
            for (int b = 0; b < F::NB; b += 4) {
                const float4 v = *reinterpret_cast<const float4*>(M + (tok + 1) * NN + ac * N + F::row(l, b));
                rm[slot][b] = v.x; rm[slot][b + 1] = v.y; rm[slot][b + 2] = v.z; rm[slot][b + 3] = v.w;
            }
        }
#pragma unroll
        for (int r = 0; r < F::NR; r += 4) {
            const float4 v = *reinterpret_cast<const float4*>(dP + tok * NN + c * N + F::row(l, r));
            rr[slot][r] = v.x; rr[slot][r + 1] = v.y; rr[slot][r + 2] = v.z; rr[slot][r + 3] = v.w;
        }
        if constexpr (GRAD) {
            if (tseq > 0)
#pragma unroll
                for (int b = 0; b < F::NB; ++b) rp[slot][b] = P[(tok - 1) * NN + poff[b]];
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < len) fetch(p, p);
    for (int i0 = 0; i0 < len; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int i = i0 + p;
            if (i < len) {
                const int pos = len - 1 - i;
                const int64_t tok = base + pos;
                const int64_t tseq = t0 + pos;
                const bool has_next = tseq + 1 < T;
                acc_t a[F::NB];
                vec_t cr;
#pragma unroll
                for (int b = 0; b < F::NB; ++b) a[b] = acc_t(rm[p][b]);
#pragma unroll
                for (int r = 0; r < F::NR; ++r) cr[r] = acc_t(rr[p][r]);
                acc_t bp[F::NB];
                if constexpr (GRAD) {
#pragma unroll
                    for (int b = 0; b < F::NB; ++b) bp[b] = acc_t(rp[p][b]);
                }
                if (i + PF < len) fetch(p, i + PF);
                if (has_next) {
                    G = chain_step<N>(a, G, cr);
                    if (!GRAD) W = chain_step<N>(a, W, vzero<N>());
                } else {
                    G = cr;
                }
                if constexpr (GRAD) {
                    float* out = dM + tok * NN;
                    if (tseq > 0) {
                        // transpose G through LDS: A operand entry b = G[col][row(l, b)]
                        __syncthreads();
#pragma unroll
                        for (int r = 0; r < F::NR; ++r) tr[F::row(l, r) * TS + c] = G[r];
                        __syncthreads();
                        acc_t ag[F::NB];
#pragma unroll
                        for (int b = 0; b < F::NB; ++b) ag[b] = tr[ac * TS + F::row(l, b)];
                        vec_t bv;
#pragma unroll
                        for (int b = 0; b < F::NB; ++b) bv[b] = bp[b];
                        const vec_t D = chain_step<N>(ag, bv, vzero<N>());
                        store_acc_rows<N, float>(out, D);
                    } else {
                        store_acc_rows<N, float>(out, G);
                    }
                }
            }
        }
    }
}

template <int N, int PF>
__global__ __launch_bounds__(64) void bwd_mfma_kernel(const float* __restrict__ M,
                                                      const float* __restrict__ P,
                                                      const float* __restrict__ dP,
                                                      float* __restrict__ dM, int64_t S, int64_t T,
                                                      int64_t K, int64_t nch, int64_t Z,
                                                      unsigned char* __restrict__ ws) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    using vec_t = typename F::vec_t;
    constexpr int NN = N * N;
    __shared__ acc_t tr[N * (N + 1)];
    __shared__ acc_t xl[NN];
    const int l = threadIdx.x & 63;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    const int64_t cidx = multi ? int64_t(wave_ticket(&hdr->ticket)) : int64_t(blockIdx.x);
    if (cidx >= nchunks) return;
    const Chunk ch = chunk_at(cidx, nch, K, T, true);

    vec_t G = vzero<N>();
    vec_t W = videntity<N>(l);
    if (!multi) {
        bwd_sweep<N, PF, true>(G, W, M, P, dP, dM, tr, ch.base, ch.t0, ch.len, T);
        return;
    }
    // Chunks run in reverse token order (position r = 0 is the sequence's last
    // chunk).  Registers hold G = Q^T; a chunk's map is G -> W G + Bl (G form),
    // stored as the rows of W^T and of Bl^T = Q.
    const WsLayout L = ws_layout(nchunks, N, sizeof(acc_t), 3);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.flags_off);
    acc_t* swt = reinterpret_cast<acc_t*>(ws + L.slot_off[0]);
    acc_t* sbl = reinterpret_cast<acc_t*>(ws + L.slot_off[1]);
    acc_t* sinc = reinterpret_cast<acc_t*>(ws + L.slot_off[2]);
    const int64_t c = ch.c;
    const int64_t r = ch.pos;
    const int64_t first = c - r % Z;
    const bool later = r >= Z;

    // 1. affine aggregate
    bwd_sweep<N, PF, false>(G, W, M, P, dP, dM, tr, ch.base, ch.t0, ch.len, T);
    store_acc_rows<N, acc_t>(sbl + c * NN, G);
    store_acc_rows<N, acc_t>(swt + c * NN, W);
    fence_release();
    if (l == 0) store_flag(&flags[c], kFlagAgg);

    // 2. compose the maps of the earlier chunks of the super (first applied first)
    wait_range_nonempty(flags, first, c, hdr);
    fence_acquire();
    acc_t a[F::NB];
    vec_t WC = videntity<N>(l);
    G = vzero<N>();
    for (int64_t j = first; j < c; ++j) {
        load_a_transposed<N, acc_t>(a, swt + j * NN);  // A entries of W_j
        if (later) WC = chain_step<N>(a, WC, vzero<N>());
        G = chain_step<N>(a, G, load_acc_rows<N, acc_t>(sbl + j * NN));
    }

    // 3. carry = WC Y + BC with Y published by the previous super
    if (later) {
        store_acc_rows<N, acc_t>(xl, WC);  // rows of WC^T
        wait_flag_eq(&flags[first - 1], kFlagPrefix, hdr);
        fence_acquire();
        __syncthreads();
        load_a_transposed<N, acc_t>(a, xl);  // A entries of WC
        G = chain_step<N>(a, load_acc_rows<N, acc_t>(sinc + (first - 1) * NN), G);
    }
    if (r % Z == Z - 1 && r + 1 < nch) {
        load_a_transposed<N, acc_t>(a, swt + c * NN);
        const vec_t inc = chain_step<N>(a, G, load_acc_rows<N, acc_t>(sbl + c * NN));
        store_acc_rows<N, acc_t>(sinc + c * NN, inc);
        fence_release();
        if (l == 0) store_flag(&flags[c], kFlagPrefix);
    }

    // 4. re-run from the carry, writing dM
    bwd_sweep<N, PF, true>(G, W, M, P, dP, dM, tr, ch.base, ch.t0, ch.len, T);
}

template <int N, int PF>
hipError_t run_fwd(const float* M, float* P, int64_t S, int64_t T, int64_t K, int64_t nch,
                   int64_t Z, void* ws, hipStream_t stream) {
    hipLaunchKernelGGL((fwd_mfma_kernel<N, PF>), dim3(unsigned(S * nch)), dim3(64), 0, stream, M,
                       P, S, T, K, nch, Z, static_cast<unsigned char*>(ws));
    return hipGetLastError();
}

template <int N, int PF>
hipError_t run_bwd(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                   int64_t T, int64_t K, int64_t nch, int64_t Z, void* ws, hipStream_t stream) {
    hipLaunchKernelGGL((bwd_mfma_kernel<N, PF>), dim3(unsigned(S * nch)), dim3(64), 0, stream, M,
                       P, dP, dM, S, T, K, nch, Z, static_cast<unsigned char*>(ws));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const float* M, float* P, int64_t S, int64_t T, int n, int64_t K,
                           int64_t nch, int64_t Z, void* ws, hipStream_t stream) {
    if (n == 16) return run_fwd<16, 16>(M, P, S, T, K, nch, Z, ws, stream);
    if (n == 32) return run_fwd<32, 4>(M, P, S, T, K, nch, Z, ws, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                           int64_t T, int n, int64_t K, int64_t nch, int64_t Z, void* ws,
                           hipStream_t stream) {
    if (n == 16) return run_bwd<16, 8>(M, P, dP, dM, S, T, K, nch, Z, ws, stream);
    if (n == 32) return run_bwd<32, 2>(M, P, dP, dM, S, T, K, nch, Z, ws, stream);
    return hipErrorInvalidValue;
}

}  // namespace mru
