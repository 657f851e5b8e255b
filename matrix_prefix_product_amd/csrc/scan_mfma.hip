// Chunked look-back scans for n = 16 and n = 32 on the CDNA matrix cores, one
// chain per wave, with an fp64 running state (fp32 inputs and outputs).
//
// The chain keeps the TRANSPOSED state X = P^T in MFMA accumulator registers
// (the tile layout of mru_mfma.h) and advances it as X_t = M_t^T X_{t-1}: the
// accumulator feeds the next step as its B operand with no lane shuffles, the
// k permutation being absorbed into which entries of M_t each lane loads (M_t
// comes from memory anyway).  Every lane then holds 4 contiguous entries of
// one row of P per tile, and every P_t is written with 16-byte stores.
//
// The fp64 state is needed for accuracy, not range: the rounding error of an
// fp32 state is amplified by the misalignment of prefix and suffix products
// and reaches the 2e-4 relative error bound within a few thousand tokens at
// n = 16 and near the fp32 range limit at n = 32.
//
// Forward: "MRU Update: ...", section "What MRU Actually Does" (cumulative
// product, state times new input).  Backward: the gradient of
// sum_t <dP_t, P_t>, with G_t = Q_t^T = dP_t^T + M_{t+1} G_{t+1} advanced the
// same way and dM_t^T = G_t P_{t-1} taken through one LDS transpose of G_t.
#include <utility>

#include "mru_device.h"
#include "mru_kernels.h"
#include "mru_build.h"
#include "mru_mfma.h"

// Prefetch depth of the retained n = 16 aggregate pass (tokens in flight; the
// whole chunk is held in registers anyway, so depth costs no registers).
#ifndef MRU_PFR16
#define MRU_PFR16 16
#endif

namespace mru {
namespace {

// Scaled state (scaled forward scan): the accumulators hold S^T with
// P = 2^ex S.  renorm_acc multiplies S by a power of two (exact) so that its
// largest entry has magnitude in [0.5, 1) and adds the shift to ex (the same in
// every lane).  An all-zero S is left as it is.
template <int N>
__device__ inline void renorm_acc(typename Mf<N>::vec_t& X, int& ex) {
    int e = kNoExp;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) e = max_exp(e, X.t[I][J][r]);
    e = group_max<64>(e);
    if (e == kNoExp) return;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) X.t[I][J][r] = ldexp(X.t[I][J][r], -e);
    ex += e;
}

// Transposed carried-in state of sequence s (2^carry_exp * carry, or I).
template <int N, bool SC>
__device__ inline typename Mf<N>::vec_t init_acc(int& ex, const ScanCarry& cy, int64_t s) {
    const int l = threadIdx.x & 63;
    ex = 0;
    typename Mf<N>::vec_t X;
    if (!cy.carry) {
        X = videntity<N>(l);
    } else {
        X = load_acc_rows<N, float>(cy.carry + s * N * N);
        const int ce = cy.carry_exp ? cy.carry_exp[s] : 0;
        if (SC) {
            ex = ce;
        } else if (ce != 0) {
#pragma unroll
            for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
                for (int J = 0; J < Mf<N>::NT; ++J)
#pragma unroll
                    for (int r = 0; r < 4; ++r) X.t[I][J][r] = ldexp(X.t[I][J][r], ce);
        }
    }
    if constexpr (SC) renorm_acc<N>(X, ex);
    return X;
}

// Workspace (look-back) accessors: the same layouts as store_acc_rows /
// load_acc_rows / load_a_transposed, element by element through ws_store /
// ws_load so that other XCDs see them coherently.
template <int N>
__device__ inline void ws_store_acc_rows(double* p, const typename Mf<N>::vec_t& X) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) {
            double* q = p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) ws_store(q + r, X.t[I][J][r]);
        }
}

template <int N>
__device__ inline typename Mf<N>::vec_t ws_load_acc_rows(const double* p) {
    const int l = threadIdx.x & 63;
    typename Mf<N>::vec_t X;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) {
            const double* q = p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) X.t[I][J][r] = ws_load(q + r);
        }
    return X;
}

template <int N>
__device__ inline void ws_load_a_transposed(typename Mf<N>::aop_t& a, const double* p) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int K = 0; K < Mf<N>::NT; ++K)
#pragma unroll
            for (int b = 0; b < 4; ++b)
                a.v[I][K][b] = ws_load(p + (16 * K + trow(l, b)) * N + 16 * I + tacol(l));
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

// Aggregates fetched per batch in the look-back walk (bounded by registers).
template <int N, bool BWD>
constexpr int walk_depth() { return N == 16 ? 4 : (BWD ? 1 : 2); }

// ---------------------------------------------------------------------------- forward

// f(integral_constant<int, I>) for I = Is..., in order: a loop expanded at
// compile time whatever its body's size.
template <int... Is, class F>
__device__ inline void static_for(std::integer_sequence<int, Is...>, F&& f) {
    (f(std::integral_constant<int, Is>{}), ...);
}

// Operand staging of the forward chain.  The A operand of M_t^T needs, in lane
// l, 4 entries of one column of M_t (M_t[16K + trow(l, b)][16I + tacol(l)],
// b = 0..3), which row-major memory holds 4*n bytes apart.  Loading them
// directly takes 4-byte loads, and the 63 loads a wave may keep in flight then
// cover only 16 KB.  Instead the wave reads each token with 16-byte loads
// (row-major, n*n/256 per lane, 1 KB per wave instruction) and turns them into
// operands through LDS: the pieces are written transposed (M^T, row stride
// n+4), after which every lane's 4 entries are contiguous and come back in one
// 16-byte LDS read per tile.  Two LDS buffers alternate by token parity, so a
// single barrier per token orders both the writes before the reads and the
// previous use of a buffer before its next writes.
template <int N>
struct Stage {
    static constexpr int NV = N * N / 256;  // 16-byte pieces per lane per token
    static constexpr int LS = N + 4;        // LDS row stride of M^T (floats)
    static constexpr int BUF = N * LS;      // floats per LDS buffer
};

template <int N>
__device__ inline void load_token(float (&v)[4 * Stage<N>::NV], const float* tok) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < Stage<N>::NV; ++q) {
        float4 w;
        if constexpr (N == 16) {  // non-temporal at n = 16 (see store_prefix)
            typedef float f4v __attribute__((ext_vector_type(4)));
            const f4v u = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(tok) + q * 64 + l);
            w = make_float4(u.x, u.y, u.z, u.w);
        } else {
            w = reinterpret_cast<const float4*>(tok)[q * 64 + l];
        }
        v[4 * q] = w.x;
        v[4 * q + 1] = w.y;
        v[4 * q + 2] = w.z;
        v[4 * q + 3] = w.w;
    }
}

// Row-major pieces v of one token -> this lane's A-operand entries of M^T
// (index (I * NT + K) * 4 + b), through the LDS buffer tb.
template <int N>
__device__ inline void operand_write(const float (&v)[4 * Stage<N>::NV], float* tb) {
    constexpr int LS = Stage<N>::LS;
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < Stage<N>::NV; ++q) {
        const int f = q * 64 + l;           // float4 index within the token
        const int r = f / (N / 4);          // row of M
        const int c0 = 4 * (f % (N / 4));   // first column of the piece
#pragma unroll
        for (int j = 0; j < 4; ++j) tb[(c0 + j) * LS + r] = v[4 * q + j];
    }
}

template <int N>
__device__ inline void operand_read(float (&o)[4 * Stage<N>::NV], const float* tb) {
    constexpr int NT = N / 16;
    constexpr int LS = Stage<N>::LS;
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const float4 w =
                *reinterpret_cast<const float4*>(tb + (16 * I + tacol(l)) * LS + 16 * K + trow(l, 0));
            float* d = &o[(I * NT + K) * 4];
            d[0] = w.x; d[1] = w.y; d[2] = w.z; d[3] = w.w;
        }
}

template <int N>
__device__ inline void to_operand(float (&o)[4 * Stage<N>::NV], const float (&v)[4 * Stage<N>::NV],
                                  float* tb) {
    operand_write<N>(v, tb);
    __syncthreads();
    operand_read<N>(o, tb);
}

template <int N>
__device__ inline void operand_from(typename Mf<N>::aop_t& a, const float (&o)[4 * Stage<N>::NV]) {
    constexpr int NT = N / 16;
#pragma unroll
    for (int e = 0; e < 4 * Stage<N>::NV; ++e)
        a.v[e / (4 * NT)][(e / 4) % NT][e % 4] = double(o[e]);
}

// Forward from raw token vectors (n = 16, 32): the operand entries of M_t^T are
// formed from the staged x_t instead of read.  With X = x_t viewed row-major,
// M = Lt W where Lt is the unit lower factor (Lt_ik = X_ik for k < i, 1 on the
// diagonal) and W = diag(e) U (W_kc = e_k X_kc for k < c, e_k on the diagonal),
// e_k = exp(X_kk - mean_j X_jj) ("Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points: LDU fill, determinant-correcting
// scalar).  The product runs on the matrix core in fp32 (four
// v_mfma_f32_16x16x4f32, D[i][j] in lane j + 16(i/4), register i%4): taking
// W's columns in the order tacol, lane l's results are exactly its A-operand
// entries M[16K + trow(l, b)][16I + tacol(l)] of the fp64 chain.  Three phases,
// separated by barriers and spread between the chain's products:
//   stage:   every lane writes its 16-byte piece of X row-major to the slot;
//   factors: every lane reads X_kk for k = l%16, sums the 16 over its row of
//            lanes (DPP butterfly: each step adds two values in either order,
//            so every lane gets the same bits), forms e_{l%16}; lanes 0..15
//            write e to the slot;
//   read:    every lane reads its 4 entries of Lt and of W from X and e and
//            issues the four fp32 products.
// A slot (X, e) per token parity, as the transpose buffers.
template <int N>
struct StageX {
    static_assert(N == 16 || N == 32, "the forward from raw token vectors: n = 16, 32");
    static constexpr int LS = Stage<N>::LS;
    static constexpr int BUF = Stage<N>::BUF;
    static constexpr int SLOT = BUF + N;  // floats: X (row stride LS), e
};

template <int N>
__device__ inline void xop_stage(const float (&v)[4 * Stage<N>::NV], float* slot) {
    using SX = StageX<N>;
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < Stage<N>::NV; ++q) {
        const int f = q * 64 + l;  // float4 index within the token, as load_token
        *reinterpret_cast<float4*>(slot + (f / (N / 4)) * SX::LS + 4 * (f % (N / 4))) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    }
}

// Sum over each row of 16 lanes (quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror).
__device__ inline float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

template <int N>
__device__ inline void xop_factors(float* slot) {
    using SX = StageX<N>;
    constexpr int NT = N / 16;
    const int l = threadIdx.x & 63;
    float dsum = 0.f;  // X_kk for k = l%16 (+ 16, n = 32)
#pragma unroll
    for (int t = 0; t < NT; ++t) dsum += slot[((l & 15) + 16 * t) * (SX::LS + 1)];
    const float mean = row16_sum(dsum) * (1.0f / N);  // exact scaling by 1/n
    const int k = l & (N - 1);
    const float ek = expf(slot[k * (SX::LS + 1)] - mean);
    if (l < N) slot[SX::BUF + l] = ek;
}

// Operand entries o[(I * NT + K) * 4 + b] = M[16K + trow(l, b)][16I + tacol(l)]:
// output tile (K, I) of Lt W with W's columns in the order tacol, summing the
// k-tiles T <= min(K, I) (the others are zero).
template <int N>
__device__ inline void xop_read(float (&o)[4 * Stage<N>::NV], const float* slot) {
    using SX = StageX<N>;
    constexpr int NT = N / 16;
    typedef float f4 __attribute__((ext_vector_type(4)));
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const int i = 16 * K + (l & 15);  // row of Lt this lane supplies (A operand)
            const int c = 16 * I + tacol(l);  // column of W this lane supplies (B operand)
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int T = 0; T <= (K < I ? K : I); ++T)
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int k = 16 * T + 4 * s4 + (l >> 4);
                    const float xik = slot[i * SX::LS + k];
                    const float xkc = slot[k * SX::LS + c];
                    const float ek = slot[SX::BUF + k];
                    const float a = k < i ? xik : (k == i ? 1.f : 0.f);
                    const float b = c > k ? ek * xkc : (c == k ? ek : 0.f);
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) o[(I * NT + K) * 4 + r] = acc[r];
        }
}

// Floats per token-parity slot of the forward from raw token vectors (0 otherwise).
template <int N, bool FX>
constexpr int xslot() {
    if constexpr (FX) return StageX<N>::SLOT;
    else return 0;
}

// The three phases back to back (a chunk's first token).
template <int N>
__device__ inline void to_operand_x(float (&o)[4 * Stage<N>::NV], const float (&v)[4 * Stage<N>::NV],
                                    float* slot) {
    xop_stage<N>(v, slot);
    __syncthreads();
    xop_factors<N>(slot);
    __syncthreads();
    xop_read<N>(o, slot);
}

// Software pipelining of the forward chain.  Instructions issue in order, and
// each of a token's products waits at issue for the previous one's
// accumulator, so anything placed after them would only start once the last
// has been issued.  Each step therefore spreads the work that does not depend
// on its products between them (chain_step_with): token t+1's operand goes
// through LDS (write after the first product, read after the second), token
// t-1's prefix is stored after the third and a load is refilled after the
// fourth, all while the matrix core runs.  (Measured against doing that work
// after the last product: C3 forward 371-376 -> 351-352 us, C5 forward
// 194-195 -> 179-184 us, bitwise the same results.)

template <int N, bool SC>
__device__ inline void store_prefix(float* __restrict__ P, int32_t* __restrict__ pexp, int64_t tok,
                                    const typename Mf<N>::vec_t& X, int ex) {
    // n = 16: the prefixes are streamed out non-temporally, as the inputs are
    // read (load_token): C3 forward 321 -> 286 us, C5 forward (between backwards)
    // 169 -> 162 us; at n = 32 either made the forward slower: ordinary accesses
    if constexpr (N == 16) store_acc_rows_nt<N>(P + tok * Mf<N>::NN, X);
    else store_acc_rows<N, float>(P + tok * Mf<N>::NN, X);
    if (SC && (threadIdx.x & 63) == 0) pexp[tok] = ex;
}

// The operand ring: PF tokens of loads stay in flight; a slot is refilled (with
// the token PF further on, address clamped into the chunk) as soon as its
// pieces have been turned into operands.  The main loop runs whole blocks of PF
// tokens so every ring slot stays in fixed registers.
template <int N, int PF, bool WRITE, bool FX, bool SC>
__device__ __attribute__((always_inline)) void fwd_sweep(typename Mf<N>::vec_t& X, int& ex, const float* __restrict__ M,
                          float* __restrict__ P, int32_t* __restrict__ pexp, int64_t base, int len,
                          float* tlds, float* xlds) {
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
    constexpr int NN = F::NN;
    constexpr int NA = 4 * Stage<N>::NV;  // A-operand entries per token and lane
    if (len <= 0) return;
    const float* Mb = M + base * NN;
    float ring[PF][NA];
#pragma unroll
    for (int p = 0; p < PF; ++p) load_token<N>(ring[p], Mb + int64_t(min(p, len - 1)) * NN);
    float o[NA];  // operands of the next token to multiply
    if constexpr (FX) {
        // Two deep: token t+1's operand is read at the start of step t from
        // factors written (and fenced) during step t-1, and token t+2 is staged
        // and factored during step t, so no LDS round trip waits in the step.
        // The ring then holds tokens t+2 .. t+1+PF at the start of step t.
        static_assert(PF >= 3, "two tokens ahead of the chain");
        to_operand_x<N>(o, ring[0], xlds);
        if (len > 1) {
            float* x1 = xlds + xslot<N, FX>();
            xop_stage<N>(ring[1], x1);
            __syncthreads();
            xop_factors<N>(x1);
            __syncthreads();
        }
        load_token<N>(ring[0], Mb + int64_t(min(PF, len - 1)) * NN);
        load_token<N>(ring[1], Mb + int64_t(min(PF + 1, len - 1)) * NN);
    } else {
        to_operand<N>(o, ring[0], tlds);
        load_token<N>(ring[0], Mb + int64_t(min(PF, len - 1)) * NN);
    }
    auto step = [&](int p, int t, bool refill) {
        typename F::aop_t a;
        operand_from<N>(a, o);
        vec_t Xn;
        if constexpr (FX) {
            const int p2 = (p + 2) % PF;  // ring slot of token t + 2
            float* x1 = xlds + ((t + 1) & 1) * xslot<N, FX>();
            float* x2 = xlds + (t & 1) * xslot<N, FX>();  // token t + 2's slot
            Xn = chain_step_with<N>(a, X, vzero<N>(), [&](int k) {
                if (k == 0 && t + 1 < len) xop_read<N>(o, x1);
                if (k == 1 && t + 2 < len) xop_stage<N>(ring[p2], x2);
                if (k == 2) {
                    if (WRITE && t > 0) store_prefix<N, SC>(P, pexp, base + t - 1, X, ex);
                    if (t + 2 < len) {
                        __syncthreads();
                        xop_factors<N>(x2);
                    }
                }
                if (k == 3 && t + 2 < len) {
                    __syncthreads();
                    if (refill) load_token<N>(ring[p2], Mb + int64_t(min(t + 2 + PF, len - 1)) * NN);
                }
            });
        } else {
            const int pn = (p + 1) % PF;  // ring slot of token t + 1
            float* tb = tlds + ((t + 1) & 1) * Stage<N>::BUF;
            // token t+1's operand goes through LDS while token t's products run
            Xn = chain_step_with<N>(a, X, vzero<N>(), [&](int k) {
                if (k == 0 && t + 1 < len) operand_write<N>(ring[pn], tb);
                if (k == 1 && t + 1 < len) {
                    __syncthreads();
                    operand_read<N>(o, tb);
                }
                if (k == 2 && WRITE && t > 0) store_prefix<N, SC>(P, pexp, base + t - 1, X, ex);
                if (k == 3 && t + 1 < len && refill)
                    load_token<N>(ring[pn], Mb + int64_t(min(t + 1 + PF, len - 1)) * NN);
            });
        }
        __builtin_amdgcn_sched_barrier(0);
        X = Xn;
        if constexpr (SC) renorm_acc<N>(X, ex);
    };
    int t0 = 0;
    for (; t0 + PF <= len; t0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) step(p, t0 + p, true);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (t0 + p < len) step(p, t0 + p, false);
    if (WRITE) store_prefix<N, SC>(P, pexp, base + len - 1, X, ex);
}

// Retained chunk (KR > 0): the aggregate pass loads the chunk's tokens into a
// register buffer of KR tokens (loads issued PF tokens ahead, clamped into the
// chunk), converts each to its operand entries in place, and the apply pass
// reuses them, so each input matrix is read from HBM once even when the chunk
// needs a carry.
template <int N, int KR, int PF, bool FX, bool SC>
__device__ __attribute__((always_inline)) void fwd_pass_retain(typename Mf<N>::vec_t& X, int& ex, const float* __restrict__ M,
                                int64_t base, int len, float (&buf)[KR][4 * Stage<N>::NV],
                                float* tlds, float* xlds) {
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
    constexpr int NN = F::NN;
    constexpr int NA = 4 * Stage<N>::NV;
    if (len <= 0) return;
    const float* Mb = M + base * NN;
#pragma unroll
    for (int p = 0; p < PF && p < KR; ++p) load_token<N>(buf[p], Mb + int64_t(min(p, len - 1)) * NN);
    {
        float o[NA];
        if constexpr (FX) to_operand_x<N>(o, buf[0], xlds);
        else to_operand<N>(o, buf[0], tlds);
#pragma unroll
        for (int e = 0; e < NA; ++e) buf[0][e] = o[e];
    }
    if constexpr (FX && KR > 1) {
        // two deep, as in fwd_sweep: token 1 is staged and factored before the
        // first step, token t+2 during step t, token t+1's operand read in step t
        static_assert(PF >= 3, "two tokens ahead of the chain");
        if (len > 1) {
            float* x1 = xlds + xslot<N, FX>();
            xop_stage<N>(buf[1], x1);
            __syncthreads();
            xop_factors<N>(x1);
            __syncthreads();
        }
    }
    // expanded at compile time (an index sequence, not the loop unroller: with
    // the forward from raw token vectors the body outgrows the unroller's size
    // limit, and a rolled loop would index buf, moving it to scratch memory)
    static_for(std::make_integer_sequence<int, KR>{}, [&](auto tc) {
        constexpr int t = decltype(tc)::value;
        if constexpr (t + PF < KR) load_token<N>(buf[t + PF], Mb + int64_t(min(t + PF, len - 1)) * NN);
        __builtin_amdgcn_sched_barrier(0);
        if (t < len) {
            typename F::aop_t a;
            operand_from<N>(a, buf[t]);
            float* tb = tlds + ((t + 1) & 1) * Stage<N>::BUF;
            float* xb = xlds + ((t + 1) & 1) * xslot<N, FX>();
            const bool next = t + 1 < KR && t + 1 < len;
            vec_t Xn = chain_step_with<N>(a, X, vzero<N>(), [&](int k) {
                if constexpr (t + 1 < KR) {  // buf[t + 1] exists
                    if constexpr (FX) {
                        if (k == 0 && next) {
                            float o[NA];
                            xop_read<N>(o, xb);
#pragma unroll
                            for (int e = 0; e < NA; ++e) buf[t + 1][e] = o[e];
                        }
                        if constexpr (t + 2 < KR) {  // buf[t + 2] exists
                            float* x2 = xlds + (t & 1) * xslot<N, FX>();
                            const bool next2 = t + 2 < len;
                            if (k == 1 && next2) xop_stage<N>(buf[t + 2], x2);
                            if (k == 2 && next2) {
                                __syncthreads();
                                xop_factors<N>(x2);
                            }
                            if (k == 3 && next2) __syncthreads();
                        }
                    } else {
                        if (k == 0 && next) operand_write<N>(buf[t + 1], tb);
                        if (k == 1 && next) {
                            float o[NA];
                            __syncthreads();
                            operand_read<N>(o, tb);
#pragma unroll
                            for (int e = 0; e < NA; ++e) buf[t + 1][e] = o[e];
                        }
                    }
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            X = Xn;
            if constexpr (SC) renorm_acc<N>(X, ex);
        }
    });
}

template <int N, int KR, bool SC>
__device__ __attribute__((always_inline)) void fwd_apply_retain(typename Mf<N>::vec_t& X, int& ex, float* __restrict__ P,
                                 int32_t* __restrict__ pexp, int64_t base, int len,
                                 const float (&buf)[KR][4 * Stage<N>::NV]) {
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
#pragma unroll
    for (int t = 0; t < KR; ++t) {
        if (t < len) {
            typename F::aop_t a;
            operand_from<N>(a, buf[t]);
            vec_t Xn = chain_step_with<N>(a, X, vzero<N>(), [&](int k) {
                if (k == 0 && t > 0) store_prefix<N, SC>(P, pexp, base + t - 1, X, ex);
            });
            __builtin_amdgcn_sched_barrier(0);
            X = Xn;
            if constexpr (SC) renorm_acc<N>(X, ex);
        }
    }
    if (len > 0) store_prefix<N, SC>(P, pexp, base + len - 1, X, ex);
}

// Waves per SIMD the forward kernel is register-budgeted for (tuning knob).
#ifndef MRU_MFMA_FWD_WAVES
#define MRU_MFMA_FWD_WAVES 1
#endif

template <int N, int PF, int KR, bool FX, bool SC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(MRU_MFMA_FWD_WAVES)))
void fwd_mfma_kernel(const float* __restrict__ M,
                                                      float* __restrict__ P, int64_t S, int64_t T,
                                                      int64_t K, int64_t nch, int64_t Z,
                                                      unsigned char* __restrict__ ws, ScanCarry cy) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    using vec_t = typename F::vec_t;
    constexpr int NN = N * N;
    __shared__ double xl[NN];
    __shared__ __align__(16) float tlds[2 * Stage<N>::BUF];
    __shared__ __align__(16) float xlds[FX ? 2 * xslot<N, FX>() : 4];  // FX: the token factors
    const int l = threadIdx.x & 63;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    const int64_t cidx =
        multi ? ticket_to_chunk(int64_t(wave_ticket(&hdr->ticket)), S, nch, 1) : int64_t(blockIdx.x);
    if (cidx >= nchunks) return;
    const Chunk ch = chunk_at(cidx, nch, K, T, false);
    const int64_t seq = cidx / nch;

    int ex = 0;
    if (!multi) {
        vec_t X = init_acc<N, SC>(ex, cy, seq);
        fwd_sweep<N, PF, true, FX, SC>(X, ex, M, P, cy.out_exp, ch.base, ch.len, tlds, xlds);
        return;
    }
    const WsLayout L = ws_layout(nchunks, N, sizeof(acc_t), 2);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.flags_off);
    acc_t* agg = reinterpret_cast<acc_t*>(ws + L.slot_off[0]);
    acc_t* incl = reinterpret_cast<acc_t*>(ws + L.slot_off[1]);
    int32_t* agg_exp = reinterpret_cast<int32_t*>(ws + L.exp_off);
    int32_t* incl_exp = agg_exp + nchunks;
    const int64_t c = ch.c;
    const int64_t k = ch.pos;
    const int64_t first = c - k % Z;

    // 1. chunk aggregate (scaled scans: 2^a_ex times the normalised matrix)
    vec_t X = videntity<N>(l);
    float buf[KR > 0 ? KR : 1][Mf<N>::NT * Mf<N>::NT * 4];
    if constexpr (KR > 0)
        fwd_pass_retain<N, KR, (N == 16 ? MRU_PFR16 : PF), FX, SC>(X, ex, M, ch.base, ch.len, buf, tlds, xlds);
    else
        fwd_sweep<N, PF, false, FX, SC>(X, ex, M, P, cy.out_exp, ch.base, ch.len, tlds, xlds);
    const int a_ex = ex;
    ws_store_acc_rows<N>(agg + c * NN, X);
    if (SC && l == 0) ws_store(&agg_exp[c], int32_t(a_ex));
    fence_release();
    if (l == 0) store_flag(&flags[c], kFlagAgg);

    // 2. Lt = (agg[first] ... agg[c-1])^T
    wait_range_nonempty(flags, first, c, hdr);
    fence_acquire();
    typename F::aop_t a;
    X = videntity<N>(l);
    int l_ex = 0;
    // aggregates are loaded kWalk at a time so their loads are in flight together
    constexpr int kWalk = walk_depth<N, false>();
    for (int64_t j0 = first; j0 < c; j0 += kWalk) {
        typename F::aop_t w[kWalk];
#pragma unroll
        for (int d = 0; d < kWalk; ++d)
            if (j0 + d < c) ws_load_a_transposed<N>(w[d], agg + (j0 + d) * NN);
#pragma unroll
        for (int d = 0; d < kWalk; ++d)
            if (j0 + d < c) {
                X = chain_step<N>(w[d], X, vzero<N>());
                if constexpr (SC) {
                    l_ex += ws_load(&agg_exp[j0 + d]);
                    renorm_acc<N>(X, l_ex);
                }
            }
    }

    // 3. carry^T = Lt * prefix^T, prefix from the previous super's last chunk
    //    (first super: the carried-in state, if any)
    if (k >= Z || cy.carry) {
        store_acc_rows<N, acc_t>(xl, X);  // L row-major
        vec_t pre;
        if (k >= Z) {
            wait_flag_eq(&flags[first - 1], kFlagPrefix, hdr);
            fence_acquire();
            pre = ws_load_acc_rows<N>(incl + (first - 1) * NN);
            ex = SC ? ws_load(&incl_exp[first - 1]) : 0;
        } else {
            pre = init_acc<N, SC>(ex, cy, seq);
        }
        __syncthreads();
        load_a_transposed<N, acc_t>(a, xl);
        X = chain_step<N>(a, pre, vzero<N>());
        if constexpr (SC) {
            ex += l_ex;
            renorm_acc<N>(X, ex);
        }
    } else {
        ex = l_ex;
    }
    if (k % Z == Z - 1 && k + 1 < nch) {
        ws_load_a_transposed<N>(a, agg + c * NN);
        vec_t inc = chain_step<N>(a, X, vzero<N>());
        int i_ex = ex + a_ex;
        if constexpr (SC) renorm_acc<N>(inc, i_ex);
        ws_store_acc_rows<N>(incl + c * NN, inc);
        if (SC && l == 0) ws_store(&incl_exp[c], int32_t(i_ex));
        fence_release();
        if (l == 0) store_flag(&flags[c], kFlagPrefix);
    }

    // 4. re-run from the carry
    if constexpr (KR > 0)
        fwd_apply_retain<N, KR, SC>(X, ex, P, cy.out_exp, ch.base, ch.len, buf);
    else
        fwd_sweep<N, PF, true, FX, SC>(X, ex, M, P, cy.out_exp, ch.base, ch.len, tlds, xlds);
}

// ---------------------------------------------------------------------------- backward

// Reverse sweep over the chunk (positions len-1 .. 0).
//   AGG:  G <- dP_t^T + M_{t+1} G from G = 0 and W <- M_{t+1} W from W = I.
//   GRAD: G <- dP_t^T + M_{t+1} G from the carry; dM_t^T = G_t P_{t-1}.
// At the last token of a sequence there is no M_{t+1}: G <- dP_t^T.
template <int N, int PF, bool GRAD>
__device__ void bwd_sweep(typename Mf<N>::vec_t& G, typename Mf<N>::vec_t& W,
                          const float* __restrict__ M, const float* __restrict__ P,
                          const float* __restrict__ dP, float* __restrict__ dM, double* tr,
                          int64_t base, int64_t t0, int len, int64_t T, const ScanCarry& cy) {
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
    constexpr int NT = F::NT;
    constexpr int NN = F::NN;
    constexpr int NA = NT * NT * 4;
    constexpr int TS = N + 1;  // LDS row stride of the transpose buffer
    if (len <= 0) return;
    const int l = threadIdx.x & 63;
    const int c = tcol(l);
    const int ac = tacol(l);
    // positions relative to the chunk start whose loads are always in bounds:
    // M_{t+1} exists for pos < hi_m, P_{t-1} for pos >= lo_p
    const int hi_m = int(min<int64_t>(len, T - 1 - t0));  // pos + 1 + t0 < T
    const int lo_p = t0 > 0 ? 0 : 1;                      // pos - 1 + t0 >= 0
    const float* Mb = M + base * NN;
    const float* Pb = P + base * NN;
    const float* Rb = dP + base * NN;

    // ring of prefetched operands per token: M_{t+1} (A operand, runs of 4),
    // dP_t (C operand, runs of 4), P_{t-1} (B operand of the dM product).  (Read
    // non-temporally the backward was faster launch after launch, but slower
    // right after the forward, as in a training step: ordinary accesses.)
    float rm[PF][NA], rr[PF][NA], rp[PF][GRAD ? NA : 1];
    auto fetch = [&](int slot, int i) {
        const int pos = max(len - 1 - i, 0);
        const int pm = min(pos, hi_m - 1) + 1;  // clamped: only used when pos < hi_m
#pragma unroll
        for (int I = 0; I < NT; ++I)
#pragma unroll
            for (int K = 0; K < NT; ++K) {
                const float4 v = *reinterpret_cast<const float4*>(
                    Mb + int64_t(hi_m > 0 ? pm : pos) * NN + (16 * I + ac) * N + 16 * K + trow(l, 0));
                float* d = &rm[slot][(I * NT + K) * 4];
                d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
            }
#pragma unroll
        for (int I = 0; I < NT; ++I)
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                const float4 v = *reinterpret_cast<const float4*>(
                    Rb + int64_t(pos) * NN + (16 * J + c) * N + 16 * I + trow(l, 0));
                float* d = &rr[slot][(I * NT + J) * 4];
                d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
            }
        if constexpr (GRAD) {
            const int pp = max(pos, lo_p) - 1;  // clamped: only used when pos >= lo_p
#pragma unroll
            for (int K = 0; K < NT; ++K)
#pragma unroll
                for (int J = 0; J < NT; ++J)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        rp[slot][(K * NT + J) * 4 + b] =
                            Pb[int64_t(pp) * NN + (16 * K + trow(l, b)) * N + 16 * J + c];
        }
    };
    auto step = [&](int p, int i, bool refill) {
        const int pos = len - 1 - i;
        const bool has_next = pos < hi_m;
        typename F::aop_t a;
        vec_t cr, bv;
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            a.v[e / (4 * NT)][(e / 4) % NT][e % 4] = double(rm[p][e]);
            cr.t[e / (4 * NT)][(e / 4) % NT][e % 4] = double(rr[p][e]);
        }
        if constexpr (GRAD) {
#pragma unroll
            for (int e = 0; e < NA; ++e) bv.t[e / (4 * NT)][(e / 4) % NT][e % 4] = double(rp[p][e]);
        }
        if (refill) fetch(p, i + PF);
        if (has_next) {
            G = chain_step<N>(a, G, cr);
            if constexpr (!GRAD) W = chain_step<N>(a, W, vzero<N>());
        } else {
            G = cr;
        }
        if constexpr (GRAD) {
            float* out = dM + (base + pos) * NN;
            const int64_t s0 = base - t0;  // token index of the sequence's first token
            if (pos < lo_p && cy.carry) {
                // t = 0 with a carried-in state: P_{-1} = carry (B operand layout)
                const float* cs = cy.carry + (s0 / T) * NN;
#pragma unroll
                for (int K = 0; K < NT; ++K)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            bv.t[K][J][b] = double(cs[(16 * K + trow(l, b)) * N + 16 * J + c]);
            }
            if (pos >= lo_p || cy.carry) {
                // transpose G through LDS: A entries of G are G[16I + acol][16K + trow(l, b)]
                __syncthreads();
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            tr[(16 * I + trow(l, r)) * TS + 16 * J + c] = G.t[I][J][r];
                __syncthreads();
                typename F::aop_t ag;
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int K = 0; K < NT; ++K)
#pragma unroll
                        for (int b = 0; b < 4; ++b)
                            ag.v[I][K][b] = tr[(16 * I + ac) * TS + 16 * K + trow(l, b)];
                const vec_t D = chain_step<N>(ag, bv, vzero<N>());
                store_acc_rows<N, float>(out, D);
            } else {
                store_acc_rows<N, float>(out, G);  // t = 0: P_{-1} = I
            }
            if (pos < lo_p && cy.dcarry) {
                // dL/dP_{-1} = Q_0 M_0^T, i.e. its transpose is M_0 G_0
                typename F::aop_t am;
                load_a_direct<N, float>(am, Mb + int64_t(pos) * NN);
                store_acc_rows<N, float>(cy.dcarry + (s0 / T) * NN, chain_step<N>(am, G, vzero<N>()));
            }
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) fetch(p, min(p, len - 1));
    int i0 = 0;
    for (; i0 + PF <= len; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) step(p, i0 + p, true);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (i0 + p < len) step(p, i0 + p, false);
}

template <int N, int PF>
__global__ __launch_bounds__(64) void bwd_mfma_kernel(const float* __restrict__ M,
                                                      const float* __restrict__ P,
                                                      const float* __restrict__ dP,
                                                      float* __restrict__ dM, int64_t S, int64_t T,
                                                      int64_t K, int64_t nch, int64_t Z,
                                                      unsigned char* __restrict__ ws, ScanCarry cy) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    using vec_t = typename F::vec_t;
    constexpr int NN = N * N;
    __shared__ double tr[N * (N + 1)];
    __shared__ double xl[NN];
    const int l = threadIdx.x & 63;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    const int64_t cidx =
        multi ? ticket_to_chunk(int64_t(wave_ticket(&hdr->ticket)), S, nch, 1) : int64_t(blockIdx.x);
    if (cidx >= nchunks) return;
    const Chunk ch = chunk_at(cidx, nch, K, T, true);

    vec_t G = vzero<N>();
    vec_t W = videntity<N>(l);
    if (!multi) {
        bwd_sweep<N, PF, true>(G, W, M, P, dP, dM, tr, ch.base, ch.t0, ch.len, T, cy);
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
    bwd_sweep<N, PF, false>(G, W, M, P, dP, dM, tr, ch.base, ch.t0, ch.len, T, cy);
    ws_store_acc_rows<N>(sbl + c * NN, G);
    ws_store_acc_rows<N>(swt + c * NN, W);
    fence_release();
    if (l == 0) store_flag(&flags[c], kFlagAgg);

    // 2. compose the maps of the earlier chunks of the super (first applied first)
    wait_range_nonempty(flags, first, c, hdr);
    fence_acquire();
    typename F::aop_t a;
    vec_t WC = videntity<N>(l);
    G = vzero<N>();
    constexpr int kWalk = walk_depth<N, true>();
    for (int64_t j0 = first; j0 < c; j0 += kWalk) {
        typename F::aop_t w[kWalk];
        vec_t bl[kWalk];
#pragma unroll
        for (int d = 0; d < kWalk; ++d)
            if (j0 + d < c) {
                ws_load_a_transposed<N>(w[d], swt + (j0 + d) * NN);  // A entries of W_j
                bl[d] = ws_load_acc_rows<N>(sbl + (j0 + d) * NN);
            }
#pragma unroll
        for (int d = 0; d < kWalk; ++d)
            if (j0 + d < c) {
                if (later) WC = chain_step<N>(w[d], WC, vzero<N>());
                G = chain_step<N>(w[d], G, bl[d]);
            }
    }

    // 3. carry = WC Y + BC with Y published by the previous super
    if (later) {
        store_acc_rows<N, acc_t>(xl, WC);  // rows of WC^T
        wait_flag_eq(&flags[first - 1], kFlagPrefix, hdr);
        fence_acquire();
        __syncthreads();
        load_a_transposed<N, acc_t>(a, xl);  // A entries of WC
        G = chain_step<N>(a, ws_load_acc_rows<N>(sinc + (first - 1) * NN), G);
    }
    if (r % Z == Z - 1 && r + 1 < nch) {
        ws_load_a_transposed<N>(a, swt + c * NN);
        const vec_t inc = chain_step<N>(a, G, ws_load_acc_rows<N>(sbl + c * NN));
        ws_store_acc_rows<N>(sinc + c * NN, inc);
        fence_release();
        if (l == 0) store_flag(&flags[c], kFlagPrefix);
    }

    // 4. re-run from the carry, writing dM
    bwd_sweep<N, PF, true>(G, W, M, P, dP, dM, tr, ch.base, ch.t0, ch.len, T, cy);
}

template <int N, int PF, int KR, bool FX>
hipError_t run_fwd(const float* M, float* P, int64_t S, int64_t T, int64_t K, int64_t nch,
                   int64_t Z, void* ws, hipStream_t stream, const ScanCarry& cy) {
    if (cy.out_exp)
        hipLaunchKernelGGL((fwd_mfma_kernel<N, PF, KR, FX, true>), dim3(unsigned(S * nch)), dim3(64),
                           0, stream, M, P, S, T, K, nch, Z, static_cast<unsigned char*>(ws), cy);
    else
        hipLaunchKernelGGL((fwd_mfma_kernel<N, PF, KR, FX, false>), dim3(unsigned(S * nch)), dim3(64),
                           0, stream, M, P, S, T, K, nch, Z, static_cast<unsigned char*>(ws), cy);
    return hipGetLastError();
}

template <int N, int PF>
hipError_t run_bwd(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                   int64_t T, int64_t K, int64_t nch, int64_t Z, void* ws, hipStream_t stream,
                   const ScanCarry& cy) {
    hipLaunchKernelGGL((bwd_mfma_kernel<N, PF>), dim3(unsigned(S * nch)), dim3(64), 0, stream, M,
                       P, dP, dM, S, T, K, nch, Z, static_cast<unsigned char*>(ws), cy);
    return hipGetLastError();
}

}  // namespace

#ifndef MRU_RETAIN16
#define MRU_RETAIN16 64
#endif
#ifndef MRU_PF16
#define MRU_PF16 16
#endif
// Tokens of one chunk kept in registers by the n = 16 forward kernel.
constexpr int kRetain16 = MRU_RETAIN16;

int mfma_retain_tokens(int n) { return n == 16 ? kRetain16 : 0; }

hipError_t launch_fwd_mfma(const float* M, float* P, int64_t S, int64_t T, int n, int64_t K,
                           int64_t nch, int64_t Z, void* ws, hipStream_t stream, bool from_x,
                           const ScanCarry& cy) {
    if (n == 16) {
        const bool retain = kRetain16 > 0 && nch > 1 && K <= kRetain16;
        if (from_x) {
            if (retain) return run_fwd<16, MRU_PF16, kRetain16, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
            return run_fwd<16, MRU_PF16, 0, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
        }
        if (retain) return run_fwd<16, MRU_PF16, kRetain16, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
        return run_fwd<16, MRU_PF16, 0, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
    }
    if (n == 32) {
        if (from_x) return run_fwd<32, 4, 0, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
        return run_fwd<32, 4, 0, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                           int64_t T, int n, int64_t K, int64_t nch, int64_t Z, void* ws,
                           hipStream_t stream, const ScanCarry& cy) {
    if (n == 16) return run_bwd<16, 8>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
    if (n == 32) return run_bwd<32, 2>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
    return hipErrorInvalidValue;
}

}  // namespace mru
