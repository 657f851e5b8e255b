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
#include "mru_build_mfma.h"
#include "mru_mfma.h"

// Prefetch depth of the retained n = 16 aggregate pass (tokens in flight; the
// whole chunk is held in registers anyway, so depth costs no registers).
constexpr int kPfRetain16 = 16;

namespace mru {
namespace {

typedef float f4v32 __attribute__((ext_vector_type(4)));

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
    wave_lds_sync();
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
// scalar).  The product runs on the matrix core in fp64 and is rounded once to
// fp32, exactly as the build kernel forms M (ldu_tile_f64): taking M's rows in
// the order pi and its columns in the order tacol, lane l's results are
// exactly its A-operand entries M[16K + trow(l, b)][16I + tacol(l)] of the fp64
// chain.  Three phases, separated by barriers and spread between the chain's
// products:
//   stage:   every lane writes its 16-byte piece of X row-major to the slot;
//   factors: every lane sums X_kk in fp64 over its 16-lane row (DPP butterfly:
//            each step adds two values in either order, so every lane gets the
//            same bits) and forms e; lanes 0..n-1 write e to the slot (fp64,
//            and rounded to fp32 for the gradient's fp32 arithmetic);
//   read:    every lane reads its entries of Lt and of W from X and e and
//            issues the fp64 products.
// A slot (X, e) per token parity, as the transpose buffers.
template <int N>
struct StageX {
    static_assert(N == 16 || N == 32, "the scans from raw token vectors: n = 16, 32");
    static constexpr int LS = Stage<N>::LS;
    static constexpr int BUF = Stage<N>::BUF;      // X (row stride LS)
    static constexpr int ED = BUF;                 // e in fp64 (N doubles)
    static constexpr int EF = BUF + 2 * N;         // e rounded to fp32 (N floats)
    static constexpr int SLOT = BUF + 3 * N;       // floats per slot
    static_assert(BUF % 4 == 0 && SLOT % 4 == 0, "16-byte aligned rows, 8-byte aligned e");
};

template <int N>
__device__ inline const double* slot_ed(const float* slot) {
    return reinterpret_cast<const double*>(slot + StageX<N>::ED);
}

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

template <int N>
__device__ inline void xop_factors(float* slot) {
    token_e_f64<N>(slot, reinterpret_cast<double*>(slot + StageX<N>::ED), slot + StageX<N>::EF);
}

// pi(i) = 4(i%4) + i/4: the row relabelling of the f64 accumulator tile (a
// lane of row group q holds rows 4q .. 4q+3 of the chain's operand).
__device__ inline int pirow(int i) { return 4 * (i & 3) + (i >> 2); }

// Operand entries o[(I * NT + K) * 4 + b] = M[16K + trow(l, b)][16I + tacol(l)]
// of the forward chain (A operand of M^T): tile (K, I) of M with its rows taken
// in the order pi and its columns in the order tacol, so that lane l's four
// accumulator entries are exactly these (ldu_tile_f64, rounded to fp32 as the
// build rounds M).
template <int N>
__device__ inline void xop_read(float (&o)[4 * Stage<N>::NV], const float* slot) {
    constexpr int NT = N / 16;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const f64x4 acc = ldu_tile_f64<N, false>(
                slot, slot_ed<N>(slot), K, I, [&](int i) { return 16 * K + pirow(i); },
                [&](int j) { return 16 * I + tacol(j); });
#pragma unroll
            for (int r = 0; r < 4; ++r) o[(I * NT + K) * 4 + r] = float(acc[r]);
        }
}

// The backward's A operand of M itself (not M^T): o[(I * NT + K) * 4 + b] =
// M[16I + tacol(l)][16K + trow(l, b)], as load_a_direct reads it: the
// transposed form of tile (I, K) (ldu_tile_f64 with TR), rows in the order
// tacol, columns in the order pi.  Every entry of M is the same sum of the same
// products as in xop_read and in the build kernel, so M is bit for bit the
// matrix the build writes.
template <int N>
__device__ inline void xop_read_direct(float (&o)[4 * Stage<N>::NV], const float* slot) {
    constexpr int NT = N / 16;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const f64x4 acc = ldu_tile_f64<N, true>(
                slot, slot_ed<N>(slot), I, K, [&](int j) { return 16 * I + tacol(j); },
                [&](int i) { return 16 * K + pirow(i); });
#pragma unroll
            for (int r = 0; r < 4; ++r) o[(I * NT + K) * 4 + r] = float(acc[r]);
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
    wave_lds_sync();
    xop_factors<N>(slot);
    wave_lds_sync();
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
// STASH (the aggregate pass from raw token vectors): each token's operand
// entries, once formed, are also written to the token's own slot of P in the
// layout the fp32 apply pass reads (stash_operands), which overwrites them.
template <int N>
__device__ inline void stash_operands(float* __restrict__ slot, const float (&o)[4 * Stage<N>::NV]);

template <int N, int PF, bool WRITE, bool FX, bool SC, bool STASH = false>
__device__ __attribute__((always_inline)) void fwd_sweep(typename Mf<N>::vec_t& X, int& ex, const float* __restrict__ M,
                          float* __restrict__ P, int32_t* __restrict__ pexp, int64_t base, int len,
                          float* tlds, float* xlds) {
    static_assert(!STASH || (FX && !WRITE), "the stash is the aggregate pass's, from raw token vectors");
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
        if constexpr (STASH) stash_operands<N>(P + base * NN, o);
        if (len > 1) {
            float* x1 = xlds + xslot<N, FX>();
            xop_stage<N>(ring[1], x1);
            wave_lds_sync();
            xop_factors<N>(x1);
            wave_lds_sync();
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
                if (k == 0 && t + 1 < len) {
                    xop_read<N>(o, x1);
                    if constexpr (STASH) stash_operands<N>(P + (base + t + 1) * NN, o);
                }
                if (k == 1 && t + 2 < len) xop_stage<N>(ring[p2], x2);
                if (k == 2) {
                    if (WRITE && t > 0) store_prefix<N, SC>(P, pexp, base + t - 1, X, ex);
                    if (t + 2 < len) {
                        wave_lds_sync();
                        xop_factors<N>(x2);
                    }
                }
                if (k == 3 && t + 2 < len) {
                    wave_lds_sync();
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
                    wave_lds_sync();
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

// The apply pass of a chunk in fp32 (n = 32): from the carry, computed in fp64
// by the look-back and rounded once, the chain runs on the fp32 matrix cores
// (v_mfma_f32_16x16x4f32, half the cycles of the fp64 product).  Its rounding
// error grows with the chunk length only, since the carry is exact to fp64 at
// every chunk start (chunks of at most kF32ChainMax tokens; measured with the
// oracle on the n = 32 workload's inputs, 512-token chunks: 3.1e-6 relative).
// The state is kept as 2^ex Y with Y in fp32: the carry is scaled by a power
// of two into range first; every fourth step the largest |entry| of the state
// the step consumes is found (while the step's products run) and, if its
// exponent has left [-60, 60], the step's result is rescaled by that power of
// two (exact).  Each P_t is stored as 2^ex Y (IEEE overflow to inf where P_t
// leaves the fp32 range, as the fp64 pass stores it).  If a checked state, or
// the chunk's final one, holds an inf or a NaN (once there, products keep one
// in the state), or a checked state holds only subnormal values, the pass gives
// up (returns false) and the caller re-runs the chunk with the fp64 pass, which
// overwrites every P_t of the chunk.  The scaled scans (SC) renormalise
// exactly after every step, as the fp64 pass does.
// Layouts: the fp32 accumulator tile holds the same entries per lane and
// register as the fp64 one (Y[16I + trow(l, r)][16J + tcol(l)], Y = P^T),
// with the natural row order instead of pi, so the A-operand entries of M_t^T
// are M_t[16K + trow(l, b)][16I + tcol(l)]: the same LDS transpose read at
// column tcol instead of tacol, and for raw token vectors the same fp64 LDU
// tile (ldu_tile_f64) with its columns in natural order, entry for entry the
// same bits as the build.
constexpr int kF32ChainMax = 1024;

template <int N>
struct Mf32 {
    static constexpr int NT = N / 16;
    struct vec_t {
        f4v32 t[NT][NT];
    };
};

// Stash layout of one token (n*n floats, the token's slot of P): lane l of the
// fp32 pass reads its 4 * NV operand entries M[16K + trow(l, b)][16I + tcol(l)]
// as NV 16-byte pieces at float offset 4 * NV * l.  The aggregate pass's lane l
// holds M[16K + trow(l, b)][16I + tacol(l)] (pi-ordered columns), i.e. the
// entries of fp32 lane (l & 48) | tacol(l), and writes them there.
template <int N>
__device__ inline void stash_operands(float* __restrict__ slot, const float (&o)[4 * Stage<N>::NV]) {
    constexpr int NA = 4 * Stage<N>::NV;
    const int l = threadIdx.x & 63;
    float* q = slot + NA * ((l & 48) | tacol(l));
#pragma unroll
    for (int e = 0; e < NA; e += 4)
        *reinterpret_cast<f4v32*>(q + e) = f4v32{o[e], o[e + 1], o[e + 2], o[e + 3]};
}

template <int N>
__device__ inline void load_stash(float (&o)[4 * Stage<N>::NV], const float* __restrict__ slot) {
    constexpr int NA = 4 * Stage<N>::NV;
    const int l = threadIdx.x & 63;
    const float* q = slot + NA * l;
#pragma unroll
    for (int e = 0; e < NA; e += 4) {
        const f4v32 v = *reinterpret_cast<const f4v32*>(q + e);
        o[e] = v[0]; o[e + 1] = v[1]; o[e + 2] = v[2]; o[e + 3] = v[3];
    }
}

template <int N>
__device__ inline void operand_read_f32(float (&o)[4 * Stage<N>::NV], const float* tb) {
    constexpr int NT = N / 16;
    constexpr int LS = Stage<N>::LS;
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const float4 w =
                *reinterpret_cast<const float4*>(tb + (16 * I + tcol(l)) * LS + 16 * K + trow(l, 0));
            float* d = &o[(I * NT + K) * 4];
            d[0] = w.x; d[1] = w.y; d[2] = w.z; d[3] = w.w;
        }
}

template <int N>
__device__ inline void xop_read_f32(float (&o)[4 * Stage<N>::NV], const float* slot) {
    constexpr int NT = N / 16;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const f64x4 acc = ldu_tile_f64<N, false>(
                slot, slot_ed<N>(slot), K, I, [&](int i) { return 16 * K + pirow(i); },
                [&](int j) { return 16 * I + j; });
#pragma unroll
            for (int r = 0; r < 4; ++r) o[(I * NT + K) * 4 + r] = float(acc[r]);
        }
}

template <int N, class Between>
__device__ inline typename Mf32<N>::vec_t chain_step_f32_with(const float (&a)[4 * Stage<N>::NV],
                                                              const typename Mf32<N>::vec_t& Y,
                                                              Between&& between) {
    constexpr int NT = N / 16;
    typename Mf32<N>::vec_t out;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J < NT; ++J) {
            f4v32 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int K = 0; K < NT; ++K)
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[(I * NT + K) * 4 + b], Y.t[K][J][b], acc, 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    between(((I * NT + J) * NT + K) * 4 + b);
                    __builtin_amdgcn_sched_barrier(0);
                }
            out.t[I][J] = acc;
        }
    return out;
}

// Largest |entry| of Y over the wave, as the bits of |x| (monotonic in |x|;
// >= 0x7f800000: inf or NaN present; 0: all zero).  The lane maxima are
// combined with DPP within each 16-lane row and across the four rows through
// scalar registers (no LDS round trips).
__device__ inline uint32_t dpp_max16(uint32_t k) {
    k = max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0xB1, 0xF, 0xF, false)));
    k = max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x4E, 0xF, 0xF, false)));
    k = max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x141, 0xF, 0xF, false)));
    k = max(k, uint32_t(__builtin_amdgcn_update_dpp(0, int(k), 0x140, 0xF, 0xF, false)));
    return k;
}

template <int N>
__device__ inline uint32_t f32_key(const typename Mf32<N>::vec_t& Y) {
    uint32_t k = 0;
#pragma unroll
    for (int I = 0; I < N / 16; ++I)
#pragma unroll
        for (int J = 0; J < N / 16; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) k = max(k, __float_as_uint(Y.t[I][J][r]) & 0x7fffffffu);
    k = dpp_max16(k);
    const uint32_t a = __builtin_amdgcn_readlane(int(k), 0), b = __builtin_amdgcn_readlane(int(k), 16);
    const uint32_t c = __builtin_amdgcn_readlane(int(k), 32), d = __builtin_amdgcn_readlane(int(k), 48);
    return max(max(a, b), max(c, d));
}

template <int N>
__device__ inline void scale_f32(typename Mf32<N>::vec_t& Y, int e) {
#pragma unroll
    for (int I = 0; I < N / 16; ++I)
#pragma unroll
        for (int J = 0; J < N / 16; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) Y.t[I][J][r] = ldexpf(Y.t[I][J][r], e);
}

template <int N, bool SC>
__device__ inline void store_prefix_f32(float* __restrict__ P, int32_t* __restrict__ pexp, int64_t tok,
                                        const typename Mf32<N>::vec_t& Y, int ex) {
    const int l = threadIdx.x & 63;
    float* p = P + tok * N * N;
    if (SC || ex == 0) {
#pragma unroll
        for (int I = 0; I < N / 16; ++I)
#pragma unroll
            for (int J = 0; J < N / 16; ++J)
                *reinterpret_cast<f4v32*>(p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0)) = Y.t[I][J];
    } else {
#pragma unroll
        for (int I = 0; I < N / 16; ++I)
#pragma unroll
            for (int J = 0; J < N / 16; ++J) {
                f4v32 v = Y.t[I][J];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = ldexpf(v[r], ex);
                *reinterpret_cast<f4v32*>(p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0)) = v;
            }
    }
    if (SC && l == 0) pexp[tok] = ex;
}

// The apply pass in fp32 from the fp64 carry X (SC: normalised, exponent ex);
// false if it gave up (see above).  STASHED (from raw token vectors): the
// aggregate pass left every token's operand entries in its slot of P
// (stash_operands), so the pass reads them there instead of forming them again.
template <int N, int PF, bool FX, bool SC, bool STASHED = false>
__device__ __attribute__((always_inline)) bool fwd_sweep_f32(const typename Mf<N>::vec_t& X, int ex,
                                                             const float* __restrict__ M, float* __restrict__ P,
                                                             int32_t* __restrict__ pexp, int64_t base, int len,
                                                             float* tlds, float* xlds) {
    using vec_t = typename Mf32<N>::vec_t;
    constexpr int NN = N * N;
    constexpr int NA = 4 * Stage<N>::NV;
    if (len <= 0) return true;
    // the carry scaled by 2^-e0 (its largest |entry| into [0.5, 1)), then rounded
    int e0 = kNoExp;
#pragma unroll
    for (int I = 0; I < N / 16; ++I)
#pragma unroll
        for (int J = 0; J < N / 16; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) e0 = max_exp(e0, X.t[I][J][r]);
    e0 = __builtin_amdgcn_readfirstlane(group_max<64>(e0));
    if (e0 == kNoExp) e0 = 0;
    vec_t Y;
#pragma unroll
    for (int I = 0; I < N / 16; ++I)
#pragma unroll
        for (int J = 0; J < N / 16; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r) Y.t[I][J][r] = float(ldexp(X.t[I][J][r], -e0));
    ex += e0;
    bool ok = true;
    static_assert(!STASHED || FX, "the stash holds operands formed from raw token vectors");
    const float* Mb = M + base * NN;
    const float* Sb = P + base * NN;  // STASHED: the operand slots
    float ring[PF][NA];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        if constexpr (STASHED) load_stash<N>(ring[p], Sb + int64_t(min(p, len - 1)) * NN);
        else load_token<N>(ring[p], Mb + int64_t(min(p, len - 1)) * NN);
    }
    float o[NA];
    if constexpr (STASHED) {
#pragma unroll
        for (int e = 0; e < NA; ++e) o[e] = ring[0][e];
        load_stash<N>(ring[0], Sb + int64_t(min(PF, len - 1)) * NN);
    } else if constexpr (FX) {
        static_assert(PF >= 3, "two tokens ahead of the chain");
        xop_stage<N>(ring[0], xlds);
        wave_lds_sync();
        xop_factors<N>(xlds);
        wave_lds_sync();
        xop_read_f32<N>(o, xlds);
        if (len > 1) {
            float* x1 = xlds + xslot<N, FX>();
            xop_stage<N>(ring[1], x1);
            wave_lds_sync();
            xop_factors<N>(x1);
            wave_lds_sync();
        }
        load_token<N>(ring[0], Mb + int64_t(min(PF, len - 1)) * NN);
        load_token<N>(ring[1], Mb + int64_t(min(PF + 1, len - 1)) * NN);
    } else {
        operand_write<N>(ring[0], tlds);
        wave_lds_sync();
        operand_read_f32<N>(o, tlds);
        load_token<N>(ring[0], Mb + int64_t(min(PF, len - 1)) * NN);
    }
    auto step = [&](int p, int t, bool refill) {
        float a[NA];
#pragma unroll
        for (int e = 0; e < NA; ++e) a[e] = o[e];
        vec_t Yn;
        uint32_t kprev = 0;  // the consumed state's largest |entry| (checked steps)
        if constexpr (STASHED) {
            // token t+1's entries from the ring, token t+1+PF's loaded into its slot
            // (never one of the slots already overwritten by a prefix)
            const int pn = (p + 1) % PF;
            Yn = chain_step_f32_with<N>(a, Y, [&](int k) {
                if (k == 0 && t + 1 < len) {
#pragma unroll
                    for (int e = 0; e < NA; ++e) o[e] = ring[pn][e];
                }
                if (k == 2 && t > 0) store_prefix_f32<N, SC>(P, pexp, base + t - 1, Y, ex);
                if (k == 3 && t + 1 < len && refill)
                    load_stash<N>(ring[pn], Sb + int64_t(min(t + 1 + PF, len - 1)) * NN);
                if (k == 8 && !SC && (t & 3) == 3) kprev = f32_key<N>(Y);
            });
        } else if constexpr (FX) {
            const int p2 = (p + 2) % PF;
            float* x1 = xlds + ((t + 1) & 1) * xslot<N, FX>();
            float* x2 = xlds + (t & 1) * xslot<N, FX>();
            Yn = chain_step_f32_with<N>(a, Y, [&](int k) {
                if (k == 0 && t + 1 < len) xop_read_f32<N>(o, x1);
                if (k == 1 && t + 2 < len) xop_stage<N>(ring[p2], x2);
                if (k == 2) {
                    if (t > 0) store_prefix_f32<N, SC>(P, pexp, base + t - 1, Y, ex);
                    if (t + 2 < len) {
                        wave_lds_sync();
                        xop_factors<N>(x2);
                    }
                }
                if (k == 3 && t + 2 < len) {
                    wave_lds_sync();
                    if (refill) load_token<N>(ring[p2], Mb + int64_t(min(t + 2 + PF, len - 1)) * NN);
                }
                if (k == 8 && !SC && (t & 3) == 3) kprev = f32_key<N>(Y);
            });
        } else {
            const int pn = (p + 1) % PF;
            float* tb = tlds + ((t + 1) & 1) * Stage<N>::BUF;
            Yn = chain_step_f32_with<N>(a, Y, [&](int k) {
                if (k == 0 && t + 1 < len) operand_write<N>(ring[pn], tb);
                if (k == 1 && t + 1 < len) {
                    wave_lds_sync();
                    operand_read_f32<N>(o, tb);
                }
                if (k == 2 && t > 0) store_prefix_f32<N, SC>(P, pexp, base + t - 1, Y, ex);
                if (k == 3 && t + 1 < len && refill)
                    load_token<N>(ring[pn], Mb + int64_t(min(t + 1 + PF, len - 1)) * NN);
                if (k == 8 && !SC && (t & 3) == 3) kprev = f32_key<N>(Y);
            });
        }
        __builtin_amdgcn_sched_barrier(0);
        Y = Yn;
        if (SC || (t & 3) == 3) {
            const uint32_t k = SC ? f32_key<N>(Y) : kprev;
            if (k >= 0x7f800000u || (k != 0 && k < 0x00800000u)) {
                ok = false;  // inf / NaN, or nothing but subnormals: the fp64 pass redoes the chunk
            } else if (k != 0) {
                const int e = int(k >> 23) - 126;  // largest |entry| in [2^(e-1), 2^e)
                if (SC || e > 60 || e < -60) {
                    scale_f32<N>(Y, -e);
                    ex += e;
                }
            }
        }
    };
    int t0 = 0;
    for (; t0 + PF <= len && ok; t0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) step(p, t0 + p, true);
    }
    if (!ok) return false;
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (t0 + p < len) step(p, t0 + p, false);
    if (!ok) return false;
    // an inf or NaN that arose after the last checked step is still in the final
    // state (a product never turns one back into a finite value)
    if (f32_key<N>(Y) >= 0x7f800000u) return false;
    store_prefix_f32<N, SC>(P, pexp, base + len - 1, Y, ex);
    return true;
}

// Retained chunk (KR > 0).  The aggregate pass loads the chunk's tokens into a
// register buffer of KR tokens (loads issued PF tokens ahead, clamped into the
// chunk) and converts each to its operand entries in place; once a token's
// product is done, its slot is overwritten with the chunk-local prefix
// L_t = M_a ... M_t (the chain state, transposed through LDS into A-operand
// entries of L_t^T, rounded to fp32).  The apply pass then needs no chain: with
// the carry C of the chunk, P_t^T = L_t^T C^T is one independent product per
// token, so the matrix core takes consecutive tokens back to back instead of
// waiting for each product's result.  Each input matrix is read from HBM once.
// The fp32 rounding of L_t enters P_t amplified by at most the condition number
// of the chunk-local product (measured with the oracle on the n = 16 workloads:
// 1.4e-7 relative, against 3.6e-8 for rounding P_t itself).
// The prefix transpose of token t-1 runs between the products of token t
// (written in the first hook, read back in the second, after the barrier the
// step has there anyway); the chunk's last token is transposed after its step.
// SC: the chain is renormalised every step; the slot holds the normalised
// L~_t and exl[t] its exponent (P_t = 2^(e_C + exl[t]) C~ L~_t).
template <int N>
__device__ inline void prefix_write(const typename Mf<N>::vec_t& X, float* pl) {
    constexpr int NT = Mf<N>::NT;
    constexpr int LS = N + 4;
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = 0; J < NT; ++J)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pl[(16 * I + trow(l, r)) * LS + 16 * J + tcol(l)] = float(X.t[I][J][r]);
}

// A-operand entries of X for the apply's fp32 products, from its transpose
// buffer: o[(I * NT + K) * 4 + b] = X[16I + l%16][16K + trow(l, b)].  (The rows
// are in natural order, not the fp64 chain's tacol order: the fp32 accumulator
// keeps rows 4(l/16) .. 4(l/16)+3 in lane l, which is then exactly the fp64
// accumulator's layout of the result.)
template <int N>
__device__ inline void prefix_read(float (&o)[4 * Stage<N>::NV], const float* pl) {
    constexpr int NT = Mf<N>::NT;
    constexpr int LS = N + 4;
    typedef float f4v __attribute__((ext_vector_type(4)));
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int K = 0; K < NT; ++K) {
            const f4v w = *reinterpret_cast<const f4v*>(pl + (16 * I + (l & 15)) * LS + 16 * K + trow(l, 0));
#pragma unroll
            for (int b = 0; b < 4; ++b) o[(I * NT + K) * 4 + b] = w[b];
        }
}

template <int N, int KR, int PF, bool FX, bool SC, bool FULL>
__device__ __attribute__((always_inline)) void fwd_pass_retain(typename Mf<N>::vec_t& X, int& ex, const float* __restrict__ M,
                                int64_t base, int len_in, float (&buf)[KR][4 * Stage<N>::NV],
                                float* tlds, float* xlds, float* plds, int* exl) {
    // FULL: a whole chunk, every per-token test resolved at compile time
    const int len = FULL ? KR : len_in;
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
    constexpr int NN = F::NN;
    constexpr int NA = 4 * Stage<N>::NV;
    constexpr int PB = N * (N + 4);  // floats per prefix transpose buffer
    if (len <= 0) return;
    const float* Mb = M + base * NN;
    const int l = threadIdx.x & 63;
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
            wave_lds_sync();
            xop_factors<N>(x1);
            wave_lds_sync();
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
            float* pl = plds + (t & 1) * PB;  // token t-1's prefix
            const bool next = t + 1 < KR && t + 1 < len;
            vec_t Xn = chain_step_with<N>(a, X, vzero<N>(), [&](int k) {
                if constexpr (FX) {
                    if constexpr (t + 1 < KR) {  // buf[t + 1] exists
                        if (k == 0 && next) {
                            float o[NA];
                            xop_read<N>(o, xb);
#pragma unroll
                            for (int e = 0; e < NA; ++e) buf[t + 1][e] = o[e];
                        }
                    }
                    if constexpr (t > 0)
                        if (k == 1) prefix_write<N>(X, pl);
                    if constexpr (t + 2 < KR) {  // buf[t + 2] exists
                        float* x2 = xlds + (t & 1) * xslot<N, FX>();
                        const bool next2 = t + 2 < len;
                        if (k == 1 && next2) xop_stage<N>(buf[t + 2], x2);
                        if (k == 2 && next2) {
                            wave_lds_sync();
                            xop_factors<N>(x2);
                        }
                    }
                    if (k == 3) {
                        wave_lds_sync();
                        if constexpr (t > 0) prefix_read<N>(buf[t - 1], pl);
                    }
                } else {
                    if constexpr (t > 0)
                        if (k == 0) prefix_write<N>(X, pl);
                    if constexpr (t + 1 < KR)
                        if (k == 0 && next) operand_write<N>(buf[t + 1], tb);
                    if (k == 1) {
                        wave_lds_sync();
                        if constexpr (t + 1 < KR) {
                            if (next) {
                                float o[NA];
                                operand_read<N>(o, tb);
#pragma unroll
                                for (int e = 0; e < NA; ++e) buf[t + 1][e] = o[e];
                            }
                        }
                        if constexpr (t > 0) prefix_read<N>(buf[t - 1], pl);
                    }
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            X = Xn;
            if constexpr (SC) {
                renorm_acc<N>(X, ex);
                if (l == 0) exl[t] = ex;
            }
            if (t + 1 == len) {
                // the chunk's last prefix: transposed right away
                float* pn = plds + ((t + 1) & 1) * PB;
                wave_lds_sync();
                prefix_write<N>(X, pn);
                wave_lds_sync();
                prefix_read<N>(buf[t], pn);
            }
        }
    });
}

// P_t^T = L_t^T C^T for every token of a retained chunk, on the fp32 matrix
// cores: X holds the carry C^T (SC: C~^T with exponent ex), buf the prefixes.
// The carry is scaled by an exact power of two 2^-s to largest |entry| in
// [0.5, 1) and rounded to fp32 once, every token is one fp32 product
// (v_mfma_f32_16x16x4f32, four per 16x16 tile), and the result is scaled back
// by 2^s (exact; IEEE overflow to inf where P_t leaves the fp32 range).  The
// running state of the sequence (the aggregate pass's chain, aggregates and
// carries) stays fp64; only this last product of each token is fp32, and its
// error does not propagate (measured with the oracle on the n = 16 workloads:
// 2.7e-7 relative).  Two tokens at a time, their products interleaved.
template <int N>
__device__ inline void store_f4_rows(float* __restrict__ p, const f4v32 (&D)[Mf<N>::NT][Mf<N>::NT]) {
    const int l = threadIdx.x & 63;
#pragma unroll
    for (int I = 0; I < Mf<N>::NT; ++I)
#pragma unroll
        for (int J = 0; J < Mf<N>::NT; ++J) {
            float* q = p + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0);
            if constexpr (N == 16) __builtin_nontemporal_store(D[I][J], reinterpret_cast<f4v32*>(q));
            else *reinterpret_cast<f4v32*>(q) = D[I][J];
        }
}

template <int N, int KR, bool SC>
__device__ __attribute__((always_inline)) void fwd_apply_retain(const typename Mf<N>::vec_t& X, int ex, float* __restrict__ P,
                                 int32_t* __restrict__ pexp, int64_t base, int len,
                                 const float (&buf)[KR][4 * Stage<N>::NV], const int* exl) {
    constexpr int NT = Mf<N>::NT;
    constexpr int NN = N * N;
    static_assert(KR % 2 == 0, "tokens in pairs");
    if constexpr (SC) wave_lds_sync();  // the prefixes' exponents in exl
    // the carry, scaled and rounded once: B entries cb[K][J][b]
    int s = kNoExp;
#pragma unroll
    for (int K = 0; K < NT; ++K)
#pragma unroll
        for (int J = 0; J < NT; ++J)
#pragma unroll
            for (int b = 0; b < 4; ++b) s = max_exp(s, X.t[K][J][b]);
    s = group_max<64>(s);
    if (s == kNoExp) s = 0;
    float cb[NT][NT][4];
#pragma unroll
    for (int K = 0; K < NT; ++K)
#pragma unroll
        for (int J = 0; J < NT; ++J)
#pragma unroll
            for (int b = 0; b < 4; ++b) cb[K][J][b] = float(ldexp(X.t[K][J][b], -s));
    // token t's product, P_t^T up to the power of two
    auto product = [&](f4v32 (&D)[NT][NT], const float (&a)[4 * Stage<N>::NV]) {
#pragma unroll
        for (int I = 0; I < NT; ++I)
#pragma unroll
            for (int J = 0; J < NT; ++J) {
                f4v32 c0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int K = 0; K < NT; ++K)
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[(I * NT + K) * 4 + b], cb[K][J][b], c0, 0, 0, 0);
                D[I][J] = c0;
            }
    };
    if constexpr (!SC) {
        if (len == KR) {
            // a whole chunk: branch-free, token t+1's products issued before token
            // t is stored.  A carry well inside the fp32 range is rounded as it is
            // and every product stored straight from the matrix-core accumulators
            // (scaling by 2^-s and back by 2^s changes no bit of a result unless
            // an intermediate leaves the normal range); any other takes the scaling
            // above and each result is multiplied back by 2^s (v_ldexp: exact, inf
            // past the fp32 range) before its store, the same bits as the paired
            // path below
            const int se = (s >= -64 && s <= 64) ? 0 : s;
            if (se == 0)
#pragma unroll
                for (int K = 0; K < NT; ++K)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
#pragma unroll
                        for (int b = 0; b < 4; ++b) cb[K][J][b] = float(X.t[K][J][b]);
            f4v32 D[2][NT][NT];
            product(D[0], buf[0]);
            static_for(std::make_integer_sequence<int, KR>{}, [&](auto tc) {
                constexpr int t = decltype(tc)::value;
                if constexpr (t + 1 < KR) product(D[(t + 1) & 1], buf[t + 1]);
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
#pragma unroll
                        for (int r = 0; r < 4; ++r) D[t & 1][I][J][r] = ldexpf(D[t & 1][I][J][r], se);
                store_f4_rows<N>(P + (base + t) * NN, D[t & 1]);
            });
            return;
        }
    }
    static_for(std::make_integer_sequence<int, KR / 2>{}, [&](auto pc) {
        constexpr int t = 2 * decltype(pc)::value;
        if (t < len) {
            f4v32 D0[NT][NT], D1[NT][NT];
#pragma unroll
            for (int I = 0; I < NT; ++I)
#pragma unroll
                for (int J = 0; J < NT; ++J) {
                    f4v32 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int K = 0; K < NT; ++K)
#pragma unroll
                        for (int b = 0; b < 4; ++b) {
                            c0 = __builtin_amdgcn_mfma_f32_16x16x4f32(buf[t][(I * NT + K) * 4 + b], cb[K][J][b], c0, 0, 0, 0);
                            c1 = __builtin_amdgcn_mfma_f32_16x16x4f32(buf[t + 1][(I * NT + K) * 4 + b], cb[K][J][b], c1, 0, 0, 0);
                        }
                    D0[I][J] = c0;
                    D1[I][J] = c1;
                }
            // 2^s back (SC: renormalised, the shift into the exponent)
            auto finish = [&](f4v32 (&D)[NT][NT], int tok) {
                int e = s;
                if constexpr (SC) {
                    int m = kNoExp;
#pragma unroll
                    for (int I = 0; I < NT; ++I)
#pragma unroll
                        for (int J = 0; J < NT; ++J)
#pragma unroll
                            for (int r = 0; r < 4; ++r) m = max_exp(m, D[I][J][r]);
                    m = group_max<64>(m);
                    const int shift = m == kNoExp ? 0 : m;
#pragma unroll
                    for (int I = 0; I < NT; ++I)
#pragma unroll
                        for (int J = 0; J < NT; ++J)
#pragma unroll
                            for (int r = 0; r < 4; ++r) D[I][J][r] = ldexpf(D[I][J][r], -shift);
                    e = ex + exl[tok] + s + shift;
                    if ((threadIdx.x & 63) == 0) pexp[base + tok] = e;
                } else {
#pragma unroll
                    for (int I = 0; I < NT; ++I)
#pragma unroll
                        for (int J = 0; J < NT; ++J)
#pragma unroll
                            for (int r = 0; r < 4; ++r) D[I][J][r] = ldexpf(D[I][J][r], s);
                }
                store_f4_rows<N>(P + (base + tok) * NN, D);
            };
            finish(D0, t);
            if (t + 1 < len) finish(D1, t + 1);
        }
    });
}

// Start delay of the one-wave-per-SIMD multi-chunk scans.  Their chunks all
// take the same time, so the waves of a launch would go through their load
// pass, look-back and store pass in step, with HBM idle during the look-backs.
// Every other wave of the first round (1024 per wave a SIMD holds) starts
// `clocks` late and only then takes its ticket, which keeps the two halves out
// of phase for the whole launch (figures at the call sites, interleaved runs on
// one box).  Launches of fewer chunks than that have no such contention and
// start at once.  The wait is bounded and the wave holds no ticket meanwhile,
// so nothing waits on it.
template <int WAVES = 1>
__device__ inline void stagger_start(int64_t nchunks, uint64_t clocks) {
    if (nchunks >= 1024 * WAVES && blockIdx.x < 1024u * WAVES && (blockIdx.x & 1)) {
        // at most 256 sleeps of 512 clocks, whatever the clock counter reads
        const uint64_t t0 = __builtin_amdgcn_s_memtime();
        for (int i = 0; i < 256 && __builtin_amdgcn_s_memtime() - t0 < clocks; ++i) __builtin_amdgcn_s_sleep(8);
    }
}

// One wave per SIMD: the forward keeps a chunk's operands (n = 16) or a deep
// operand ring (n = 32) in the whole register file.  The forwards from raw token
// vectors run more waves per SIMD: a wave's own vector-ALU instructions do not
// overlap its matrix-core products (measured: each adds its issue time to the
// product chain), another wave's do, and forming each token's matrix on chip is
// vector-ALU work.  n = 16: 24-token retained chunks at three waves (two for
// the scaled instance, which needs more registers); n = 32 (unscaled): two.
template <int N, int KR, bool FX, bool SC>
constexpr int fwd_waves() {
    return KR == 24 ? (SC ? 2 : 3) : ((N == 32 && FX && !SC) ? 2 : 1);
}

template <int N, int PF, int KR, bool FX, bool SC>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(fwd_waves<N, KR, FX, SC>(), fwd_waves<N, KR, FX, SC>())))
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
    // retained chunks: the prefix transpose buffers, and (SC) the prefixes' exponents
    __shared__ __align__(16) float plds[KR > 0 ? 2 * N * (N + 4) : 4];
    __shared__ int exl[KR > 0 && SC ? KR : 1];
    const int l = threadIdx.x & 63;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    // retained n = 16 chunks: 16k clocks (C3 250.5 -> 246.5-247 us, C5 141 ->
    // 136 us; four groups 8k clocks apart timed the same); n = 32 (one round of
    // 512-token chunks): 50k clocks (1462 -> 1448 us; 150k: 1488 us); the
    // forwards from raw token vectors, three and two waves per SIMD: no gain
    if constexpr (KR == 64) stagger_start(multi ? nchunks : 0, 16000);
    if constexpr (N == 32 && KR == 0 && !FX) stagger_start(multi ? nchunks : 0, 50000);
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
    // n = 32: the apply pass runs in fp32 (fwd_sweep_f32); from raw token vectors
    // it reads the token matrices the aggregate pass formed and left in P's slots
    constexpr bool kF32Apply = N == 32 && KR == 0;
    constexpr bool kStash = kF32Apply && FX;
    float buf[KR > 0 ? KR : 1][Mf<N>::NT * Mf<N>::NT * 4];
    if constexpr (KR > 0) {
        constexpr int PFR = N == 16 ? kPfRetain16 : PF;
        if (ch.len == KR)
            fwd_pass_retain<N, KR, PFR, FX, SC, true>(X, ex, M, ch.base, ch.len, buf, tlds, xlds, plds, exl);
        else
            fwd_pass_retain<N, KR, PFR, FX, SC, false>(X, ex, M, ch.base, ch.len, buf, tlds, xlds, plds, exl);
    } else {
        fwd_sweep<N, PF, false, FX, SC, kStash>(X, ex, M, P, cy.out_exp, ch.base, ch.len, tlds, xlds);
    }
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
        wave_lds_sync();
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
    if constexpr (KR > 0) {
        fwd_apply_retain<N, KR, SC>(X, ex, P, cy.out_exp, ch.base, ch.len, buf, exl);
    } else {
        bool done = false;
        if constexpr (kF32Apply)
            if (ch.len <= kF32ChainMax)
                done = fwd_sweep_f32<N, PF, FX, SC, kStash>(X, ex, M, P, cy.out_exp, ch.base, ch.len, tlds, xlds);
        if (!done)
            fwd_sweep<N, PF, true, FX, SC>(X, ex, M, P, cy.out_exp, ch.base, ch.len, tlds, xlds);
    }
}

// ---------------------------------------------------------------------------- backward

// A operand of M (load_a_direct's layout) from the raw token vector at xt: the
// token is loaded, staged in LDS slot xs and multiplied out on the matrix core
// (xop_stage, xop_factors, xop_read_direct).  Wave-uniform; xs is free on entry.
template <int N>
__device__ inline void x_operand_direct(typename Mf<N>::aop_t& a, const float* xt, float* xs) {
    constexpr int NA = 4 * Stage<N>::NV;
    const int l = threadIdx.x & 63;
    float v[NA], o[NA];
#pragma unroll
    for (int q = 0; q < Stage<N>::NV; ++q) {
        const float4 w = reinterpret_cast<const float4*>(xt)[q * 64 + l];
        v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
    }
    wave_lds_sync();
    xop_stage<N>(v, xs);
    wave_lds_sync();
    xop_factors<N>(xs);
    wave_lds_sync();
    xop_read_direct<N>(o, xs);
    operand_from<N>(a, o);
}

// Reverse sweep over the chunk (positions len-1 .. 0).
//   AGG:  G <- dP_t^T + M_{t+1} G from G = 0 and W <- M_{t+1} W from W = I.
//   GRAD: G <- dP_t^T + M_{t+1} G from the carry; dM_t^T = G_t P_{t-1}.
// At the last token of a sequence there is no M_{t+1}: G <- dP_t^T.
// FX: M holds raw token vectors and each input matrix is formed on chip (the
// LDU factors of the build, "Improving Matrix Recurrent Units as an Attention
// Alternative", Key Points) from the token staged in the LDS slots xs (two,
// alternating by step).  Step i stages its own token x_t and forms from it the
// A operand of M_t, which is the next step's M_{t+1}: every token is staged
// once, and the operand is ready a whole step before the chain needs it (the
// chunk's first step takes the operand of the token after the chunk from the
// prologue).
// DX (with FX and GRAD): the output is dL/dx_t instead of dM_t.  dM_t, rounded
// to fp32 as the backward to dM stores it, goes through LDS (gs) with the
// staged x_t and its e into build_vjp_token, the same routine as the build's
// gradient kernel, so dx is bit for bit build_inputs_bwd(x, dM); dxl holds gs,
// the dx staging ds (both row stride n + 4) and 4 floats for the mean.
// KR > 0 (a whole chunk of KR tokens, len == KR): the sweep runs expanded at
// compile time and keeps dL/dP in registers across the two passes: the
// aggregate pass copies each token's dP_t operand into keep, the pass from
// the carry takes it from there and reads only M and P.
template <int N, int PF, bool GRAD, bool FX, bool DX, int KR = 0, int KB>
__device__ __attribute__((always_inline)) void bwd_sweep(typename Mf<N>::vec_t& G, typename Mf<N>::vec_t& W,
                          const float* __restrict__ M, const float* __restrict__ P,
                          const float* __restrict__ dP, float* __restrict__ dM, double* tr,
                          float* xs, float* dxl, int64_t base, int64_t t0, int len_in, int64_t T,
                          const ScanCarry& cy,
                          float (&keep)[KB][4 * (N / 16) * (N / 16)]) {
    static_assert(!DX || (FX && GRAD), "the gradient to x starts from raw token vectors");
    static_assert(KR == 0 || (!FX && !DX), "the retained sweep starts from M");
    static_assert(KR <= KB, "the buffer holds the chunk");
    const int len = KR > 0 ? KR : len_in;
    using F = Mf<N>;
    using vec_t = typename F::vec_t;
    constexpr int NT = F::NT;
    constexpr int NN = F::NN;
    constexpr int NA = NT * NT * 4;
    constexpr int TS = N + 1;  // LDS row stride of the transpose buffer
    constexpr int LS = N + 4;  // row stride of the token and gradient staging
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

    // ring of prefetched operands per token: M_{t+1} (A operand, runs of 4; FX:
    // the raw token x_t itself), dP_t (C operand, runs of 4), P_{t-1} (B operand
    // of the dM product).  (Read non-temporally the backward was faster launch
    // after launch, but slower right after the forward, as in a training step:
    // ordinary accesses.)
    float rm[PF][NA], rr[PF][NA], rp[PF][GRAD ? NA : 1];
    auto fetch = [&](int slot, int i) {
        const int pos = max(len - 1 - i, 0);
        if constexpr (FX) {
            // the raw token x_t, row-major 16-byte pieces (as load_token)
#pragma unroll
            for (int q = 0; q < Stage<N>::NV; ++q) {
                const float4 v = reinterpret_cast<const float4*>(Mb + int64_t(pos) * NN)[q * 64 + l];
                float* d = &rm[slot][4 * q];
                d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
            }
        } else {
            const int pm = min(pos, hi_m - 1) + 1;  // clamped: only used when pos < hi_m
            const float* mt = Mb + int64_t(hi_m > 0 ? pm : pos) * NN;
#pragma unroll
            for (int I = 0; I < NT; ++I)
#pragma unroll
                for (int K = 0; K < NT; ++K) {
                    const float4 v = *reinterpret_cast<const float4*>(
                        mt + (16 * I + ac) * N + 16 * K + trow(l, 0));
                    float* d = &rm[slot][(I * NT + K) * 4];
                    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
                }
        }
        if constexpr (!(KR > 0 && GRAD)) {  // the retained pass from the carry keeps dP_t
#pragma unroll
            for (int I = 0; I < NT; ++I)
#pragma unroll
                for (int J = 0; J < NT; ++J) {
                    const float4 v = *reinterpret_cast<const float4*>(
                        Rb + int64_t(pos) * NN + (16 * J + c) * N + 16 * I + trow(l, 0));
                    float* d = &rr[slot][(I * NT + J) * 4];
                    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
                }
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
    // FX: A operand of M_{t+1} for the coming step (from the previous step, or
    // the prologue: the token after the chunk, when the sequence has one)
    typename F::aop_t a_next;
    if constexpr (FX) {
        if (hi_m == len) x_operand_direct<N>(a_next, Mb + int64_t(len) * NN, xs);
        else a_next = typename F::aop_t{};
    }
    auto step = [&](int p, int i, bool refill) {
        const int pos = len - 1 - i;
        const bool has_next = pos < hi_m;
        typename F::aop_t a;
        vec_t cr;
        float bp[NT][NT][4];  // GRAD: B entries of P_{t-1}, fp32 as read
        float* xsl = xs + (i & 1) * xslot<N, FX>();  // FX: this step's token slot
        if constexpr (FX) {
            a = a_next;
            // x_t: stage, factors, and M_t's operand for the next step
            float o[NA];
            xop_stage<N>(rm[p], xsl);
            wave_lds_sync();
            xop_factors<N>(xsl);
            wave_lds_sync();
            xop_read_direct<N>(o, xsl);
            operand_from<N>(a_next, o);
        } else {
#pragma unroll
            for (int e = 0; e < NA; ++e) a.v[e / (4 * NT)][(e / 4) % NT][e % 4] = double(rm[p][e]);
        }
#pragma unroll
        for (int e = 0; e < NA; ++e) cr.t[e / (4 * NT)][(e / 4) % NT][e % 4] = double(rr[p][e]);
        if constexpr (GRAD) {
#pragma unroll
            for (int e = 0; e < NA; ++e) bp[e / (4 * NT)][(e / 4) % NT][e % 4] = rp[p][e];
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
                            bp[K][J][b] = cs[(16 * K + trow(l, b)) * N + 16 * J + c];
            }
            // dM_t^T = G_t P_{t-1} on the fp32 matrix cores, from G_t rounded to
            // fp32 once: its error stays in dM_t (the recurrence runs on in fp64)
            f4v32 D[NT][NT];
            if (pos >= lo_p || cy.carry) {
                // transpose G through LDS: A entries of G are G[16I + tcol][16K + trow(l, b)]
                // (natural row order: the fp32 accumulator keeps rows 4(l/16) .. +3 in lane l)
                // (row stride n + 4 floats: conflict-free writes, 16-byte reads)
                float* trf = reinterpret_cast<float*>(tr);
                wave_lds_sync();
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            trf[(16 * I + trow(l, r)) * LS + 16 * J + c] = float(G.t[I][J][r]);
                wave_lds_sync();
                float ag[NT][NT][4];
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int K = 0; K < NT; ++K) {
                        const f4v32 v = *reinterpret_cast<const f4v32*>(trf + (16 * I + c) * LS + 16 * K + trow(l, 0));
#pragma unroll
                        for (int b = 0; b < 4; ++b) ag[I][K][b] = v[b];
                    }
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J) {
                        f4v32 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int K = 0; K < NT; ++K)
#pragma unroll
                            for (int b = 0; b < 4; ++b)
                                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(ag[I][K][b], bp[K][J][b], acc, 0, 0, 0);
                        D[I][J] = acc;
                    }
            } else {
                // t = 0: P_{-1} = I
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
#pragma unroll
                        for (int r = 0; r < 4; ++r) D[I][J][r] = float(G.t[I][J][r]);
            }
            if constexpr (DX) {
                // dM_t (fp32, row-major) into gs, then the build's gradient
                float* gs = dxl;
                float* ds = dxl + N * LS;
                float* part = dxl + 2 * N * LS;
                typedef float f4v __attribute__((ext_vector_type(4)));
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
                        *reinterpret_cast<f4v*>(gs + (16 * J + tcol(l)) * LS + 16 * I + trow(l, 0)) = D[I][J];
                wave_lds_sync();
                build_vjp_token<N>(xsl, gs, xsl + StageX<N>::EF, part, ds);
                wave_lds_sync();
                store_rows_from_lds<N>(out, ds);
            } else {
#pragma unroll
                for (int I = 0; I < NT; ++I)
#pragma unroll
                    for (int J = 0; J < NT; ++J)
                        *reinterpret_cast<f4v32*>(out + (16 * J + tcol(l)) * N + 16 * I + trow(l, 0)) = D[I][J];
            }
            if (pos < lo_p && cy.dcarry) {
                // dL/dP_{-1} = Q_0 M_0^T, i.e. its transpose is M_0 G_0
                typename F::aop_t am;
                if constexpr (FX) am = a_next;  // M_0's operand, formed from x_0 in this step
                else load_a_direct<N, float>(am, Mb + int64_t(pos) * NN);
                store_acc_rows<N, float>(cy.dcarry + (s0 / T) * NN, chain_step<N>(am, G, vzero<N>()));
            }
        }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p) fetch(p, min(p, len - 1));
    if constexpr (KR > 0) {
        static_for(std::make_integer_sequence<int, KR>{}, [&](auto ic) {
            constexpr int i = decltype(ic)::value;
            constexpr int p = i % PF;
#pragma unroll
            for (int e = 0; e < NA; ++e) {
                if constexpr (GRAD) rr[p][e] = keep[i][e];
                else keep[i][e] = rr[p][e];
            }
            step(p, i, i + PF < KR);
        });
        return;
    }
    int i0 = 0;
    for (; i0 + PF <= len; i0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) step(p, i0 + p, true);
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (i0 + p < len) step(p, i0 + p, false);
}

// The n = 16 instances from raw token vectors run two waves per SIMD (a
// shallower prefetch ring fits them in half the register file): forming each
// input matrix on chip lengthens a step, and the second wave's products fill
// the first one's waits (C5 backward from x 653 -> 457 us, the layer backward
// to dx 907 -> 579 us); the backward from M gained nothing and keeps one wave
// with the deeper ring.
template <int N, bool FX>
constexpr int bwd_waves() { return (N == 16 && FX) ? 2 : 1; }

template <int N, int PF, bool FX, bool DX, int KRB>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(bwd_waves<N, FX>(), bwd_waves<N, FX>())))
void bwd_mfma_kernel(const float* __restrict__ M,
                                                      const float* __restrict__ P,
                                                      const float* __restrict__ dP,
                                                      float* __restrict__ dM, int64_t S, int64_t T,
                                                      int64_t K, int64_t nch, int64_t Z,
                                                      unsigned char* __restrict__ ws, ScanCarry cy) {
    using F = Mf<N>;
    using acc_t = typename F::acc_t;
    using vec_t = typename F::vec_t;
    constexpr int NN = N * N;
    __shared__ __align__(16) double tr[N * (N + 1)];  // also the fp32 transpose (row stride n + 4)
    __shared__ double xl[NN];
    __shared__ __align__(16) float xs[FX ? 2 * StageX<N>::SLOT : 4];  // FX: token slots
    __shared__ __align__(16) float dxl[DX ? 2 * N * (N + 4) + 4 : 4];  // DX: gradient staging
    const int l = threadIdx.x & 63;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    // the retained backward from M (one wave per SIMD): C5 299 -> 290 us; the
    // n = 16 backwards from raw token vectors (two waves per SIMD): C5 to dM
    // 455 -> 447 us, to dx 567 -> 559 us
    if constexpr (KRB == 64) stagger_start(multi ? nchunks : 0, 16000);
    if constexpr (N == 16 && FX) stagger_start<bwd_waves<N, FX>()>(multi ? nchunks : 0, 16000);
    const int64_t cidx =
        multi ? ticket_to_chunk(int64_t(wave_ticket(&hdr->ticket)), S, nch, 1) : int64_t(blockIdx.x);
    if (cidx >= nchunks) return;
    const Chunk ch = chunk_at(cidx, nch, K, T, true);

    vec_t G = vzero<N>();
    vec_t W = videntity<N>(l);
    float keep[KRB > 0 ? KRB : 1][4 * (N / 16) * (N / 16)];  // KRB: a whole chunk's dL/dP operands
    if (!multi) {
        bwd_sweep<N, PF, true, FX, DX>(G, W, M, P, dP, dM, tr, xs, dxl, ch.base, ch.t0, ch.len, T, cy, keep);
        return;
    }
    const bool retain = KRB > 0 && ch.len == KRB;
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
    if (retain)
        bwd_sweep<N, PF, false, FX, false, KRB>(G, W, M, P, dP, dM, tr, xs, dxl, ch.base, ch.t0, ch.len, T, cy,
                                                keep);
    else
        bwd_sweep<N, PF, false, FX, false>(G, W, M, P, dP, dM, tr, xs, dxl, ch.base, ch.t0, ch.len, T, cy, keep);
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
        wave_lds_sync();
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
    if (retain)
        bwd_sweep<N, PF, true, FX, DX, KRB>(G, W, M, P, dP, dM, tr, xs, dxl, ch.base, ch.t0, ch.len, T, cy, keep);
    else
        bwd_sweep<N, PF, true, FX, DX>(G, W, M, P, dP, dM, tr, xs, dxl, ch.base, ch.t0, ch.len, T, cy, keep);
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

template <int N, int PF, bool FX, bool DX, int KRB = 0>
hipError_t run_bwd(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                   int64_t T, int64_t K, int64_t nch, int64_t Z, void* ws, hipStream_t stream,
                   const ScanCarry& cy) {
    hipLaunchKernelGGL((bwd_mfma_kernel<N, PF, FX, DX, KRB>), dim3(unsigned(S * nch)), dim3(64), 0,
                       stream, M, P, dP, dM, S, T, K, nch, Z, static_cast<unsigned char*>(ws), cy);
    return hipGetLastError();
}

}  // namespace

// Tokens of one chunk kept in registers by the n = 16 forward kernel, and the
// operand prefetch depth of its streamed sweeps (tokens in flight).
constexpr int kRetain16 = 64;
// from raw token vectors: 24-token chunks at three waves per SIMD (the token
// build's vector-ALU work of one wave runs while another's products run on the
// matrix cores; measured faster than 32-token chunks at two waves and 64-token
// chunks at one)
constexpr int kRetain16x = 24;
// the n = 16 backward from M: whole chunks of this length keep dL/dP in registers
constexpr int kRetainBwd16 = 64;
constexpr int kPf16 = 16;

int mfma_retain_tokens(int n, bool from_x) { return n == 16 ? (from_x ? kRetain16x : kRetain16) : 0; }

hipError_t launch_fwd_mfma(const float* M, float* P, int64_t S, int64_t T, int n, int64_t K,
                           int64_t nch, int64_t Z, void* ws, hipStream_t stream, bool from_x,
                           const ScanCarry& cy) {
    if (n == 16) {
        const bool retain = kRetain16 > 0 && nch > 1 && K <= kRetain16;
        if (from_x) {
            // chunks of up to 64 tokens keep their prefixes (the same arithmetic
            // at either buffer size, so the same bits as the scan from M)
            if (nch > 1 && K <= kRetain16x)
                return run_fwd<16, kPf16, kRetain16x, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
            if (retain) return run_fwd<16, kPf16, kRetain16, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
            return run_fwd<16, kPf16, 0, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
        }
        if (retain) return run_fwd<16, kPf16, kRetain16, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
        return run_fwd<16, kPf16, 0, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
    }
    if (n == 32) {
        if (from_x) return run_fwd<32, 4, 0, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
        return run_fwd<32, 4, 0, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_mfma(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                           int64_t T, int n, int64_t K, int64_t nch, int64_t Z, void* ws,
                           hipStream_t stream, bool from_x, bool to_dx, const ScanCarry& cy) {
    if (to_dx && !from_x) return hipErrorInvalidValue;
    // prefetch depth: the n = 16 instances from raw token vectors 4 tokens (two
    // waves per SIMD), the n = 32 ones 1 (two spill)
    if (n == 16) {
        if (to_dx) return run_bwd<16, 2, true, true>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        if (from_x) return run_bwd<16, 4, true, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        // 64-token chunks keep dL/dP in registers between the passes (a shallower
        // ring makes room for them)
        if (nch > 1 && K == kRetainBwd16)
            return run_bwd<16, 4, false, false, kRetainBwd16>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        return run_bwd<16, 8, false, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
    }
    if (n == 32) {
        if (to_dx) return run_bwd<32, 1, true, true>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        if (from_x) return run_bwd<32, 1, true, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        return run_bwd<32, 2, false, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
    }
    return hipErrorInvalidValue;
}

}  // namespace mru
