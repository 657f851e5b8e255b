// Chunked look-back scans for small matrices (n = 4, 8) on the vector ALUs.
//
// Right multiplication acts on each row of the running state separately:
// row_i(P_{t-1} M_t) = row_i(P_{t-1}) M_t.  So a chain is a group of n/R lanes,
// each owning R rows of the n-by-n state, and no lane ever needs another lane's
// state to advance; each needs the whole input matrix of the step, which the
// wave stages through LDS from fully coalesced global loads (one 1 KiB wave
// load per instruction) and then reads back as a broadcast.  A wave runs
// 64*R/n chains side by side, each on its own chunk.
//
// Forward ("MRU Update: ...", section "What MRU Actually Does"): the chain
// state is R rows of P_t = P_{t-1} M_t.
// Backward (gradient of sum_t <dP_t, P_t>): the chain state is R rows of
// Q_t = dP_t + Q_{t+1} M_{t+1}^T, swept from the last token to the first, and
// dM_t = P_{t-1}^T Q_t needs all rows of Q_t and of P_{t-1}, exchanged through
// LDS.  From M the backward reads every stored prefix; from raw token vectors
// it reads one stored prefix per TB tokens and recomputes the others from it
// (VALU work is cheap here, HBM bytes are not).
#include <type_traits>

#include "mru_build.h"
#include "mru_device.h"
#include "mru_kernels.h"

namespace mru {
namespace {

struct ChainInfo {
    int64_t base;  // token index (s*T + t0) of the chunk's first token
    int32_t len;   // tokens in the chunk (0 for an idle chain)
    int32_t t0;    // position of the chunk's first token in its sequence
};

template <int N, int R, int TB>
struct Valu {
    static constexpr int NN = N * N;
    static constexpr int LPC = N / R;             // lanes per chain
    static constexpr int G = 64 / LPC;            // chains per wave
    static constexpr int F4_TOK = NN / 4;         // float4 per matrix
    static constexpr int F4_BLK = TB * F4_TOK;    // float4 per chain per staged block
    static constexpr int LD = (G * F4_BLK) / 64;  // float4 loads per lane per staged array
    static constexpr int CH_STRIDE = TB * NN + 4; // floats per chain in LDS (16 B skew)
    // LDS buffers through which a chain's lanes swap rows: every lane writes its
    // rows (16-byte stores), then reads its chain's whole matrix (16-byte
    // broadcasts within the chain) and single columns (4-byte reads).  XR floats
    // per row, QX_STRIDE per chain.  n = 8: rows of 12 floats, so that the 8
    // lanes of a chain (one 8-lane group of a 16-byte access) store to distinct
    // banks (with 8-float rows lanes li and li+4 share banks), and chains 8 banks
    // apart, so that the 4 chains of a 32-lane half read a column from distinct
    // banks.  n = 4: rows of 4 floats with a 16 B skew per chain (an unskewed
    // n*n-float stride sends all chains of a wave to the same banks).
    static constexpr int XR = N == 8 ? 12 : N;
    static constexpr int QX_STRIDE = N == 8 ? 104 : NN + 4;
    static_assert(XR * N <= QX_STRIDE, "a chain's exchanged matrix fits its stride");
    // floats per chain of the backward's kept input matrix (16 B skew, as above)
    static constexpr int NX_STRIDE = NN + 4;
    static_assert((G * F4_BLK) % 64 == 0, "staging must tile the wave");
    static_assert(N % R == 0 && 64 % LPC == 0, "bad row split");
};

__device__ inline ChainInfo make_chain(int64_t c, int64_t nchunks, int64_t nch, int64_t K,
                                       int64_t T, bool reverse) {
    ChainInfo ci{0, 0, 0};
    if (c < nchunks) {
        const int64_t s = c / nch;
        const int64_t r = c - s * nch;
        const int64_t k = reverse ? nch - 1 - r : r;
        const int64_t t0 = k * K;
        const int64_t t1 = min(T, t0 + K);
        ci.base = s * T + t0;
        ci.len = int32_t(t1 > t0 ? t1 - t0 : 0);  // chunks past T (padding) are empty
        ci.t0 = int32_t(t0);
    }
    return ci;
}

template <int N, int R>
__device__ inline void set_identity_rows(float (&st)[R][N], int r0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] = (r0 + r == j) ? 1.f : 0.f;
}

template <int N, int R>
__device__ inline void set_zero_rows(float (&st)[R][N]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] = 0.f;
}

template <int N>
__device__ inline void load_matrix(float (&m)[N * N], const float* src) {
#pragma unroll
    for (int q = 0; q < N * N / 4; ++q) {
        const float4 v = reinterpret_cast<const float4*>(src)[q];
        m[4 * q + 0] = v.x;
        m[4 * q + 1] = v.y;
        m[4 * q + 2] = v.z;
        m[4 * q + 3] = v.w;
    }
}

template <int N>
__device__ inline void load_vec_lds(float (&v)[N], const float* src) {
#pragma unroll
    for (int q = 0; q < N / 4; ++q) {
        const float4 t = reinterpret_cast<const float4*>(src)[q];
        v[4 * q] = t.x;
        v[4 * q + 1] = t.y;
        v[4 * q + 2] = t.z;
        v[4 * q + 3] = t.w;
    }
}

// st <- st * m   (m row-major n-by-n in registers)
template <int N, int R>
__device__ inline void rows_times(float (&st)[R][N], const float (&m)[N * N]) {
    float o[R][N];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) o[r][j] = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < N; ++j) o[r][j] = fmaf(st[r][k], m[k * N + j], o[r][j]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] = o[r][j];
}

// st <- st * m^T   (m row-major n-by-n in registers)
template <int N, int R>
__device__ inline void rows_times_t(float (&st)[R][N], const float (&m)[N * N]) {
    float o[R][N];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) o[r][j] = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < N; ++j) o[r][j] = fmaf(st[r][k], m[j * N + k], o[r][j]);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] = o[r][j];
}

template <int N, int R>
__device__ inline void store_rows(float* dst, const float (&st)[R][N]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < N / 4; ++q)
            reinterpret_cast<float4*>(dst + r * N)[q] =
                make_float4(st[r][4 * q], st[r][4 * q + 1], st[r][4 * q + 2], st[r][4 * q + 3]);
}

template <int N, int R>
__device__ inline void load_rows(float (&st)[R][N], const float* src) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            const float4 v = reinterpret_cast<const float4*>(src + r * N)[q];
            st[r][4 * q] = v.x;
            st[r][4 * q + 1] = v.y;
            st[r][4 * q + 2] = v.z;
            st[r][4 * q + 3] = v.w;
        }
}

template <int N, int R>
__device__ inline void add_rows(float (&st)[R][N], const float* src) {
    float t[R][N];
    load_rows<N, R>(t, src);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] += t[r][j];
}

// The same with rows XR floats apart (the row-exchange buffers).
template <int N, int R, int XR>
__device__ inline void store_rows_x(float* dst, const float (&st)[R][N]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int q = 0; q < N / 4; ++q)
            reinterpret_cast<float4*>(dst + r * XR)[q] =
                make_float4(st[r][4 * q], st[r][4 * q + 1], st[r][4 * q + 2], st[r][4 * q + 3]);
}

template <int N, int XR>
__device__ inline void load_matrix_x(float (&m)[N * N], const float* src) {
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
        for (int q = 0; q < N / 4; ++q) {
            const float4 v = reinterpret_cast<const float4*>(src + i * XR)[q];
            m[i * N + 4 * q + 0] = v.x;
            m[i * N + 4 * q + 1] = v.y;
            m[i * N + 4 * q + 2] = v.z;
            m[i * N + 4 * q + 3] = v.w;
        }
}

// Workspace (look-back) accessors, element by element through ws_store /
// ws_load so that other XCDs see them coherently.
template <int N, int R>
__device__ inline void ws_store_rows(float* dst, const float (&st)[R][N]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) ws_store(dst + r * N + j, st[r][j]);
}

template <int N, int R>
__device__ inline void ws_load_rows(float (&st)[R][N], const float* src) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] = ws_load(src + r * N + j);
}

template <int N, int R>
__device__ inline void ws_add_rows(float (&st)[R][N], const float* src) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] += ws_load(src + r * N + j);
}

template <int N>
__device__ inline void ws_load_matrix(float (&m)[N * N], const float* src) {
#pragma unroll
    for (int q = 0; q < N * N; ++q) m[q] = ws_load(src + q);
}

// Staging of one block of TB tokens for every chain of the wave.  Token slot
// tau of chain ch holds global token  base + pos(tau) + shift, where
// pos(tau) = blk + tau going forward and len-1-(blk+tau) going backward, when
// that token lies inside the chunk (pos < len, pos >= 0) and inside the
// sequence (0 <= t0 + pos + shift < T).  Other slots hold the array's first
// token; the sweeps read them only into results they discard.
template <int N, int R, int TB, bool REV>
__device__ inline void stage_load(float4* reg, const float* src,
                                  const ChainInfo* info, int blk, int shift, int64_t T) {
    using V = Valu<N, R, TB>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < V::LD; ++i) {
        const int f = i * 64 + lane;
        const int ch = f / V::F4_BLK;
        const int off = f % V::F4_BLK;
        const int tau = off / V::F4_TOK;
        const int q = off % V::F4_TOK;
        const ChainInfo ci = info[ch];
        const int pos = REV ? ci.len - 1 - (blk + tau) : blk + tau;
        const int64_t tseq = int64_t(ci.t0) + pos + shift;
        const bool ok = (pos >= 0) & (pos < ci.len) & (tseq >= 0) & (tseq < T);
        // The load is unconditional (slots outside take token 0) and its value is
        // not touched until it is staged: a branch around the load, or a select on
        // its value, would make the compiler wait for it right here instead of
        // one block later.
        const int64_t tok = ok ? ci.base + pos + shift : 0;
        const float4 v = reinterpret_cast<const float4*>(src + tok * V::NN)[q];
        reg[i] = make_float4(v.x, v.y, v.z, v.w);
    }
}

template <int N, int R, int TB>
__device__ inline void stage_store(float* lds, const float4* reg) {
    using V = Valu<N, R, TB>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < V::LD; ++i) {
        const int f = i * 64 + lane;
        const int ch = f / V::F4_BLK;
        const int off = f % V::F4_BLK;
        reinterpret_cast<float4*>(lds + ch * V::CH_STRIDE)[off] = reg[i];
    }
}

// Scans that start from raw token vectors (FX) never form an input matrix.
// With X the staged token vector viewed n-by-n, M = L diag(e) U where L is unit
// lower with L_ij = X_ij (i > j), U unit upper with U_ij = X_ij (i < j) and
// e_k = exp(X_kk - mean_j X_jj) ("Improving Matrix Recurrent Units as an
// Attention Alternative", Key Points).  A row vector times L, diag(e), U in
// turn costs n(n-1)/2 + n + n(n-1)/2 = n^2 multiply-adds, the same as one
// times a dense M, so the fused scans do the same work as the plain ones and
// move x in place of M.
//
// stage_e: replaces the diagonal of every staged token by its e values (the
// diagonal of X is needed for nothing else), so a product reads the token's
// factors as one n-by-n block with full 16-byte loads.  A token's e values are
// shared out over 64/(G*TB) lanes (or a lane takes G*TB/64 whole tokens); each
// lane reads its token's diagonal once and forms the mean from it.  All of a
// token's reads precede its writes in the one wave's program order.
template <int N, int R, int TB>
__device__ inline void stage_e(float* lds) {
    using V = Valu<N, R, TB>;
    constexpr int TOKS = V::G * TB;                  // staged tokens of the wave
    constexpr int LPT = TOKS >= 64 ? 1 : 64 / TOKS;  // lanes per token
    constexpr int TPL = TOKS >= 64 ? TOKS / 64 : 1;  // tokens per lane
    constexpr int KPL = N / LPT;                     // e values per lane and token
    static_assert(TOKS % 64 == 0 || 64 % TOKS == 0, "tokens must tile the wave");
    static_assert(N % LPT == 0, "e values must split evenly over a token's lanes");
    const int lane = threadIdx.x & 63;
    const int part = lane % LPT;
#pragma unroll
    for (int u = 0; u < TPL; ++u) {
        const int tok = u * 64 + lane / LPT;
        float* X = lds + (tok / TB) * V::CH_STRIDE + (tok % TB) * V::NN;
        float d[N];
#pragma unroll
        for (int k = 0; k < N; ++k) d[k] = X[k * N + k];
        const float mean = ldu_mean_diag<N>(d);
#pragma unroll
        for (int kk = 0; kk < KPL; ++kk) {
            float v = d[kk];
#pragma unroll
            for (int h = 1; h < LPT; ++h) v = part == h ? d[h * KPL + kk] : v;
            const int k = part * KPL + kk;
            X[k * N + k] = expf(v - mean);
        }
    }
}

// st <- st * L, in place per row (L the unit lower factor held below x's
// diagonal): r_j += sum_{i > j} r_i X_ij, ascending j reads only untouched r_i.
template <int N, int R>
__device__ inline void rows_times_l(float (&st)[R][N], const float (&x)[N * N]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j)
#pragma unroll
            for (int i = j + 1; i < N; ++i) st[r][j] = fmaf(st[r][i], x[i * N + j], st[r][j]);
}

// st <- st * (L diag(e) U), in place per row; x holds L below, e on and U
// above the diagonal.
template <int N, int R>
__device__ inline void rows_times_ldu(float (&st)[R][N], const float (&x)[N * N]) {
    rows_times_l<N, R>(st, x);
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] *= x[j * N + j];
        // times U: r_j += sum_{k < j} r_k X_kj, descending j reads only untouched r_k
#pragma unroll
        for (int j = N - 1; j > 0; --j)
#pragma unroll
            for (int k = 0; k < j; ++k) st[r][j] = fmaf(st[r][k], x[k * N + j], st[r][j]);
    }
}

template <int N, int R>
__device__ inline void rows_times_ldu(float (&st)[R][N], const float* X) {
    float x[N * N];
    load_matrix<N>(x, X);
    rows_times_ldu<N, R>(st, x);
}

// st <- st * (L diag(e) U)^T = st * U^T diag(e) L^T, in place per row (x as
// for rows_times_ldu).
template <int N, int R>
__device__ inline void rows_times_ldu_t(float (&st)[R][N], const float (&x)[N * N]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        // times U^T: r_j += sum_{k > j} r_k X_jk, ascending j
#pragma unroll
        for (int j = 0; j < N; ++j)
#pragma unroll
            for (int k = j + 1; k < N; ++k) st[r][j] = fmaf(st[r][k], x[j * N + k], st[r][j]);
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] *= x[j * N + j];
        // times L^T: r_j += sum_{k < j} r_k X_jk, descending j
#pragma unroll
        for (int j = N - 1; j > 0; --j)
#pragma unroll
            for (int k = 0; k < j; ++k) st[r][j] = fmaf(st[r][k], x[j * N + k], st[r][j]);
    }
}

template <int N, int R>
__device__ inline void rows_times_ldu_t(float (&st)[R][N], const float* X) {
    float x[N * N];
    load_matrix<N>(x, X);
    rows_times_ldu_t<N, R>(st, x);
}

// Look-back aggregates (or backward maps) loaded per batch: their loads are in
// flight together (bounded by registers: n*n floats each per lane).
template <int N>
constexpr int kLookback = N == 4 ? 4 : 2;

// Scaled state (scaled forward scan): a chain's rows hold S with P = 2^ex S.
// renorm_rows multiplies S by a power of two (exact) so that its largest entry
// has magnitude in [0.5, 1) and adds the shift to ex; ex is the same in every
// lane of the chain.  An all-zero S is left as it is.
template <int N, int R>
__device__ inline void renorm_rows(float (&st)[R][N], int& ex) {
    int e = kNoExp;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) e = max_exp(e, st[r][j]);
    e = group_max<N / R>(e);
    if (e == kNoExp) return;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) st[r][j] = ldexpf(st[r][j], -e);
    ex += e;
}

// The lane's rows of a sequence's carried-in state (2^carry_exp * carry, or I).
template <int N, int R, bool SC>
__device__ inline void init_rows(float (&st)[R][N], int& ex, const ScanCarry& cy, int64_t s,
                                 int li) {
    ex = 0;
    if (!cy.carry) {
        set_identity_rows<N, R>(st, li * R);
        if constexpr (SC) renorm_rows<N, R>(st, ex);
        return;
    }
    load_rows<N, R>(st, cy.carry + s * N * N + li * R * N);
    const int ce = cy.carry_exp ? cy.carry_exp[s] : 0;
    if constexpr (SC) {
        ex = ce;
        renorm_rows<N, R>(st, ex);
    } else if (ce != 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int j = 0; j < N; ++j) st[r][j] = ldexpf(st[r][j], ce);
    }
}

// One sweep of a forward chain over its chunk: st <- st * M_t for each token,
// optionally storing the rows of every P_t.  With FX the input is x and each
// step multiplies by M_t's factors (stage_e puts each staged token's e on its
// diagonal).
template <int N, int R, int TB, bool WRITE, bool FX, bool SC>
__device__ __attribute__((always_inline)) void fwd_sweep(
    float (&st)[R][N], int& ex, const float* __restrict__ M, float* __restrict__ P,
    int32_t* __restrict__ pexp, float* lds, const ChainInfo* info, int g, int li, int maxlen,
    int64_t T) {
    using V = Valu<N, R, TB>;
    const ChainInfo me = info[g];
    float4 reg[V::LD];
    // One block.  FULL: every chain of the wave has all TB tokens of this block
    // and of the next, so the body has no data-dependent branches and the next
    // block is prefetched unconditionally; the compiler then waits for the
    // staged loads without waiting for the previous block's stores.
    auto block = [&](int blk, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        wave_lds_sync();
        stage_store<N, R, TB>(lds, reg);
        wave_lds_sync();
        if (FULL || blk + TB < maxlen) stage_load<N, R, TB, false>(reg, M, info, blk + TB, 0, T);
        if constexpr (FX) {
            stage_e<N, R, TB>(lds);
            wave_lds_sync();
        }
#pragma unroll
        for (int tau = 0; tau < TB; ++tau) {
            const int pos = blk + tau;
            if (FULL || pos < me.len) {
                const float* slot = lds + g * V::CH_STRIDE + tau * V::NN;
                if constexpr (FX) {
                    rows_times_ldu<N, R>(st, slot);
                } else {
                    float m[V::NN];
                    load_matrix<N>(m, slot);
                    rows_times<N, R>(st, m);
                }
                if constexpr (SC) renorm_rows<N, R>(st, ex);
                if (WRITE) {
                    store_rows<N, R>(P + (me.base + pos) * V::NN + li * R * N, st);
                    if (SC) pexp[me.base + pos] = ex;  // the same value from every lane of the chain
                }
            }
        }
    };
    int minlen = maxlen;
#pragma unroll
    for (int c = 0; c < V::G; ++c) minlen = min(minlen, info[c].len);
    const std::integral_constant<bool, true> full;
    const std::integral_constant<bool, false> partial;
    if (maxlen > 0) stage_load<N, R, TB, false>(reg, M, info, 0, 0, T);
    int blk = 0;
    if (blk + 2 * TB <= minlen) {
        // the first full block is peeled, so that the loop is entered only from
        // a full block (the same memory operations in flight on every entry)
        block(blk, full);
        for (blk += TB; blk + 2 * TB <= minlen; blk += TB) block(blk, full);
    }
    for (; blk < maxlen; blk += TB) block(blk, partial);
}

template <int N, int R, int TB, bool FX, bool SC>
__global__ __launch_bounds__(64) void fwd_valu_kernel(const float* __restrict__ M,
                                                      float* __restrict__ P, int64_t S, int64_t T,
                                                      int64_t K, int64_t nch, int64_t Z,
                                                      unsigned char* __restrict__ ws, ScanCarry cy) {
    using V = Valu<N, R, TB>;
    __shared__ __align__(16) float lds[V::G * V::CH_STRIDE];
    __shared__ __align__(16) float xch[V::G * V::QX_STRIDE];
    __shared__ ChainInfo info[V::G];
    __shared__ int aex[SC ? V::G : 1];
    const int lane = threadIdx.x;
    const int g = lane / V::LPC;
    const int li = lane % V::LPC;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    const int64_t cbase =
        multi ? ticket_to_chunk(int64_t(wave_ticket(&hdr->ticket)), S, nch / V::G, V::G)
              : int64_t(blockIdx.x) * V::G;
    if (lane < V::G) info[lane] = make_chain(cbase + lane, nchunks, nch, K, T, false);
    wave_lds_sync();
    int maxlen = 0;
#pragma unroll
    for (int i = 0; i < V::G; ++i) maxlen = max(maxlen, info[i].len);

    float st[R][N];
    int ex = 0;
    const int64_t c = cbase + g;
    const int64_t seq = c < nchunks ? c / nch : 0;  // idle chains read sequence 0, write nothing
    if (!multi) {
        init_rows<N, R, SC>(st, ex, cy, seq, li);
        fwd_sweep<N, R, TB, true, FX, SC>(st, ex, M, P, cy.out_exp, lds, info, g, li, maxlen, T);
        return;
    }

    // Multi-chunk: nch and Z are multiples of G, so the wave's G chunks lie in
    // one sequence and one super.
    const WsLayout L = ws_layout(nchunks, N, 4, 2);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.flags_off);
    float* agg = reinterpret_cast<float*>(ws + L.slot_off[0]);
    float* incl = reinterpret_cast<float*>(ws + L.slot_off[1]);
    int32_t* agg_exp = reinterpret_cast<int32_t*>(ws + L.exp_off);
    int32_t* incl_exp = agg_exp + nchunks;
    const int64_t k = c - (c / nch) * nch;
    const int64_t first = c - k % Z;  // first chunk of the super (same for the whole wave)
    const bool later_super = k >= Z;  // wave-uniform

    // 1. chunk aggregate (scaled scans: 2^a_ex times the normalised rows)
    set_identity_rows<N, R>(st, li * R);
    fwd_sweep<N, R, TB, false, FX, SC>(st, ex, M, P, cy.out_exp, lds, info, g, li, maxlen, T);
    const int a_ex = ex;
    ws_store_rows<N, R>(agg + c * V::NN + li * R * N, st);
    if (SC && li == 0) ws_store(&agg_exp[c], int32_t(a_ex));
    fence_release();
    if (li == 0) store_flag(&flags[c], kFlagAgg);
    // the wave's own aggregates also go to LDS, for its later chains
    wave_lds_sync();
    store_rows<N, R>(lds + g * V::CH_STRIDE + li * R * N, st);
    if (SC && li == 0) aex[g] = a_ex;

    // 2. product of the earlier aggregates of the super, left to right: those of
    // earlier waves (chunks first .. cbase-1) from the workspace, then those of
    // the wave's earlier chains (cbase .. c-1) from LDS
    wait_range_nonempty(flags, first, cbase, hdr);
    fence_acquire();
    float lrow[R][N];
    int l_ex = 0;
    set_identity_rows<N, R>(lrow, li * R);
    float m[V::NN];
    // workspace aggregates are loaded kLookback at a time (clamped into range) so
    // that their loads are in flight together; the products stay in order
    for (int64_t j0 = first; j0 < cbase; j0 += kLookback<N>) {
        float mb[kLookback<N>][V::NN];
        int eb[kLookback<N>];
#pragma unroll
        for (int d = 0; d < kLookback<N>; ++d) {
            const int64_t j = min(j0 + d, cbase - 1);
            ws_load_matrix<N>(mb[d], agg + j * V::NN);
            if constexpr (SC) eb[d] = ws_load(&agg_exp[j]);
        }
#pragma unroll
        for (int d = 0; d < kLookback<N>; ++d)
            if (j0 + d < cbase) {
                rows_times<N, R>(lrow, mb[d]);
                if constexpr (SC) {
                    l_ex += eb[d];
                    renorm_rows<N, R>(lrow, l_ex);
                }
            }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < V::G - 1; ++j)
        if (j < g) {
            load_matrix<N>(m, lds + j * V::CH_STRIDE);
            rows_times<N, R>(lrow, m);
            if constexpr (SC) {
                l_ex += aex[j];
                renorm_rows<N, R>(lrow, l_ex);
            }
        }
    wave_lds_sync();  // the LDS is the staging buffer again in step 4

    // 3. carry = (prefix of the previous super, or the carried-in state) * lrow
    if (later_super || cy.carry) {  // wave-uniform
        store_rows<N, R>(xch + g * V::QX_STRIDE + li * R * N, lrow);
        if (later_super) {
            wait_flag_eq(&flags[first - 1], kFlagPrefix, hdr);
            fence_acquire();
        }
        wave_lds_sync();
        load_matrix<N>(m, xch + g * V::QX_STRIDE);
        if (later_super) {
            ws_load_rows<N, R>(st, incl + (first - 1) * V::NN + li * R * N);
            ex = SC ? ws_load(&incl_exp[first - 1]) : 0;
        } else {
            init_rows<N, R, SC>(st, ex, cy, seq, li);
        }
        rows_times<N, R>(st, m);
        if constexpr (SC) {
            ex += l_ex;
            renorm_rows<N, R>(st, ex);
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < N; ++q) st[r][q] = lrow[r][q];
        ex = l_ex;
    }
    const bool boundary = (k % Z == Z - 1) && (k + 1 < nch);
    if (boundary) {
        float inc[R][N];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < N; ++q) inc[r][q] = st[r][q];
        ws_load_matrix<N>(m, agg + c * V::NN);
        rows_times<N, R>(inc, m);
        int i_ex = ex + a_ex;
        if constexpr (SC) renorm_rows<N, R>(inc, i_ex);
        ws_store_rows<N, R>(incl + c * V::NN + li * R * N, inc);
        if (SC && li == 0) ws_store(&incl_exp[c], int32_t(i_ex));
    }
    fence_release();
    if (boundary && li == 0) store_flag(&flags[c], kFlagPrefix);

    // 4. re-run the chunk from its carry and write every prefix
    fwd_sweep<N, R, TB, true, FX, SC>(st, ex, M, P, cy.out_exp, lds, info, g, li, maxlen, T);
}

// ---------------------------------------------------------------------------- backward

// Sum over aligned groups of W (1, 2, 4 or 8) lanes with DPP moves: swap
// neighbours, swap pairs, then mirror the halves of each 8-lane group.  Every
// lane of a group gets the same value (each step adds two values in either
// order, and a + b == b + a).
template <int W>
__device__ inline float group_sum(float v) {
    static_assert(W == 1 || W == 2 || W == 4 || W == 8, "groups of at most 8 lanes");
    if constexpr (W >= 2)  // quad_perm [1, 0, 3, 2]
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    if constexpr (W >= 4)  // quad_perm [2, 3, 0, 1]
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    if constexpr (W >= 8)  // row_half_mirror
        v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    return v;
}

// The lane's rows a = a0 .. a0+R-1 of dL/dX_t, the gradient through the LDU
// build of M_t ("Improving Matrix Recurrent Units as an Attention
// Alternative", Key Points: LDU fill, determinant-correcting scalar), from its
// rows of G = dL/dM_t (d) and of L^T G (u).  x holds the token's factors (L
// below, e on and U above the diagonal); xa points at row a0 of the same
// matrix in LDS.  With H = G U^T and g_k = (L^T G U^T)_kk:
//   dX_aj = e_j H_aj (j < a),  e_a (L^T G)_aj (j > a),  e_a g_a - mean_k e_k g_k (j = a);
// the mean's derivative is the determinant correction's.  W = lanes per chain.
template <int N, int R, int W>
__device__ inline void dx_rows(float (&out)[R][N], const float (&d)[R][N], const float (&u)[R][N],
                               const float (&x)[N * N], const float* xa, int a0) {
    float seg[R], part = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int a = a0 + r;
        float xr[N];
        load_vec_lds<N>(xr, xa + r * N);  // row a of x: U_aj above, e_a on the diagonal
        float ea = 0.f, g = 0.f;
#pragma unroll
        for (int j = 0; j < N; ++j) {
            ea = j == a ? xr[j] : ea;
            const float uj = j > a ? xr[j] : (j == a ? 1.f : 0.f);  // U_aj
            g = fmaf(uj, u[r][j], g);
        }
        seg[r] = ea * g;
        part += seg[r];
#pragma unroll
        for (int j = 0; j < N; ++j) {
            // H_aj = G_aj + sum_{m > j} G_am U_jm
            float h = d[r][j];
#pragma unroll
            for (int m = j + 1; m < N; ++m) h = fmaf(d[r][m], x[j * N + m], h);
            out[r][j] = j < a ? x[j * N + j] * h : ea * u[r][j];
        }
    }
    const float mean = group_sum<W>(part) * (1.0f / N);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < N; ++j) out[r][j] = j == a0 + r ? seg[r] - mean : out[r][j];
}

// One reverse sweep over the chunk, from its last token down, TB tokens per
// staged block.  A block stages M_t (x_t) and dP_t of its own tokens; M_{t+1}
// of a token is the slot staged before it, and for the block's first token the
// previous block's last slot, kept per chain in nx (before the first block: the
// token after the chunk, when the sequence has one).
//   AGG pass  (GRAD = false): q <- dP_t + q M_{t+1}^T and w <- w M_{t+1}^T, from
//             q = 0, w = I; afterwards q is the chunk's local adjoint at its first
//             token and w the rows of (M_{a+1} ... M_{b+1})^T.
//   GRAD pass (GRAD = true):  q <- dP_t + q M_{t+1}^T from the carry, and
//             dM_t = P_{t-1}^T Q_t written for the lane's rows.  From M (FX
//             false) every P_{t-1} is read from P, which is an input of the
//             call.  From raw token vectors (FX) only the prefix just before
//             each block's lowest token is read; the block's other P_{t-1} are
//             recomputed from it by the forward recurrence P_t = P_{t-1} M_t,
//             with the same products as the forward scan (bit for bit the
//             stored prefixes when the forward ran one chunk per sequence, equal
//             up to rounding otherwise).  This reads n^2 floats per block
//             instead of per token.  With DX the output is dL/dx_t instead of
//             dM_t (dx_rows), from the exchanged rows of P_{t-1} L_t as well.
// At the last token of a sequence there is no M_{t+1}: q <- dP_t.
template <int N, int R, int TB, bool GRAD, bool FX, bool DX>
__device__ __attribute__((always_inline)) void bwd_sweep(
    float (&q)[R][N], float (&w)[R][N], const float* __restrict__ M, const float* __restrict__ P,
    const float* __restrict__ dP, float* __restrict__ dM, float* lds, float* nx, float* qx,
    const ChainInfo* info, int g, int li, int maxlen, int64_t T, const ScanCarry& cy) {
    using V = Valu<N, R, TB>;
    constexpr bool RP = !FX;     // read every prefix (else one per block)
    constexpr int NCK = RP ? TB : 1;
    const ChainInfo me = info[g];
    const int64_t s0 = me.base - me.t0;  // token index of the sequence's first token
    const int64_t seq = s0 / T;          // its sequence
    float* const xl = lds + g * V::CH_STRIDE;                          // staged M_t
    float* const rl = lds + V::G * V::CH_STRIDE + g * V::CH_STRIDE;    // staged dP_t
    float* const nxg = nx + g * V::NX_STRIDE;                          // M_{t+1}
    float* const qxg = qx + g * V::QX_STRIDE;                          // Q_t rows
    float* const pxg = qx + (V::G + g) * V::QX_STRIDE;                 // P_{t-1} rows
    float* const lxg = qx + (2 * V::G + g) * V::QX_STRIDE;             // DX: P_{t-1} L_t rows
    float4 rm[V::LD], rr[V::LD];
    // rows of the prefixes of the next block: RP, P_{t-1} of its tokens
    // tau = 0 .. TB-1; else the prefix just before its lowest token
    float ck[NCK][R][N];
    bool ck_id[NCK];
    // Rows of P_{tc} at token tc of the sequence: P itself inside the sequence,
    // else P_0 (the carried-in state, or I).  The load is unconditional from a
    // valid address.
    auto load_prefix = [&](int u, int rel) {  // rel: token position in the chunk (>= 0)
        const int64_t tc = int64_t(me.t0) + rel - 1;
        const float* src = P;  // idle chains (a padding chunk may lie past the array)
        if (me.len > 0) {
            if (tc >= 0) src = P + (me.base + rel - 1) * V::NN;
            else if (cy.carry) src = cy.carry + seq * V::NN;
        }
        ck_id[u] = tc < 0 && !cy.carry;
        load_rows<N, R>(ck[u], src + li * R * N);
    };
    auto load_checkpoint = [&](int blk) {
        if constexpr (RP) {
#pragma unroll
            for (int tau = 0; tau < TB; ++tau) load_prefix(tau, max(me.len - 1 - blk - tau, 0));
        } else {
            load_prefix(0, max(me.len - blk - TB, 0));
        }
    };
    auto load_block = [&](int blk) {
        stage_load<N, R, TB, true>(rm, M, info, blk, 0, T);
        stage_load<N, R, TB, true>(rr, dP, info, blk, 0, T);
        if constexpr (GRAD) load_checkpoint(blk);
    };
    {
        // M_{t+1} of the chunk's last token
        float t[R][N];
        if (me.len > 0 && int64_t(me.t0) + me.len < T)
            load_rows<N, R>(t, M + (me.base + me.len) * V::NN + li * R * N);
        else
            set_zero_rows<N, R>(t);
        store_rows<N, R>(nxg + li * R * N, t);
        if constexpr (FX) {
            // its e on the diagonal, as stage_e does for staged tokens
            wave_lds_sync();
            const float mean = ldu_mean<N>(nxg);
            float e[R];
#pragma unroll
            for (int r = 0; r < R; ++r) e[r] = expf(nxg[(li * R + r) * (N + 1)] - mean);
            wave_lds_sync();
#pragma unroll
            for (int r = 0; r < R; ++r) nxg[(li * R + r) * (N + 1)] = e[r];
        }
    }
    // One block.  FULL: every chain of the wave has all TB tokens and none is
    // its sequence's first, so the body has no data-dependent branches and the
    // next block is prefetched unconditionally; the compiler then knows how many
    // memory operations follow each load and waits for the staged loads
    // without waiting for the previous block's dM stores.
    auto block = [&](int blk, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        wave_lds_sync();
        stage_store<N, R, TB>(lds, rm);
        stage_store<N, R, TB>(lds + V::G * V::CH_STRIDE, rr);
        float cur[NCK][R][N];
        if constexpr (GRAD) {
#pragma unroll
            for (int u = 0; u < NCK; ++u)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < N; ++j)
                        cur[u][r][j] = ck_id[u] ? (li * R + r == j ? 1.f : 0.f) : ck[u][r][j];
        }
        wave_lds_sync();
        if (FULL || blk + TB < maxlen) load_block(blk + TB);
        if constexpr (FX) {
            stage_e<N, R, TB>(lds);
            wave_lds_sync();
        }
        // rp[tau]: the lane's rows of P_{t-1} for the block's token tau, from the
        // block's lowest live token (tau = min(TB-1, hi)) upward
        float rp[GRAD ? TB : 1][R][N];
        if constexpr (GRAD && RP) {
#pragma unroll
            for (int tau = 0; tau < TB; ++tau)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < N; ++j) rp[tau][r][j] = cur[tau][r][j];
        } else if constexpr (GRAD) {
            const int hi = me.len - 1 - blk;
#pragma unroll
            for (int tau = TB - 1; tau >= 0; --tau) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int j = 0; j < N; ++j) rp[tau][r][j] = tau == TB - 1 ? cur[0][r][j] : rp[tau + 1][r][j];
                if (tau < TB - 1) {
                    // P_{t-1} of token tau = P_{t-1} of token tau+1 times M_t of token tau+1
                    const float* slot = xl + (tau + 1) * V::NN;
                    if constexpr (FX) {
                        rows_times_ldu<N, R>(rp[tau], slot);
                    } else {
                        float m[V::NN];
                        load_matrix<N>(m, slot);
                        rows_times<N, R>(rp[tau], m);
                    }
                    if (!FULL && tau >= hi)
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int j = 0; j < N; ++j) rp[tau][r][j] = cur[0][r][j];
                }
            }
        }
#pragma unroll
        for (int tau = 0; tau < TB; ++tau) {
            const int i = blk + tau;
            const int pos = me.len - 1 - i;
            const bool live = FULL || i < me.len;
            const int64_t tseq = int64_t(me.t0) + pos;
            const float* mslot = tau == 0 ? nxg : xl + (tau - 1) * V::NN;
            if (live) {
                if (FULL || tseq + 1 < T) {
                    if constexpr (FX) {
                        float x[V::NN];
                        load_matrix<N>(x, mslot);
                        rows_times_ldu_t<N, R>(q, x);
                        if (!GRAD) rows_times_ldu_t<N, R>(w, x);
                    } else {
                        float m[V::NN];
                        load_matrix<N>(m, mslot);
                        rows_times_t<N, R>(q, m);
                        if (!GRAD) rows_times_t<N, R>(w, m);
                    }
                }
                if (FULL || tseq + 1 >= T) {
                    // the sequence's last token has no M_{t+1} (a select, not a branch)
                    const bool last = tseq + 1 >= T;
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int j = 0; j < N; ++j) q[r][j] = last ? 0.f : q[r][j];
                }
                add_rows<N, R>(q, rl + tau * V::NN + li * R * N);
            }
            if constexpr (GRAD) {
                // DX: the rows of P_{t-1} L_t (L_t the unit lower factor of M_t)
                // as well; (L^T G)[a][:] = sum_i (P_{t-1} L_t)[i][a] Q_t[i][:]
                // comes from them as G's rows come from P_{t-1}'s.
                float pl[DX ? R : 1][N];
                float xt[DX ? V::NN : 1];  // DX: M_t's factors (its lower part dies here)
                if constexpr (DX) {
                    if (live) {
                        load_matrix<N>(xt, xl + tau * V::NN);
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int j = 0; j < N; ++j) pl[r][j] = rp[tau][r][j];
                        rows_times_l<N, R>(pl, xt);
                    }
                }
                // exchange the rows of Q_t and P_{t-1} within the chain, then
                // dM rows a = own rows: dM[a][:] = sum_i P_{t-1}[i][a] Q_t[i][:]
                wave_lds_sync();
                if (live) {
                    store_rows_x<N, R, V::XR>(qxg + li * R * V::XR, q);
                    store_rows_x<N, R, V::XR>(pxg + li * R * V::XR, rp[tau]);
                    if constexpr (DX) store_rows_x<N, R, V::XR>(lxg + li * R * V::XR, pl);
                }
                wave_lds_sync();
                if (live) {
                    float d[R][N], u[DX ? R : 1][N];
                    if (DX || FULL || tseq > 0 || cy.carry) {
                        float qa[V::NN];
                        load_matrix_x<N, V::XR>(qa, qxg);
                        set_zero_rows<N, R>(d);
                        if constexpr (DX) set_zero_rows<N, R>(u);
#pragma unroll
                        for (int ii = 0; ii < N; ++ii) {
                            float pc[R], lc[R];
#pragma unroll
                            for (int r = 0; r < R; ++r) pc[r] = pxg[ii * V::XR + li * R + r];
                            if constexpr (DX)
#pragma unroll
                                for (int r = 0; r < R; ++r) lc[r] = lxg[ii * V::XR + li * R + r];
#pragma unroll
                            for (int r = 0; r < R; ++r)
#pragma unroll
                                for (int j = 0; j < N; ++j) {
                                    d[r][j] = fmaf(pc[r], qa[ii * N + j], d[r][j]);
                                    if constexpr (DX) u[r][j] = fmaf(lc[r], qa[ii * N + j], u[r][j]);
                                }
                        }
                    } else {
                        // P_0 = I
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int j = 0; j < N; ++j) d[r][j] = q[r][j];
                    }
                    if constexpr (DX) {
                        float o[R][N];
                        dx_rows<N, R, V::LPC>(o, d, u, xt, xl + tau * V::NN + li * R * N, li * R);
                        store_rows<N, R>(dM + (me.base + pos) * V::NN + li * R * N, o);
                    } else {
                        store_rows<N, R>(dM + (me.base + pos) * V::NN + li * R * N, d);
                    }
                    if (!FULL && tseq == 0 && cy.dcarry) {
                        // dL/dP_0 = Q_1 M_1^T, M_1 this token's input
                        float dc[R][N];
#pragma unroll
                        for (int r = 0; r < R; ++r)
#pragma unroll
                            for (int j = 0; j < N; ++j) dc[r][j] = q[r][j];
                        const float* m1 = M + s0 * V::NN;
                        if constexpr (FX) {
                            float x[V::NN];
                            load_matrix<N>(x, m1);
                            const float mean = ldu_mean<N>(m1);
#pragma unroll
                            for (int kk = 0; kk < N; ++kk) x[kk * (N + 1)] = expf(x[kk * (N + 1)] - mean);
                            rows_times_ldu_t<N, R>(dc, x);
                        } else {
                            float mm[V::NN];
                            load_matrix<N>(mm, m1);
                            rows_times_t<N, R>(dc, mm);
                        }
                        store_rows<N, R>(cy.dcarry + seq * V::NN + li * R * N, dc);
                    }
                }
            }
        }
        // the block's last slot (e on its diagonal) is M_{t+1} of the next
        // block's first token
        {
            float t[R][N];
            load_rows<N, R>(t, xl + (TB - 1) * V::NN + li * R * N);
            store_rows<N, R>(nxg + li * R * N, t);
        }
    };
    int minlen = maxlen;
#pragma unroll
    for (int c = 0; c < V::G; ++c) minlen = min(minlen, info[c].len);
    const std::integral_constant<bool, true> full;
    const std::integral_constant<bool, false> partial;
    if (maxlen > 0) load_block(0);
    int blk = 0;
    // full blocks end one token short of the shortest chain: the first token of
    // a sequence is handled by the partial body
    if (blk + TB < minlen) {
        // the first full block is peeled, so that the loop is entered only from
        // a full block (the same memory operations in flight on every entry)
        block(blk, full);
        for (blk += TB; blk + TB < minlen; blk += TB) block(blk, full);
    }
    for (; blk < maxlen; blk += TB) block(blk, partial);
}

// DX at n = 8 runs alone on its SIMD at the shapes it is for (one chain per
// sequence), so it may use the whole register file (AGPRs included) instead
// of spilling; the other instances keep the default occupancy target.
template <int N, int R, int TB, bool FX, bool DX>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, DX && N == 8 ? 1 : 8)))
void bwd_valu_kernel(const float* __restrict__ M, const float* __restrict__ P,
                     const float* __restrict__ dP, float* __restrict__ dM, int64_t S, int64_t T,
                     int64_t K, int64_t nch, int64_t Z, unsigned char* __restrict__ ws,
                     ScanCarry cy) {
    using V = Valu<N, R, TB>;
    __shared__ __align__(16) float lds[2 * V::G * V::CH_STRIDE];
    __shared__ __align__(16) float nx[V::G * V::NX_STRIDE];
    __shared__ __align__(16) float qx[(DX ? 3 : 2) * V::G * V::QX_STRIDE];
    __shared__ ChainInfo info[V::G];
    static_assert(V::CH_STRIDE >= 2 * V::NN, "a chain's staging slot holds its map (W^T and Bl)");
    const int lane = threadIdx.x;
    const int g = lane / V::LPC;
    const int li = lane % V::LPC;
    const int64_t nchunks = S * nch;
    const bool multi = nch > 1;
    WsHeader* hdr = reinterpret_cast<WsHeader*>(ws);
    const int64_t cbase =
        multi ? ticket_to_chunk(int64_t(wave_ticket(&hdr->ticket)), S, nch / V::G, V::G)
              : int64_t(blockIdx.x) * V::G;
    if (lane < V::G) info[lane] = make_chain(cbase + lane, nchunks, nch, K, T, true);
    wave_lds_sync();
    int maxlen = 0;
#pragma unroll
    for (int i = 0; i < V::G; ++i) maxlen = max(maxlen, info[i].len);

    float q[R][N], w[R][N];
    set_zero_rows<N, R>(q);
    set_identity_rows<N, R>(w, li * R);
    if (!multi) {
        bwd_sweep<N, R, TB, true, FX, DX>(q, w, M, P, dP, dM, lds, nx, qx, info, g, li, maxlen, T, cy);
        return;
    }

    // Chunks run in reverse token order: position r = 0 is the sequence's last
    // chunk.  The carry of a chunk is the adjoint Q at the first token of the
    // next chunk (in token order); each chunk's map is Y -> Bl + Y W^T.
    const WsLayout L = ws_layout(nchunks, N, 4, 3);
    uint32_t* flags = reinterpret_cast<uint32_t*>(ws + L.flags_off);
    float* swt = reinterpret_cast<float*>(ws + L.slot_off[0]);   // rows of W^T
    float* sbl = reinterpret_cast<float*>(ws + L.slot_off[1]);   // rows of the local adjoint Bl
    float* sinc = reinterpret_cast<float*>(ws + L.slot_off[2]);  // rows of the true adjoint
    const int64_t c = cbase + g;
    const int64_t r = c - (c / nch) * nch;
    const int64_t first = c - r % Z;
    const bool later_super = r >= Z;

    // 1. affine aggregate of the chunk
    bwd_sweep<N, R, TB, false, FX, DX>(q, w, M, P, dP, dM, lds, nx, qx, info, g, li, maxlen, T, cy);
    ws_store_rows<N, R>(sbl + c * V::NN + li * R * N, q);
    ws_store_rows<N, R>(swt + c * V::NN + li * R * N, w);
    fence_release();
    if (li == 0) store_flag(&flags[c], kFlagAgg);
    // the wave's own maps also go to LDS (W^T, then Bl), for its later chains
    wave_lds_sync();
    store_rows<N, R>(lds + g * V::CH_STRIDE + li * R * N, w);
    store_rows<N, R>(lds + g * V::CH_STRIDE + V::NN + li * R * N, q);

    // 2. compose the maps of the earlier chunks of the super (first applied
    // first): those of earlier waves from the workspace, then those of the
    // wave's earlier chains from LDS
    wait_range_nonempty(flags, first, cbase, hdr);
    fence_acquire();
    float wc[R][N], bc[R][N];
    set_identity_rows<N, R>(wc, li * R);
    set_zero_rows<N, R>(bc);
    float m[V::NN];
    // workspace maps loaded kLookback at a time (clamped into range), composed in order
    for (int64_t j0 = first; j0 < cbase; j0 += kLookback<N>) {
        float mb[kLookback<N>][V::NN], bb[kLookback<N>][R][N];
#pragma unroll
        for (int d = 0; d < kLookback<N>; ++d) {
            const int64_t j = min(j0 + d, cbase - 1);
            ws_load_matrix<N>(mb[d], swt + j * V::NN);
            ws_load_rows<N, R>(bb[d], sbl + j * V::NN + li * R * N);
        }
#pragma unroll
        for (int d = 0; d < kLookback<N>; ++d)
            if (j0 + d < cbase) {
                if (later_super) rows_times<N, R>(wc, mb[d]);
                rows_times<N, R>(bc, mb[d]);
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int q = 0; q < N; ++q) bc[r][q] += bb[d][r][q];
            }
    }
    wave_lds_sync();
#pragma unroll
    for (int j = 0; j < V::G - 1; ++j)
        if (j < g) {
            float bj[R][N];
            load_matrix<N>(m, lds + j * V::CH_STRIDE);
            load_rows<N, R>(bj, lds + j * V::CH_STRIDE + V::NN + li * R * N);
            if (later_super) rows_times<N, R>(wc, m);
            rows_times<N, R>(bc, m);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int q = 0; q < N; ++q) bc[r][q] += bj[r][q];
        }
    wave_lds_sync();  // the LDS is the staging buffer again in step 4

    // 3. carry = Y Wc^T + Bc with Y the adjoint published by the previous super
    if (later_super) {
        wait_flag_eq(&flags[first - 1], kFlagPrefix, hdr);
        fence_acquire();
        store_rows<N, R>(qx + g * V::QX_STRIDE + li * R * N, wc);
        wave_lds_sync();
        load_matrix<N>(m, qx + g * V::QX_STRIDE);
        ws_load_rows<N, R>(q, sinc + (first - 1) * V::NN + li * R * N);
        rows_times<N, R>(q, m);
#pragma unroll
        for (int a = 0; a < R; ++a)
#pragma unroll
            for (int b = 0; b < N; ++b) q[a][b] += bc[a][b];
        wave_lds_sync();
    } else {
#pragma unroll
        for (int a = 0; a < R; ++a)
#pragma unroll
            for (int b = 0; b < N; ++b) q[a][b] = bc[a][b];
    }
    const bool boundary = (r % Z == Z - 1) && (r + 1 < nch);
    if (boundary) {
        float inc[R][N];
#pragma unroll
        for (int a = 0; a < R; ++a)
#pragma unroll
            for (int b = 0; b < N; ++b) inc[a][b] = q[a][b];
        ws_load_matrix<N>(m, swt + c * V::NN);
        rows_times<N, R>(inc, m);
        ws_add_rows<N, R>(inc, sbl + c * V::NN + li * R * N);
        ws_store_rows<N, R>(sinc + c * V::NN + li * R * N, inc);
    }
    fence_release();
    if (boundary && li == 0) store_flag(&flags[c], kFlagPrefix);

    // 4. re-run the chunk from the carry and write dM
    bwd_sweep<N, R, TB, true, FX, DX>(q, w, M, P, dP, dM, lds, nx, qx, info, g, li, maxlen, T, cy);
}

template <int N, int R, int TB, bool FX, bool SC>
hipError_t run_fwd(const float* M, float* P, int64_t S, int64_t T, int64_t K, int64_t nch,
                   int64_t Z, void* ws, hipStream_t stream, const ScanCarry& cy) {
    using V = Valu<N, R, TB>;
    const int64_t waves = (S * nch + V::G - 1) / V::G;
    hipLaunchKernelGGL((fwd_valu_kernel<N, R, TB, FX, SC>), dim3(unsigned(waves)), dim3(64), 0,
                       stream, M, P, S, T, K, nch, Z, static_cast<unsigned char*>(ws), cy);
    return hipGetLastError();
}

template <int N, int R, int TB, bool FX>
hipError_t run_fwd_any(const float* M, float* P, int64_t S, int64_t T, int64_t K, int64_t nch,
                       int64_t Z, void* ws, hipStream_t stream, const ScanCarry& cy) {
    if (cy.out_exp) return run_fwd<N, R, TB, FX, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
    return run_fwd<N, R, TB, FX, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
}

template <int N, int R, int TB, bool FX, bool DX>
hipError_t run_bwd(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                   int64_t T, int64_t K, int64_t nch, int64_t Z, void* ws, hipStream_t stream,
                   const ScanCarry& cy) {
    using V = Valu<N, R, TB>;
    const int64_t waves = (S * nch + V::G - 1) / V::G;
    hipLaunchKernelGGL((bwd_valu_kernel<N, R, TB, FX, DX>), dim3(unsigned(waves)), dim3(64), 0,
                       stream, M, P, dP, dM, S, T, K, nch, Z, static_cast<unsigned char*>(ws), cy);
    return hipGetLastError();
}

}  // namespace

// Row split and staging depth per n and direction: one row of the state per
// lane (R = 1: more waves for the same vector work, measured best) and TB
// tokens per staged block (forward 8 at n = 4, 4 at n = 8; backward 4).
#define MRU_VALU_CFG4 4, 1, 8
#define MRU_VALU_CFG8 8, 1, 4
#define MRU_VALU_BWD_CFG4 4, 1, 4
#define MRU_VALU_BWD_CFG8 8, 1, 4

int valu_chains_per_wave(int n, int dir) {
    if (n == 4) return dir == 0 ? Valu<MRU_VALU_CFG4>::G : Valu<MRU_VALU_BWD_CFG4>::G;
    return dir == 0 ? Valu<MRU_VALU_CFG8>::G : Valu<MRU_VALU_BWD_CFG8>::G;
}

hipError_t launch_fwd_valu(const float* M, float* P, int64_t S, int64_t T, int n, int64_t K,
                           int64_t nch, int64_t Z, void* ws, hipStream_t stream, bool from_x,
                           const ScanCarry& cy) {
    if (n == 4) {
        if (from_x) return run_fwd_any<MRU_VALU_CFG4, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
        return run_fwd_any<MRU_VALU_CFG4, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
    }
    if (n == 8) {
        if (from_x) return run_fwd_any<MRU_VALU_CFG8, true>(M, P, S, T, K, nch, Z, ws, stream, cy);
        return run_fwd_any<MRU_VALU_CFG8, false>(M, P, S, T, K, nch, Z, ws, stream, cy);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_valu(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                           int64_t T, int n, int64_t K, int64_t nch, int64_t Z, void* ws,
                           hipStream_t stream, bool from_x, bool to_dx, const ScanCarry& cy) {
    if (to_dx && !from_x) return hipErrorInvalidValue;
    if (n == 4) {
        if (to_dx)
            return run_bwd<MRU_VALU_BWD_CFG4, true, true>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        if (from_x)
            return run_bwd<MRU_VALU_BWD_CFG4, true, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        return run_bwd<MRU_VALU_BWD_CFG4, false, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
    }
    if (n == 8) {
        if (to_dx)
            return run_bwd<MRU_VALU_BWD_CFG8, true, true>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        if (from_x)
            return run_bwd<MRU_VALU_BWD_CFG8, true, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
        return run_bwd<MRU_VALU_BWD_CFG8, false, false>(M, P, dP, dM, S, T, K, nch, Z, ws, stream, cy);
    }
    return hipErrorInvalidValue;
}

}  // namespace mru
