/*
 * mru.h -- C ABI of the MRU prefix-scan library (libmru.so, gfx950 / MI355X).
 *
 * Matrix Recurrent Units turn every token's vector into an n-by-n "input state
 * matrix", multiply those matrices one after another along the sequence (the
 * running product is the "output state matrix"), and turn each running product
 * back into a vector.  Matrix multiplication is associative, which is what lets
 * the running product be computed as a parallel scan instead of a serial loop.
 *   Source: "MRU Update: An independent developer's alternative to Attention is
 *   now running successfully", section "What MRU Actually Does".
 * The input state matrix is built by LDU factor filling with a
 * determinant-correcting scalar.
 *   Source: "Improving Matrix Recurrent Units as an Attention Alternative",
 *   Key Points.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Shapes      B (batch), H (heads), T (tokens) >= 0; n in {4, 8, 16, 32}.
 *             S = B*H independent sequences.
 * Layout      dense, contiguous, row-major fp32 device arrays [B][H][T][n][n];
 *             a raw token vector x is the same bytes viewed as [B][H][T][n*n]
 *             and an output vector is P viewed as [B][H][T][n*n] (row-major
 *             flatten, heads kept separate).  Every pointer must be 16-byte
 *             aligned.
 * Ownership   the caller allocates and frees every buffer, including the
 *             workspace (size from mru_scan_workspace_bytes).  The library
 *             allocates no device memory and keeps no mutable global state;
 *             calls are re-entrant.  Two calls that run at the same time need
 *             distinct workspaces.
 * Streams     all work is enqueued on `stream` (a hipStream_t; NULL = the
 *             default stream) and the call returns without synchronising.
 *             Device-side faults surface at the caller's next synchronisation.
 * Errors      every argument is validated on the host before anything is
 *             enqueued; a non-OK status means nothing was launched.  An empty
 *             problem (B*H*T == 0) returns MRU_OK without launching.  The
 *             library never prints, aborts or exits.
 * Arithmetic  inputs and outputs are IEEE fp32.  The running product is kept
 *             in fp32 for n = 4, 8 and in fp64 for n = 16, 32.  Values beyond
 *             the fp32 range become +-inf / nan exactly as IEEE arithmetic
 *             gives them: nothing is clamped or renormalised, except in the
 *             scaled form of mru_scan_fwd_ex, which writes each P_t as a power
 *             of two times a normalised matrix.
 */
#ifndef MRU_H
#define MRU_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MRU_ABI_VERSION 2

typedef enum mru_status {
    MRU_OK = 0,
    MRU_ERR_NULL = 1,       /* a required pointer is NULL                         */
    MRU_ERR_SHAPE = 2,      /* B, H or T negative, n not in {4,8,16,32}, overflow,
                               or an option the entry point does not support     */
    MRU_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned (exponent arrays:
                               4-byte)                                            */
    MRU_ERR_ALIAS = 4,      /* an output overlaps an input or another output      */
    MRU_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than required            */
    MRU_ERR_CHUNK = 6,      /* chunk < 0                                          */
    MRU_ERR_HIP = 7,        /* the HIP runtime reported an error at launch        */
    MRU_ERR_TIMEOUT = 8     /* never returned by a call: the code bindings raise
                               when mru_scan_ws_status reports
                               MRU_WS_STATUS_SPIN_TIMEOUT                         */
} mru_status;

/* Bits of the workspace status word (mru_scan_ws_status). */
#define MRU_WS_STATUS_SPIN_TIMEOUT 1u /* a look-back wait gave up: outputs invalid */

/* Scan direction for the workspace / chunk queries. */
#define MRU_DIR_FWD 0
#define MRU_DIR_BWD 1
/* The forward from raw token vectors, for mru_scan_chunk and mru_scan_plan (its
 * automatic plan may differ from the scan from M's). */
#define MRU_DIR_FWD_X 2

/* Orthogonal input constructions (mru_build_orthogonal). */
#define MRU_ORTHO_CAYLEY 0
#define MRU_ORTHO_EXPM 1

/* MRU_ABI_VERSION of the loaded library. */
int32_t mru_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* mru_status_string(int32_t status);

/*
 * Input state matrices from raw token vectors (LDU fill + determinant
 * correction).  Source: "Improving Matrix Recurrent Units as an Attention
 * Alternative", Key Points.
 *
 * x  [B][H][T][n*n] fp32, read.  Viewed row-major as X (n-by-n): the strictly
 *    lower part fills a unit lower-triangular L, the strictly upper part a unit
 *    upper-triangular U, and the diagonal is log D (D_ii = exp X_ii).
 * M  [B][H][T][n][n] fp32, written: M = c L D U with c = |det(L D U)|^(-1/n),
 *    so det(M) = 1.  Computed as L diag(exp(X_ii - mean_j X_jj)) U, which is
 *    the same matrix because det L = det U = 1.
 * x and M must not overlap.
 */
mru_status mru_build_inputs(const float* x, float* M, int64_t B, int64_t H, int64_t T,
                            int32_t n, void* stream);

/*
 * Orthogonal input state matrices, the variant "Improving Matrix Recurrent
 * Units as an Attention Alternative" (Key Points) describes as orthogonal
 * constraints via the Cayley map or the matrix exponential.  For each token,
 * with X the row-major n-by-n view of x and A = (X - X^T) / 2 its
 * skew-symmetric part (the pages do not say how the entries fill A; this is
 * the reading taken):
 *   method MRU_ORTHO_CAYLEY:  M = (I - A)^{-1} (I + A)
 *   method MRU_ORTHO_EXPM:    M = exp(A)
 * Both are orthogonal with det M = 1, so every prefix product has
 * |P_t|_F = sqrt(n) and a scan of them never leaves the fp32 range.
 * Computed in fp64 and rounded once to fp32 (relative error per matrix below
 * 1e-7).  x, M as for mru_build_inputs; any other method returns
 * MRU_ERR_SHAPE.
 */
mru_status mru_build_orthogonal(const float* x, float* M, int64_t B, int64_t H, int64_t T,
                                int32_t n, int32_t method, void* stream);

/*
 * Gradient through the input construction: dx = d<dM, build(x)>/dx, i.e. the
 * vector-Jacobian product of mru_build_inputs.  Source of the construction:
 * "Improving Matrix Recurrent Units as an Attention Alternative", Key Points;
 * the pages train through it but give no formula (this is the exact gradient,
 * including the scalar's dependence on the diagonal: dx has zero trace).
 *
 * x   [B][H][T][n*n] fp32, read (the forward's raw token vectors).
 * dM  [B][H][T][n][n] fp32, read (e.g. the output of mru_scan_bwd).
 * dx  [B][H][T][n*n] fp32, written.  dx must not overlap x or dM.
 */
mru_status mru_build_inputs_bwd(const float* x, const float* dM, float* dx, int64_t B, int64_t H,
                                int64_t T, int32_t n, void* stream);

/*
 * Chunk length (tokens per scan chunk) of the automatic plan for this shape
 * and direction (MRU_DIR_FWD, MRU_DIR_BWD, or MRU_DIR_FWD_X for the forward
 * from raw token vectors, which at n = 16 plans 24-token chunks where the scan
 * from M takes up to 64, and at n = 32 twice the chunks: it runs three / two
 * waves per SIMD); a pure function of its arguments.  Returns 0 for an invalid
 * shape.
 */
int32_t mru_scan_chunk(int64_t B, int64_t H, int64_t T, int32_t n, int32_t direction);

/*
 * The scan plan for this shape, direction (as for mru_scan_chunk) and chunk
 * (0 = automatic), as
 * out4[0] = chunk length K, out4[1] = chunks per sequence (the token chunks,
 * rounded up with empty chunks to a multiple of the chains a wave runs),
 * out4[2] = chunks per super (the unit of the carry chain), out4[3] = workspace
 * bytes.  A plan with one chunk per sequence needs no workspace.  Returns
 * MRU_OK, MRU_ERR_NULL (out4 NULL), MRU_ERR_SHAPE or MRU_ERR_CHUNK.
 */
int32_t mru_scan_plan(int64_t B, int64_t H, int64_t T, int32_t n, int32_t direction,
                      int32_t chunk, int64_t* out4);

/*
 * Workspace bytes that mru_scan_fwd (direction MRU_DIR_FWD) or mru_scan_bwd
 * (MRU_DIR_BWD) needs for this shape with the automatic plan; the same size
 * serves every entry point of that direction (from M or from raw token
 * vectors, with or without a carried state: the largest of their plans).  May be 0, in which case ws may
 * be NULL.  Returns 0 for an invalid shape as well; callers validate through
 * the scan call itself.
 */
size_t mru_scan_workspace_bytes(int64_t B, int64_t H, int64_t T, int32_t n, int32_t direction);

/* The same for an explicit chunk length (0 = automatic), as taken by the
 * entry points with a chunk argument. */
size_t mru_scan_workspace_bytes_chunked(int64_t B, int64_t H, int64_t T, int32_t n,
                                        int32_t direction, int32_t chunk);

/*
 * Status word of a scan's workspace, copied in stream order to *status (one
 * int32 in device memory, 4-byte aligned): 0 when every look-back wait of the
 * last multi-chunk scan that used ws completed, MRU_WS_STATUS_SPIN_TIMEOUT
 * when one gave up.  Chunks wait only on chunks whose owners are already
 * running, so every wait ends; the bounded poll turns a logic error into this
 * bit instead of a hang, and a scan that sets it has invalid outputs.  Pass
 * the ws and ws_bytes of that scan, enqueued after it on the same stream.  A
 * plan with one chunk per sequence (workspace size 0) never waits: with ws
 * NULL or ws_bytes below 256, *status is set to 0.  A single-chunk scan does
 * not touch the word, so query right after the scan it concerns.  Returns
 * MRU_ERR_NULL (status NULL), MRU_ERR_ALIGN, MRU_ERR_ALIAS (status inside the
 * header) or MRU_ERR_HIP.
 */
mru_status mru_scan_ws_status(const void* ws, size_t ws_bytes, int32_t* status, void* stream);

/*
 * Forward scan: every running product of the input state matrices.
 * Source: "MRU Update: ...", section "What MRU Actually Does" (cumulative
 * multiplication, state matrix times new input matrix; associativity allows a
 * parallel scan).
 *
 * M      [B][H][T][n][n] fp32, read.
 * P      [B][H][T][n][n] fp32, written: P_t = M_1 M_2 ... M_t for every sequence,
 *        inclusive, with P_0 = I (right multiplication, P_t = P_{t-1} M_t).
 *        P viewed as [B][H][T][n*n] is the flattened output vector.
 * ws     device workspace of at least mru_scan_workspace_bytes(B, H, T, n,
 *        MRU_DIR_FWD) bytes (16-byte aligned), or NULL when that size is 0.
 *        Its contents on entry are ignored; on exit it holds scratch state and
 *        the status word (mru_scan_ws_status).
 * stream a hipStream_t.
 * M and P must not overlap; P must not overlap ws.
 */
mru_status mru_scan_fwd(const float* M, float* P, int64_t B, int64_t H, int64_t T, int32_t n,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * mru_scan_fwd with an explicit plan: chunk = tokens per scan chunk, 0 =
 * automatic (mru_scan_chunk).  Any positive value gives the same result up to
 * rounding order; ws as for mru_scan_fwd with
 * mru_scan_workspace_bytes_chunked(..., MRU_DIR_FWD, chunk).  MRU_ERR_CHUNK
 * for chunk < 0.
 */
mru_status mru_scan_fwd_chunked(const float* M, float* P, int64_t B, int64_t H, int64_t T,
                                int32_t n, int32_t chunk, void* ws, size_t ws_bytes,
                                void* stream);

/*
 * Forward scan straight from raw token vectors: mru_build_inputs followed by
 * mru_scan_fwd in one pass that reads x once and writes P once.  No input
 * state matrix is stored.  For n in {4, 8} each step multiplies the running
 * state by the LDU factors in turn (L, then diag(e), then U, same cost as a
 * dense product); for n = 16, 32 each token's matrix is formed on chip, in
 * fp32 as by mru_build_inputs (as the unit lower factor times diag(e) U), and
 * fed to the same fp64 chain as mru_scan_fwd.  Results agree with the two-call
 * path up to rounding order.  Arguments as for mru_scan_fwd_chunked with x
 * ([B][H][T][n*n]) in place of M; x and P must not overlap.  n in {4, 8, 16,
 * 32}.
 */
mru_status mru_scan_fwd_x(const float* x, float* P, int64_t B, int64_t H, int64_t T, int32_t n,
                          int32_t chunk, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward scan: vector-Jacobian product of the forward scan.
 * Given dP = dL/dP_t for every t, writes dM = dL/dM_t, where (chain rule on
 * P_t = P_{t-1} M_t) with Q_T = dP_T and Q_t = dP_t + Q_{t+1} M_{t+1}^T,
 * dM_t = P_{t-1}^T Q_t and P_0 = I.  The pages describe training through the
 * product ("MRU Update: ...", section "The Two Fatal Issues From a Year Ago":
 * unbounded states make gradients blow up) but give no formula; this is the
 * exact gradient.
 *
 * M   [B][H][T][n][n] fp32, read (the forward inputs).
 * P   [B][H][T][n][n] fp32, read (the forward outputs of mru_scan_fwd on M).
 *     Every prefix P_{t-1} is read and used as given.
 * dP  [B][H][T][n][n] fp32, read.
 * dM  [B][H][T][n][n] fp32, written.
 * ws  device workspace of at least mru_scan_workspace_bytes(B, H, T, n,
 *     MRU_DIR_BWD) bytes (16-byte aligned), or NULL when that size is 0.
 * dM must not overlap M, P, dP or ws.
 */
mru_status mru_scan_bwd(const float* M, const float* P, const float* dP, float* dM, int64_t B,
                        int64_t H, int64_t T, int32_t n, void* ws, size_t ws_bytes,
                        void* stream);

/*
 * mru_scan_bwd with an explicit plan (chunk as for mru_scan_fwd_chunked, ws
 * sized by mru_scan_workspace_bytes_chunked(..., MRU_DIR_BWD, chunk)).
 */
mru_status mru_scan_bwd_chunked(const float* M, const float* P, const float* dP, float* dM,
                                int64_t B, int64_t H, int64_t T, int32_t n, int32_t chunk,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Backward scan from raw token vectors: dM as from mru_build_inputs followed
 * by mru_scan_bwd, multiplying by the transposed factors of M_{t+1}
 * (U^T, diag(e), L^T) read from x.  Arguments as for mru_scan_bwd_chunked with
 * x in place of M.  For n in {4, 8} only one prefix in four is read (the one
 * before each block of four tokens, counted from a chunk's end) and the
 * prefixes in between are recomputed from it and x, so P must be the
 * forward's output on this x (mru_scan_fwd_x; equal up to rounding).  For
 * n = 16, 32 every prefix is read, and each M_{t+1} is formed on chip in fp32
 * exactly as mru_build_inputs forms it (the same products and sums), so dM is
 * bit for bit that of mru_build_inputs followed by mru_scan_bwd_chunked.
 * n in {4, 8, 16, 32}.
 */
mru_status mru_scan_bwd_x(const float* x, const float* P, const float* dP, float* dM, int64_t B,
                          int64_t H, int64_t T, int32_t n, int32_t chunk, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Forward scan with a carried-in state and an optional exponent side output:
 * segment continuation, token-by-token streaming and sequences whose products
 * leave the fp32 range.  The running product is the same recurrence, state
 * times new input ("MRU Update: ...", section "What MRU Actually Does"),
 * started from a given state instead of I:
 *   P_t = P_0 M_1 ... M_t,   P_0 = 2^carry_exp[b][h] * carry[b][h]  (t = 1..T).
 *
 * in         M [B][H][T][n][n], or x [B][H][T][n*n] when from_x != 0 (then
 *            any n, as mru_scan_fwd_x).
 * carry      [B][H][n][n] fp32, 16-byte aligned, or NULL for P_0 = I.
 * carry_exp  [B][H] int32, or NULL for exponents 0.
 * P          [B][H][T][n][n] fp32, written.
 * P_exp      NULL: P holds P_t itself (IEEE fp32, +-inf where it overflows).
 *            Otherwise [B][H][T] int32, written, and the scan is scaled:
 *            P_t = 2^P_exp[t] * P[t] with the largest |entry| of P[t] in
 *            [0.5, 1] (exactly 0 only if P_t is 0).  The running state is
 *            rescaled by exact powers of two, so wherever P_t is a normal fp32
 *            matrix, 2^P_exp[t] * P[t] carries the same bits as the unscaled
 *            result, and beyond that range the scan keeps going.
 * The carry out of a segment is its last token's (P, P_exp); passing it as
 * the next segment's (carry, carry_exp) continues the scan.
 * chunk, ws, ws_bytes as for mru_scan_fwd_chunked (the same workspace size).
 * Errors: as mru_scan_fwd; MRU_ERR_ALIGN for a misaligned carry (16 bytes)
 * or exponent array (4 bytes); MRU_ERR_ALIAS if P or P_exp overlaps an input,
 * each other or ws.  B*H*T = 0 writes nothing.
 */
mru_status mru_scan_fwd_ex(const float* in, int32_t from_x, const float* carry,
                           const int32_t* carry_exp, float* P, int32_t* P_exp, int64_t B,
                           int64_t H, int64_t T, int32_t n, int32_t chunk, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Backward of mru_scan_fwd_ex's unscaled form: with L = sum_t <dP_t, P_t> and
 * P_t = P_0 M_1 ... M_t, writes dM = dL/dM_t (dM_1 = P_0^T Q_1) and, when
 * dcarry is not NULL, dL/dP_0 = Q_1 M_1^T, where Q_t is the adjoint of P_t.
 * in, from_x  as for mru_scan_fwd_ex.
 * carry       [B][H][n][n] fp32 (P_0, with any exponent already applied) or
 *             NULL for I.
 * P, dP       [B][H][T][n][n] fp32: the plain forward outputs and dL/dP.
 * dM          [B][H][T][n][n] fp32, written.
 * dcarry      [B][H][n][n] fp32, written, or NULL.  For a segmented
 *             sequence, the next segment's dcarry is added into this
 *             segment's dP at its last token.
 * chunk, ws, ws_bytes as for mru_scan_bwd_chunked.  Errors as mru_scan_bwd, plus
 * MRU_ERR_ALIGN / MRU_ERR_ALIAS for carry and dcarry.  B*H*T = 0 writes
 * nothing (dcarry included).
 */
mru_status mru_scan_bwd_ex(const float* in, int32_t from_x, const float* carry, const float* P,
                           const float* dP, float* dM, float* dcarry, int64_t B, int64_t H,
                           int64_t T, int32_t n, int32_t chunk, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * Gradient of the whole layer with respect to the raw token vectors, in one
 * pass: dx = dL/dx_t for L = sum_t <dP_t, P_t>, P_t = P_0 M_1 ... M_t with M_t
 * built from x_t by mru_build_inputs (LDU fill and determinant-correcting
 * scalar, "Improving Matrix Recurrent Units as an Attention Alternative", Key
 * Points).  The same result as mru_scan_bwd_ex (from_x = 1) followed by
 * mru_build_inputs_bwd on its dM, up to rounding, without writing dM or reading
 * x a second time: per token it reads x, dP and the stored prefixes (n = 4, 8:
 * one in four) and writes dx.  With G = dL/dM_t, H = G U^T and
 * g_k = (L^T G U^T)_kk:
 *   dX_ij = e_j H_ij (i > j),  e_i (L^T G)_ij (i < j),  e_i g_i - mean_k e_k g_k (i = j).
 * For n = 4, 8, (L^T G) is formed from the rows of P_{t-1} L_t, as G from
 * those of P_{t-1}; for n = 16, 32 from G itself on the matrix core.
 *
 * x       [B][H][T][n*n] fp32, read (the forward's inputs).
 * carry   [B][H][n][n] fp32 (P_0) or NULL for I; 16-byte aligned.
 * P, dP   [B][H][T][n][n] fp32, read: the forward's outputs on x (mru_scan_fwd_x
 *         or mru_scan_fwd_ex) and dL/dP.  For n = 4, 8 one prefix in four is
 *         read, as for mru_scan_bwd_x.
 * dx      [B][H][T][n*n] fp32, written.
 * dcarry  [B][H][n][n] fp32, written (dL/dP_0), or NULL.
 * chunk, ws, ws_bytes as for mru_scan_bwd_chunked.  n in {4, 8, 16, 32}.  For
 * n = 16, 32 every prefix is read, and each token's dM_t (rounded to fp32)
 * goes through the same per-token routine as mru_build_inputs_bwd, so dx is
 * bit for bit mru_build_inputs_bwd applied to mru_scan_bwd_ex's dM.  Errors as
 * mru_scan_bwd_ex; dx must not overlap any input, dcarry or ws.  B*H*T = 0
 * writes nothing.
 */
mru_status mru_scan_bwd_dx(const float* x, const float* carry, const float* P, const float* dP,
                           float* dx, float* dcarry, int64_t B, int64_t H, int64_t T, int32_t n,
                           int32_t chunk, void* ws, size_t ws_bytes, void* stream);

/*
 * mru_scan_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, allocation-free serving loops, harnesses that forbid
 * hipMalloc.  The same kernels and results as mru_scan_fwd (bitwise), but the
 * look-back workspace is a static array inside the library, one per device
 * (MRU_NOALLOC_SCRATCH_BYTES, held from the library's load on that device
 * until the process ends), so the call takes no ws argument and allocates
 * nothing.  The caller still passes M and P.
 * Returns MRU_ERR_WORKSPACE, before launching anything, when the automatic
 * plan for this shape needs more than MRU_NOALLOC_SCRATCH_BYTES (at most
 * mru_scan_workspace_bytes(B, H, T, n, MRU_DIR_FWD)); MRU_ERR_HIP if the
 * array's device address cannot be found; otherwise as mru_scan_fwd.
 * Every call on a device shares that device's array, which keeps the last
 * call's contents (each call clears what must start at zero): two calls that
 * may run at the same time on one device, on different streams or from
 * different threads, race and give wrong results; order them on one stream.
 */
#define MRU_NOALLOC_SCRATCH_BYTES (64u << 20)
mru_status mru_scan_fwd_noalloc(const float* M, float* P, int64_t B, int64_t H, int64_t T,
                                int32_t n, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MRU_H */
