// C ABI of libmru.so: argument validation, scan planning, launches.
// The contract of every entry point is documented in include/mru.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "mru.h"
#include "mru_device.h"
#include "mru_kernels.h"

namespace mru {

__global__ void ws_reset_kernel(uint32_t* words, int64_t nwords) {
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < nwords;
         i += int64_t(gridDim.x) * blockDim.x)
        words[i] = 0u;
}

// Copies the status word of a workspace header to *out (0 without a header).
__global__ void ws_status_kernel(const WsHeader* hdr, int32_t* out) {
    if (threadIdx.x == 0) *out = hdr ? int32_t(ws_load(&hdr->status)) : 0;
}

namespace {

constexpr int64_t kMaxT = int64_t(1) << 30;

bool valid_n(int32_t n) { return n == 4 || n == 8 || n == 16 || n == 32; }

int acc_bytes(int n) { return n >= 16 ? 8 : 4; }

int chains_per_wave(int n, int dir) { return n <= 8 ? valu_chains_per_wave(n, dir) : 1; }

// Shape check shared by every entry point; fills S and the element count.
bool shape_ok(int64_t B, int64_t H, int64_t T, int32_t n, int64_t* S, int64_t* elems) {
    if (!valid_n(n) || B < 0 || H < 0 || T < 0 || T > kMaxT) return false;
    const int64_t lim = INT64_MAX / 64;
    if (B > 0 && H > lim / B) return false;
    const int64_t s = B * H;
    if (s > 0 && T > lim / s) return false;
    const int64_t st = s * T;
    if (st > lim / (int64_t(n) * n)) return false;
    *S = s;
    *elems = st * n * n;
    return true;
}

struct Plan {
    int64_t K = 0;        // tokens per chunk
    int64_t nch = 0;      // chunks per sequence (incl. padding)
    int64_t Z = 1;        // chunks per super
    int64_t nchunks = 0;  // S * nch
    size_t ws = 0;        // workspace bytes
    size_t reset_words = 0;
    bool multi = false;
};

// Chunk length used when the caller passes chunk = 0.  Single-chunk scans need
// no carries at all (one product per token); they are chosen when the
// sequences alone give the GPU enough independent chains.
int64_t auto_chunk_len(int64_t S, int64_t T, int n, int dir, bool from_x = false) {
    if (T <= 0) return 0;
    int64_t target;
    if (n <= 8) {
        const int64_t lanes_per_chain = 64 / chains_per_wave(n, dir);
        if (S * lanes_per_chain >= 32768) return T;  // >= 512 waves
        target = 16384;                              // 1024 waves of chains
    } else {
        // one wave per chain, one wave per SIMD (1024 SIMDs on MI355X).  Chains
        // wanted (measured, C3-C5 shapes): n = 32 runs best with one round of
        // waves (its chunks are long enough to hide the look-back; the forward
        // from raw token vectors runs two waves per SIMD, so two chains per
        // SIMD), the n = 16 backward with four, the n = 16 forward with two
        // (then capped by the register buffer below).
        target = n == 32 ? (from_x && dir == MRU_DIR_FWD ? 2048 : 1024) : (dir == 1 ? 4096 : 2048);
        if (S >= target) return T;
    }
    const int64_t nch = (target + S - 1) / S;
    int64_t K = (T + nch - 1) / nch;
    // shortest chunk (measured on the C1 / C2 shapes): the vector-ALU backward does
    // about twice the forward's work per token, so its chains gain from 8-token
    // chunks where the forward's look-back would cost more than it saves
    const int64_t kmin = (n <= 8 && dir == 1) ? 8 : 16;
    if (K < kmin) K = kmin;
    // a forward chunk that fits the register buffer reads its inputs once
    const int64_t keep = dir == 0 ? mfma_retain_tokens(n, from_x) : 0;
    if (keep > 0 && K > keep) K = keep;
    return K < T ? K : T;
}

Plan make_plan(int64_t S, int64_t T, int n, int dir, int64_t chunk, bool from_x = false) {
    Plan p;
    if (S <= 0 || T <= 0) return p;
    p.K = chunk > 0 ? (chunk < T ? chunk : T) : auto_chunk_len(S, T, n, dir, from_x);
    p.nch = (T + p.K - 1) / p.K;
    if (p.nch <= 1) {
        p.nch = 1;
        p.nchunks = S;
        return p;
    }
    p.multi = true;
    const int G = chains_per_wave(n, dir);
    if (G > 1) {
        p.nch = (p.nch + G - 1) / G * G;  // a wave never spans two sequences
        int64_t z = llround(sqrt(double(p.nch / G)));
        z = z < 1 ? 1 : (z > 4 ? 4 : z);
        p.Z = G * z;                      // a wave never spans two supers
    } else {
        // supers of about sqrt(chunks) chunks balance the walk over a super's
        // aggregates against the chain of super prefixes; at n = 16 half that
        // measured faster (C5 backward 323-329 -> 313-317 us, C3 forward from raw
        // token vectors 466-469 -> 451-453 us), a quarter (at least 5) for the
        // forward from M, whose retained chunks leave the look-back on the
        // critical path (with its staggered start, interleaved runs on one box:
        // C3 Z = 2, 3, 4, 5, 6 -> 259, 247-248, 249-250, 247-248, 249-252 us, C5
        // 148, 136, 136-137, 133, 136 us), at n = 32 neither
        const bool fwd16 = n == 16 && dir == 0 && !from_x;
        const double zf = n == 16 ? (fwd16 ? 0.25 : 0.5) : 1.0;
        int64_t z = llround(zf * sqrt(double(p.nch)));
        if (fwd16 && z < 5) z = 5;
        p.Z = z < 1 ? 1 : (z > 64 ? 64 : z);
    }
    p.nchunks = S * p.nch;
    const WsLayout L = ws_layout(p.nchunks, n, acc_bytes(n), dir == MRU_DIR_FWD ? 2 : 3);
    p.ws = L.total;
    p.reset_words = (L.flags_off + size_t(p.nchunks) * 4 + 3) / 4;
    return p;
}

// Blocks of 64 lanes the scan kernel launches; the dispatch grid must stay
// below 2^32 work-items.
bool grid_ok(const Plan& p, int n, int dir) {
    const int64_t G = chains_per_wave(n, dir);
    const int64_t blocks = (p.nchunks + G - 1) / G;
    return blocks * 64 <= int64_t(UINT32_MAX);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

mru_status launched(hipError_t e) { return e == hipSuccess ? MRU_OK : MRU_ERR_HIP; }

mru_status reset_ws(void* ws, const Plan& p, hipStream_t stream) {
    const int64_t words = int64_t(p.reset_words);
    int64_t blocks = (words + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(ws_reset_kernel, dim3(unsigned(blocks)), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ws), words);
    return launched(hipGetLastError());
}

}  // namespace
}  // namespace mru

using namespace mru;

extern "C" {

int32_t mru_abi_version(void) { return MRU_ABI_VERSION; }

const char* mru_status_string(int32_t status) {
    switch (status) {
        case MRU_OK: return "MRU_OK";
        case MRU_ERR_NULL: return "MRU_ERR_NULL: a required pointer is NULL";
        case MRU_ERR_SHAPE: return "MRU_ERR_SHAPE: bad B/H/T, n not in {4,8,16,32}, or an unsupported option";
        case MRU_ERR_ALIGN: return "MRU_ERR_ALIGN: a pointer is misaligned (16 bytes; exponent arrays 4)";
        case MRU_ERR_ALIAS: return "MRU_ERR_ALIAS: an output overlaps an input";
        case MRU_ERR_WORKSPACE: return "MRU_ERR_WORKSPACE: workspace missing or too small";
        case MRU_ERR_CHUNK: return "MRU_ERR_CHUNK: chunk must be >= 0";
        case MRU_ERR_HIP: return "MRU_ERR_HIP: the HIP runtime reported a launch error";
        case MRU_ERR_TIMEOUT: return "MRU_ERR_TIMEOUT: a look-back wait of a scan timed out; its outputs are invalid";
        default: return "unknown mru_status";
    }
}

mru_status mru_build_inputs(const float* x, float* M, int64_t B, int64_t H, int64_t T, int32_t n,
                            void* stream) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (elems == 0) return MRU_OK;
    if (!x || !M) return MRU_ERR_NULL;
    if (!aligned16(x) || !aligned16(M)) return MRU_ERR_ALIGN;
    const size_t bytes = size_t(elems) * sizeof(float);
    if (overlap(x, bytes, M, bytes)) return MRU_ERR_ALIAS;
    (void)hipGetLastError();
    return launched(launch_build(x, M, S * T, n, static_cast<hipStream_t>(stream)));
}

mru_status mru_build_orthogonal(const float* x, float* M, int64_t B, int64_t H, int64_t T,
                                int32_t n, int32_t method, void* stream) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (method != MRU_ORTHO_CAYLEY && method != MRU_ORTHO_EXPM) return MRU_ERR_SHAPE;
    if (elems == 0) return MRU_OK;
    if (!x || !M) return MRU_ERR_NULL;
    if (!aligned16(x) || !aligned16(M)) return MRU_ERR_ALIGN;
    const size_t bytes = size_t(elems) * sizeof(float);
    if (overlap(x, bytes, M, bytes)) return MRU_ERR_ALIAS;
    (void)hipGetLastError();
    return launched(launch_build_orth(x, M, S * T, n, method, static_cast<hipStream_t>(stream)));
}

mru_status mru_build_inputs_bwd(const float* x, const float* dM, float* dx, int64_t B, int64_t H,
                                int64_t T, int32_t n, void* stream) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (elems == 0) return MRU_OK;
    if (!x || !dM || !dx) return MRU_ERR_NULL;
    if (!aligned16(x) || !aligned16(dM) || !aligned16(dx)) return MRU_ERR_ALIGN;
    const size_t bytes = size_t(elems) * sizeof(float);
    if (overlap(dx, bytes, x, bytes) || overlap(dx, bytes, dM, bytes)) return MRU_ERR_ALIAS;
    (void)hipGetLastError();
    return launched(launch_build_bwd(x, dM, dx, S * T, n, static_cast<hipStream_t>(stream)));
}

int32_t mru_scan_chunk(int64_t B, int64_t H, int64_t T, int32_t n, int32_t direction) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems) || elems == 0) return 0;
    return int32_t(auto_chunk_len(S, T, n, direction == MRU_DIR_BWD ? 1 : 0, direction == MRU_DIR_FWD_X));
}

size_t mru_scan_workspace_bytes_chunked(int64_t B, int64_t H, int64_t T, int32_t n,
                                        int32_t direction, int32_t chunk) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems) || elems == 0 || chunk < 0) return 0;
    const int dir = direction == MRU_DIR_BWD ? 1 : 0;
    if (direction == MRU_DIR_FWD_X) return make_plan(S, T, n, 0, chunk, true).ws;
    // one workspace serves the scan from M and from raw token vectors, whose
    // automatic plans may differ
    const size_t a = make_plan(S, T, n, dir, chunk).ws, b = make_plan(S, T, n, dir, chunk, true).ws;
    return a > b ? a : b;
}

size_t mru_scan_workspace_bytes(int64_t B, int64_t H, int64_t T, int32_t n, int32_t direction) {
    return mru_scan_workspace_bytes_chunked(B, H, T, n, direction, 0);
}

mru_status mru_scan_ws_status(const void* ws, size_t ws_bytes, int32_t* status, void* stream) {
    if (!status) return MRU_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(status) & 3u) != 0) return MRU_ERR_ALIGN;
    const bool has_header = ws && ws_bytes >= sizeof(WsHeader);
    if (has_header && !aligned16(ws)) return MRU_ERR_ALIGN;
    if (has_header && overlap(ws, sizeof(WsHeader), status, 4)) return MRU_ERR_ALIAS;
    (void)hipGetLastError();
    hipLaunchKernelGGL(ws_status_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       has_header ? static_cast<const WsHeader*>(ws) : nullptr, status);
    return launched(hipGetLastError());
}

int32_t mru_scan_plan(int64_t B, int64_t H, int64_t T, int32_t n, int32_t direction,
                      int32_t chunk, int64_t* out4) {
    int64_t S, elems;
    if (!out4) return MRU_ERR_NULL;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (chunk < 0) return MRU_ERR_CHUNK;
    const Plan p = make_plan(S, T, n, direction == MRU_DIR_BWD ? 1 : 0, chunk, direction == MRU_DIR_FWD_X);
    out4[0] = p.K;
    out4[1] = p.nch;
    out4[2] = p.Z;
    out4[3] = int64_t(p.ws);
    return MRU_OK;
}

}  // extern "C"

namespace {

bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

mru_status scan_fwd_impl(const float* M, float* P, int64_t B, int64_t H, int64_t T, int32_t n,
                         int32_t chunk, void* ws, size_t ws_bytes, void* stream, bool from_x,
                         const ScanCarry& cy) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (chunk < 0) return MRU_ERR_CHUNK;
    if (elems == 0) return MRU_OK;
    if (!M || !P) return MRU_ERR_NULL;
    if (!aligned16(M) || !aligned16(P)) return MRU_ERR_ALIGN;
    if ((cy.carry && !aligned16(cy.carry)) || (cy.carry_exp && !aligned4(cy.carry_exp)) ||
        (cy.out_exp && !aligned4(cy.out_exp)))
        return MRU_ERR_ALIGN;
    const Plan p = make_plan(S, T, n, 0, chunk, from_x);
    if (!grid_ok(p, n, 0)) return MRU_ERR_SHAPE;
    const size_t bytes = size_t(elems) * sizeof(float);
    const size_t cbytes = size_t(S) * n * n * sizeof(float);
    const size_t ebytes = size_t(S) * T * sizeof(int32_t);
    if (overlap(M, bytes, P, bytes) || overlap(cy.carry, cbytes, P, bytes) ||
        overlap(cy.carry_exp, size_t(S) * 4, P, bytes))
        return MRU_ERR_ALIAS;
    if (cy.out_exp && (overlap(cy.out_exp, ebytes, P, bytes) || overlap(cy.out_exp, ebytes, M, bytes) ||
                       overlap(cy.out_exp, ebytes, cy.carry, cbytes) ||
                       overlap(cy.out_exp, ebytes, cy.carry_exp, size_t(S) * 4)))
        return MRU_ERR_ALIAS;
    if (p.ws > 0) {
        if (!ws) return MRU_ERR_WORKSPACE;
        if (!aligned16(ws)) return MRU_ERR_ALIGN;
        if (ws_bytes < p.ws) return MRU_ERR_WORKSPACE;
        if (overlap(ws, p.ws, P, bytes) || overlap(ws, p.ws, M, bytes) ||
            overlap(ws, p.ws, cy.carry, cbytes) || overlap(ws, p.ws, cy.carry_exp, size_t(S) * 4) ||
            overlap(ws, p.ws, cy.out_exp, ebytes))
            return MRU_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (p.multi) {
        const mru_status st = reset_ws(ws, p, s);
        if (st != MRU_OK) return st;
    }
    if (n <= 8) return launched(launch_fwd_valu(M, P, S, T, n, p.K, p.nch, p.Z, ws, s, from_x, cy));
    return launched(launch_fwd_mfma(M, P, S, T, n, p.K, p.nch, p.Z, ws, s, from_x, cy));
}

mru_status scan_bwd_impl(const float* M, const float* P, const float* dP, float* dM, int64_t B,
                         int64_t H, int64_t T, int32_t n, int32_t chunk, void* ws,
                         size_t ws_bytes, void* stream, bool from_x, const ScanCarry& cy,
                         bool to_dx = false) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (chunk < 0) return MRU_ERR_CHUNK;
    if (elems == 0) return MRU_OK;
    if (!M || !P || !dP || !dM) return MRU_ERR_NULL;
    if (!aligned16(M) || !aligned16(P) || !aligned16(dP) || !aligned16(dM)) return MRU_ERR_ALIGN;
    if ((cy.carry && !aligned16(cy.carry)) || (cy.dcarry && !aligned16(cy.dcarry)))
        return MRU_ERR_ALIGN;
    const Plan p = make_plan(S, T, n, 1, chunk);
    if (!grid_ok(p, n, 1)) return MRU_ERR_SHAPE;
    const size_t bytes = size_t(elems) * sizeof(float);
    const size_t cbytes = size_t(S) * n * n * sizeof(float);
    if (overlap(dM, bytes, M, bytes) || overlap(dM, bytes, P, bytes) ||
        overlap(dM, bytes, dP, bytes) || overlap(dM, bytes, cy.carry, cbytes))
        return MRU_ERR_ALIAS;
    if (cy.dcarry && (overlap(cy.dcarry, cbytes, M, bytes) || overlap(cy.dcarry, cbytes, P, bytes) ||
                      overlap(cy.dcarry, cbytes, dP, bytes) || overlap(cy.dcarry, cbytes, dM, bytes) ||
                      overlap(cy.dcarry, cbytes, cy.carry, cbytes)))
        return MRU_ERR_ALIAS;
    if (p.ws > 0) {
        if (!ws) return MRU_ERR_WORKSPACE;
        if (!aligned16(ws)) return MRU_ERR_ALIGN;
        if (ws_bytes < p.ws) return MRU_ERR_WORKSPACE;
        if (overlap(ws, p.ws, dM, bytes) || overlap(ws, p.ws, M, bytes) ||
            overlap(ws, p.ws, P, bytes) || overlap(ws, p.ws, dP, bytes) ||
            overlap(ws, p.ws, cy.carry, cbytes) || overlap(ws, p.ws, cy.dcarry, cbytes))
            return MRU_ERR_ALIAS;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (p.multi) {
        const mru_status st = reset_ws(ws, p, s);
        if (st != MRU_OK) return st;
    }
    if (n <= 8)
        return launched(
            launch_bwd_valu(M, P, dP, dM, S, T, n, p.K, p.nch, p.Z, ws, s, from_x, to_dx, cy));
    return launched(launch_bwd_mfma(M, P, dP, dM, S, T, n, p.K, p.nch, p.Z, ws, s, from_x, to_dx, cy));
}

}  // namespace

extern "C" {

mru_status mru_scan_fwd(const float* M, float* P, int64_t B, int64_t H, int64_t T, int32_t n,
                        void* ws, size_t ws_bytes, void* stream) {
    return scan_fwd_impl(M, P, B, H, T, n, 0, ws, ws_bytes, stream, false, ScanCarry{});
}

mru_status mru_scan_fwd_chunked(const float* M, float* P, int64_t B, int64_t H, int64_t T,
                                int32_t n, int32_t chunk, void* ws, size_t ws_bytes,
                                void* stream) {
    return scan_fwd_impl(M, P, B, H, T, n, chunk, ws, ws_bytes, stream, false, ScanCarry{});
}

mru_status mru_scan_fwd_x(const float* x, float* P, int64_t B, int64_t H, int64_t T, int32_t n,
                          int32_t chunk, void* ws, size_t ws_bytes, void* stream) {
    return scan_fwd_impl(x, P, B, H, T, n, chunk, ws, ws_bytes, stream, true, ScanCarry{});
}

mru_status mru_scan_bwd(const float* M, const float* P, const float* dP, float* dM, int64_t B,
                        int64_t H, int64_t T, int32_t n, void* ws, size_t ws_bytes,
                        void* stream) {
    return scan_bwd_impl(M, P, dP, dM, B, H, T, n, 0, ws, ws_bytes, stream, false, ScanCarry{});
}

mru_status mru_scan_bwd_chunked(const float* M, const float* P, const float* dP, float* dM,
                                int64_t B, int64_t H, int64_t T, int32_t n, int32_t chunk,
                                void* ws, size_t ws_bytes, void* stream) {
    return scan_bwd_impl(M, P, dP, dM, B, H, T, n, chunk, ws, ws_bytes, stream, false, ScanCarry{});
}

mru_status mru_scan_bwd_x(const float* x, const float* P, const float* dP, float* dM, int64_t B,
                          int64_t H, int64_t T, int32_t n, int32_t chunk, void* ws,
                          size_t ws_bytes, void* stream) {
    return scan_bwd_impl(x, P, dP, dM, B, H, T, n, chunk, ws, ws_bytes, stream, true, ScanCarry{});
}

mru_status mru_scan_fwd_ex(const float* in, int32_t from_x, const float* carry,
                           const int32_t* carry_exp, float* P, int32_t* P_exp, int64_t B,
                           int64_t H, int64_t T, int32_t n, int32_t chunk, void* ws,
                           size_t ws_bytes, void* stream) {
    ScanCarry cy;
    cy.carry = carry;
    cy.carry_exp = carry_exp;
    cy.out_exp = P_exp;
    return scan_fwd_impl(in, P, B, H, T, n, chunk, ws, ws_bytes, stream, from_x != 0, cy);
}

mru_status mru_scan_bwd_ex(const float* in, int32_t from_x, const float* carry, const float* P,
                           const float* dP, float* dM, float* dcarry, int64_t B, int64_t H,
                           int64_t T, int32_t n, int32_t chunk, void* ws, size_t ws_bytes,
                           void* stream) {
    ScanCarry cy;
    cy.carry = carry;
    cy.dcarry = dcarry;
    return scan_bwd_impl(in, P, dP, dM, B, H, T, n, chunk, ws, ws_bytes, stream, from_x != 0, cy);
}

mru_status mru_scan_bwd_dx(const float* x, const float* carry, const float* P, const float* dP,
                           float* dx, float* dcarry, int64_t B, int64_t H, int64_t T, int32_t n,
                           int32_t chunk, void* ws, size_t ws_bytes, void* stream) {
    ScanCarry cy;
    cy.carry = carry;
    cy.dcarry = dcarry;
    return scan_bwd_impl(x, P, dP, dx, B, H, T, n, chunk, ws, ws_bytes, stream, true, cy, true);
}

}  // extern "C"

// ----------------------------------------------------------------------------
// Allocation-free forward scan (mru_scan_fwd_noalloc).  Its look-back
// workspace is this file-scope array: one copy per device, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device copy, so its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever
// passed to kernels.
namespace {

constexpr size_t kScratchBytes = size_t(MRU_NOALLOC_SCRATCH_BYTES);
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on device dev (looked up on first use).
hipError_t scratch_address(int dev, void** out) {
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return e;
        if (g != hipSuccess) return g;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" mru_status mru_scan_fwd_noalloc(const float* M, float* P, int64_t B, int64_t H,
                                           int64_t T, int32_t n, void* stream) {
    int64_t S, elems;
    if (!shape_ok(B, H, T, n, &S, &elems)) return MRU_ERR_SHAPE;
    if (elems == 0) return MRU_OK;
    const size_t need = make_plan(S, T, n, 0, 0).ws;
    if (need > kScratchBytes) return MRU_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        // validate first, so that a rejected call has no side effects at all
        if (!M || !P) return MRU_ERR_NULL;
        hipStream_t s = static_cast<hipStream_t>(stream);
        int dev = 0;
        hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
        if (e != hipSuccess || scratch_address(dev, &ws) != hipSuccess) return MRU_ERR_HIP;
    }
    return scan_fwd_impl(M, P, B, H, T, n, 0, ws, kScratchBytes, stream, false, ScanCarry{});
}
