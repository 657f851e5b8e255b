// Host-side launch functions of the MRU kernels (internal to libmru.so).
// Shapes are validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mru {

// LDU fill + determinant correction for ntok = B*H*T token matrices.
hipError_t launch_build(const float* x, float* M, int64_t ntok, int n, hipStream_t stream);
// Orthogonal inputs from the skew-symmetric part of each token: method 0 the
// Cayley map, 1 the matrix exponential.
hipError_t launch_build_orth(const float* x, float* M, int64_t ntok, int n, int method,
                             hipStream_t stream);
// Its gradient: dx from x and dL/dM.
hipError_t launch_build_bwd(const float* x, const float* dM, float* dx, int64_t ntok, int n,
                            hipStream_t stream);

// Optional carried state of a scan (all pointers may be null).
//   carry      [S][n][n]  state before each sequence's first token (null: I)
//   carry_exp  [S]        power-of-two exponent of carry (null: 0)
//   out_exp    [S][T]     forward: write P_t as 2^out_exp * P~_t with P~_t
//                         normalised (scaled scan); null: plain P_t
//   dcarry     [S][n][n]  backward: gradient with respect to carry
struct ScanCarry {
    const float* carry = nullptr;
    const int32_t* carry_exp = nullptr;
    int32_t* out_exp = nullptr;
    float* dcarry = nullptr;
};

// Chunked scans over S sequences of T tokens: chunk length K, nch chunks per
// sequence (possibly padded with empty chunks), supers of Z chunks.  nch == 1
// runs without workspace; nch > 1 needs a cleared workspace header and flags.
// from_x: the first array holds raw token vectors and the kernel builds the
// input matrices on the fly (never writing them); n = 4, 8, 16, 32.  to_dx
// (backward, with
// from_x): the output is dL/dx, the gradient through the build, instead of dL/dM.
hipError_t launch_fwd_valu(const float* M, float* P, int64_t S, int64_t T, int n, int64_t K,
                           int64_t nch, int64_t Z, void* ws, hipStream_t stream, bool from_x,
                           const ScanCarry& cy);
hipError_t launch_bwd_valu(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                           int64_t T, int n, int64_t K, int64_t nch, int64_t Z, void* ws,
                           hipStream_t stream, bool from_x, bool to_dx, const ScanCarry& cy);
hipError_t launch_fwd_mfma(const float* M, float* P, int64_t S, int64_t T, int n, int64_t K,
                           int64_t nch, int64_t Z, void* ws, hipStream_t stream, bool from_x,
                           const ScanCarry& cy);
hipError_t launch_bwd_mfma(const float* M, const float* P, const float* dP, float* dM, int64_t S,
                           int64_t T, int n, int64_t K, int64_t nch, int64_t Z, void* ws,
                           hipStream_t stream, bool from_x, bool to_dx, const ScanCarry& cy);

// Tokens per chunk the matrix-core forward kernel keeps in registers between
// its two passes (0 = none): chunks of at most this length read M once.
int mfma_retain_tokens(int n, bool from_x);

// Chains per wave of the vector-ALU kernels (n = 4, 8) for direction dir.
int valu_chains_per_wave(int n, int dir);

}  // namespace mru
