// gemm.h -- host-side description of one GEMM with a fused epilogue.
//   C[m][n] = sum_k A(m,k) * B(n,k),  0 <= m < M, 0 <= n < N, 0 <= k < K
//   A(m,k) = a_kmajor ? A[m*lda + k] : A[k*lda + m]
//   B(n,k) = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
// Forward projections (Y = X W^T) are (A k-major, B k-major); input
// gradients (dX = dY W) are (A k-major, B n-major); weight gradients
// (dW = dY^T X) are (A m-major, B n-major).
#pragma once
#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime.h>
#include "tel_common.h"
#include "fastdiv.h"

namespace tel {

enum EpiKind {
    EPI_STORE = 0,         // out = v                               (T, or f32 if out_f32)
    EPI_QKV = 1,           // v + bias, scattered to [3][B][N][S][d]
    EPI_BIAS_DROP_RES = 2, // out = res + drop(v + bias)            (res T|f32, out T|f32)
    EPI_BIAS_GELU = 3,     // u = v + bias -> out (or GELU'(u) if gelu_grad_out); GELU(u) -> out2 (if non-null)
    EPI_GELU_BWD = 4,      // out = v * round_T(GELU'(aux)); out2 (optional) = GELU(aux)
    EPI_HEADSPLIT = 5,     // v scattered to [B][N][S][d]
    EPI_ADD_RES = 6,       // out = v + res(f32)
    EPI_MUL_AUX = 7,       // out = v * aux                         (aux T)
    EPI_ATOMIC_ADD = 8,    // out += v with packed dtype atomics (k-splits of a relaxed-determinism launch)
};

struct EpiArgs {
    void* out = nullptr;
    int ldo = 0;
    int out_f32 = 0;
    const void* bias = nullptr;
    const void* res = nullptr;
    int res_f32 = 0;
    void* out2 = nullptr;
    int gelu_grad_out = 0;  // EPI_BIAS_GELU: out receives GELU'(u) instead of u
    const void* aux = nullptr;
    int B = 0, S = 0, H = 0, NH = 0, d = 0;  // head-split geometry
    FastDiv fS, fH, fd;                       // dividers by S, H and d (set by the launch)
    Drop drop{};                              // thr == 0: no dropout
    // Packed rows: row m of the GEMM holds token row_map[m] (b*S + s) of the
    // padded batch, or no token (-1, a filler row).  The head-split scatters
    // place a row at its token (filler rows are not stored) and the dropout
    // element index uses the token, so masks match the padded layout.
    const int32_t* row_map = nullptr;
};

struct GemmDesc {
    int dtype = 0;  // tel_dtype
    int M = 0, N = 0, K = 0;
    const void* A = nullptr;
    int lda = 0;
    bool a_kmajor = true;
    const void* B = nullptr;
    int ldb = 0;
    bool b_kmajor = true;
    int epi = EPI_STORE;
    EpiArgs ea;
    float* splitk_ws = nullptr;  // fp32 [splits][M][N] partials (+ [splits][M] row sums)
    size_t splitk_ws_elems = 0;
    // Grouped weight gradients only: the k-splits add their partials (and row
    // sums) into the zeroed outputs with packed dtype atomics -- no workspace,
    // no reduction launch, but a summation order that follows arrival.
    bool splitk_atomic = false;
    // Optional row sums of A over k (sum_k A(m,k), dtype, M values): for a
    // weight gradient dW = dY^T X these are the bias gradients sum_t dY[t][m].
    // Only computed when gemm_rowsum_fused() is true; the caller sums
    // otherwise.
    void* rowsum_out = nullptr;
};

// True if gemm_launch computes rowsum_out for this GEMM inside its kernel.
bool gemm_rowsum_fused(const GemmDesc& g);

// Two weight gradients (A and B m/n-major, EPI_STORE, M
// and N multiples of 256) in one persistent launch, so that the tiles of
// both fill the chip with fewer k-splits than either alone; a's workspace
// (splitk_ws, splitk_ws_elems) holds the partials of both.  Row sums are
// fused as in gemm_launch.  gemm_group_ok tells whether the pair qualifies;
// gemm_launch_group returns hipErrorInvalidValue (launching nothing) if not.
//
// Column sums that only need to be done by the end of the launch (the
// LayerNorm gamma/beta gradients: out[n] = sum_p part[p][n] of fp32 [P][N]
// partial rows, out in the GEMM dtype) can ride along: they run as extra
// workgroups of the launch that reduces the split-K partials (or of a launch
// of their own when the pair needs no reduction), summed in the same fixed
// order as the standalone LayerNorm finalize, so the results are the same
// bits either way.
struct ColsumJob {
    const float* part;
    int P, N;
    void* out;
};
constexpr int kMaxColsumJobs = 4;
// Optional timing events (any may be null), recorded on the stream right
// around the grouped GEMM kernel and around the launch after it (the split-K
// reduction with the column sums; back to back when there is none).
struct GroupEvents {
    hipEvent_t gemm_start = nullptr, gemm_stop = nullptr;
    hipEvent_t red_start = nullptr, red_stop = nullptr;
};
bool gemm_group_ok(const GemmDesc& a, const GemmDesc& b);
hipError_t gemm_launch_group(const GemmDesc& a, const GemmDesc& b, hipStream_t stream,
                             const ColsumJob* colsums = nullptr, int n_colsums = 0,
                             const GroupEvents* events = nullptr);
// Workspace elements gemm_launch_group needs for the pair (0: none).
size_t gemm_splitk_group_elems(const GemmDesc& a, const GemmDesc& b);

// Launch; returns hipSuccess or the launch error.  force_simt selects the
// generic SIMT kernel regardless of shape (used by tests).
hipError_t gemm_launch(const GemmDesc& g, hipStream_t stream, bool force_simt = false);

// Elements of split-K workspace the dispatcher will use for this GEMM (0 if none).
size_t gemm_splitk_elems(const GemmDesc& g);

}  // namespace tel
