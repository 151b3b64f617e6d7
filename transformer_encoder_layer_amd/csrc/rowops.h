// rowops.h -- LayerNorm forward/backward, dropout application, column
// reductions (bias / gamma / beta gradients) and the mask test hook.
#pragma once
#include <hip/hip_runtime.h>
#include "tel_common.h"

namespace tel {

enum { K_F32 = 0, K_LOWP = 1 };  // element kind of an optional tensor: fp32, or the layer dtype

struct LnFwdArgs {
    int dtype;
    int T, H;
    float eps;
    const void* x; int x_f32;       // input rows
    const void* gamma; const void* beta;
    void* out;                      // dtype
    float* out_f32;                 // optional fp32 copy of the output
    void* out_copy;                 // optional second dtype copy of the output
    float* mu; float* rstd;         // [T]
};

struct LnBwdArgs {
    int dtype;
    int T, H;
    const void* dout;               // dtype: gradient w.r.t. the LN output
    const float* dout_add;          // optional fp32 term added to dout
    const void* src; int src_f32;   // LN input (from_output = 0) or LN output (1)
    int from_output;
    const float* mu; const float* rstd;
    const void* gamma; const void* beta;
    const void* res; int res_f32;   // optional term added to the input gradient
    void* out; int out_f32;         // input gradient
    void* drop_out;                 // optional dtype copy of drop(out) (site given by drop)
    Drop drop;
    const int32_t* row_map;         // optional: token of each row (packed rows) for the dropout index
    float* part_g; float* part_b;   // [gridDim.x][H] partial sums of dgamma, dbeta
};

hipError_t ln_forward(const LnFwdArgs& a, hipStream_t st);
// Returns the number of partial rows written to part_g / part_b.
int ln_backward_parts(int T);
hipError_t ln_backward(const LnBwdArgs& a, hipStream_t st);

// out[n] = sum_p part[p][n] (fixed order), stored as dtype.
hipError_t colsum_finalize(int dtype, const float* part, int P, int N, void* out, hipStream_t st);
// The same for two vectors in one launch: out0 from part0, out1 from part1.
hipError_t colsum_finalize2(int dtype, const float* part0, const float* part1, int P, int N, void* out0, void* out1,
                            hipStream_t st);
// Column sums of a dtype matrix [rows][N] -> fp32 partials [P][N]; returns P.
int colsum_parts(int rows);
hipError_t colsum_partial(int dtype, const void* in, int rows, int N, float* part, hipStream_t st);

// out = drop(in) elementwise over n elements (index = element id), dtype.
// With row_map (packed rows of width H, H % 8 == 0) the element id of row r,
// column c is row_map[r] * H + c (filler rows, row_map < 0, use token 0).
hipError_t dropout_apply(int dtype, const void* in, void* out, size_t n, const Drop& d, hipStream_t st,
                         const int32_t* row_map = nullptr, int H = 0);

// ---- token packing (rows of sequences shorter than S dropped)
// Packed row p of a batch with lengths len[B] holds token
// t = b*S + s (s < len[b]) in order of t; rows sum(len) .. P-1 are fillers.
// map[p] = t or -1 (filler); inv[t] = p or -1 (padding token).
hipError_t build_row_maps(const int32_t* len, int B, int S, int P, int32_t* map, int32_t* inv, hipStream_t st);
// dst[p] = src[map[p]] (zero for fillers), rows of H elements of dtype.
hipError_t gather_rows(int dtype, const void* src, void* dst, const int32_t* map, int P, int H, hipStream_t st);
// dst[t] = src[inv[t]] (zero for padding tokens), T = B*S rows of H elements.
hipError_t scatter_rows(int dtype, const void* src, void* dst, const int32_t* inv, int T, int H, hipStream_t st);
// Zero the rows s >= len[b] of a head-split tensor [G][B][NH][S][d] (dtype).
hipError_t zero_padded_heads(int dtype, void* buf, int G, int B, int NH, int S, int d, const int32_t* len,
                             hipStream_t st);
// Zero rows r0 .. r1-1 of a [rows][W] dtype matrix.
hipError_t zero_rows(int dtype, void* buf, int r0, int r1, int W, hipStream_t st);
// keep bits of n elements (n % 4 == 0) of one site, as uint8.
hipError_t dropout_mask_dump(const Drop& d, uint8_t* out, size_t n, hipStream_t st);

}  // namespace tel
