// rowops.hip -- LayerNorm forward/backward and small HBM-bound kernels.
//
// LayerNorm (DeepSpeed Transformer Kernel guide, "Step 2" epsilon; AI-infra
// blog 2.x: statistics in fp32): one 64-wide wave per row, each lane holding
// up to 16 groups of 4 consecutive elements in registers; mean and variance
// (biased, two-pass over the registers) reduce with wave shuffles.  The
// backward is the standard one, with the normalised value taken either from
// the LN input and saved statistics or -- the invertible mode of the guide's
// "Step 3" -- from the LN output as (y - beta) / gamma.  Residual-gradient
// adds and the next dropout are fused in.  dgamma/dbeta are reduced
// deterministically: per-block partial rows, then a fixed-order column sum.
#include "rowops.h"

namespace tel {


template <typename T>
__device__ __forceinline__ void load4(const void* p, int is_f32, size_t off, float v[4]) {
    if (is_f32) Vec4<float>::load((const float*)p + off, v);
    else Vec4<T>::load((const T*)p + off, v);
}
template <typename T>
__device__ __forceinline__ void store4(void* p, int is_f32, size_t off, const float v[4]) {
    if (is_f32) Vec4<float>::store((float*)p + off, v);
    else Vec4<T>::store((T*)p + off, v);
}

// Lane layout shared by the LayerNorm kernels: one 64-lane wave per row;
// lane l holds the NC groups of 4 consecutive columns c*256 + 4l .. +3
// (c < NC, NC = ceil(H / 256)), so each load or store of a group is one
// 8- or 16-byte access and a wave covers 256 contiguous columns per group.
template <int NC>
__device__ __forceinline__ bool col_ok(int c, int lane, int H) { return c * 256 + lane * 4 < H; }

template <typename T, int NC>
__global__ __launch_bounds__(256) void ln_fwd_kernel(LnFwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.T) return;
    const int H = a.H;
    const size_t base = (size_t)row * H;
    float v[NC][4];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int idx = c * 256 + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[c][i] = 0.0f;
        if (col_ok<NC>(c, lane, H)) {
            load4<T>(a.x, a.x_f32, base + idx, v[c]);
            s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
        }
    }
    const float mean = wave_sum(s) / (float)H;
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (col_ok<NC>(c, lane, H)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float dlt = v[c][i] - mean;
                s2 += dlt * dlt;
            }
        }
    }
    const float var = wave_sum(s2) / (float)H;
    const float rs = 1.0f / sqrtf(var + a.eps);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int idx = c * 256 + lane * 4;
        if (col_ok<NC>(c, lane, H)) {
            float g[4], b[4], y[4];
            Vec4<T>::load((const T*)a.gamma + idx, g);
            Vec4<T>::load((const T*)a.beta + idx, b);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (v[c][i] - mean) * rs * g[i] + b[i];
            Vec4<T>::store((T*)a.out + base + idx, y);
            if (a.out_f32) Vec4<float>::store(a.out_f32 + base + idx, y);
            if (a.out_copy) Vec4<T>::store((T*)a.out_copy + base + idx, y);
        }
    }
    if (lane == 0) {
        a.mu[row] = mean;
        a.rstd[row] = rs;
    }
}

// LayerNorm backward: 4 waves per workgroup, each wave LN_RPW rows (two at
// a time, so that twice the loads are in flight).  Per row: gh = dy * gamma,
// dx = rstd * (gh - mean(gh) - xhat * mean(gh * xhat)) with the two means
// reduced by wave shuffles; dgamma/dbeta partials stay in the lanes' own
// columns and are added over the 4 waves in fixed order at the end, giving
// one partial row per workgroup.
constexpr int LN_RPW = 4;

template <typename T, int NC>
__global__ __launch_bounds__(256) void ln_bwd_kernel(LnBwdArgs a) {
    __shared__ float red[4][NC * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H;
    float gam[NC][4], bet[NC][4], pg[NC][4], pb[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) { gam[c][i] = 1.0f; bet[c][i] = 0.0f; pg[c][i] = 0.0f; pb[c][i] = 0.0f; }
        if (col_ok<NC>(c, lane, H)) {
            Vec4<T>::load((const T*)a.gamma + c * 256 + lane * 4, gam[c]);
            if (a.from_output) Vec4<T>::load((const T*)a.beta + c * 256 + lane * 4, bet[c]);
        }
    }
    const int row0 = (blockIdx.x * 4 + wave) * LN_RPW;
    for (int rr = 0; rr < LN_RPW; rr += 2) {
        float dy[2][NC][4], xh[2][NC][4], r[2][NC][4];
        float s1[2] = {0, 0}, s2[2] = {0, 0}, rsv[2] = {0, 0};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = row0 + rr + u;
            const bool rok = row < a.T;
            const size_t base = (size_t)(rok ? row : 0) * H;
            const float rs = rok ? a.rstd[row] : 0.0f;
            const float mu = (rok && !a.from_output) ? a.mu[row] : 0.0f;
            rsv[u] = rs;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int idx = c * 256 + lane * 4;
#pragma unroll
                for (int i = 0; i < 4; ++i) { dy[u][c][i] = 0.0f; xh[u][c][i] = 0.0f; r[u][c][i] = 0.0f; }
                if (rok && col_ok<NC>(c, lane, H)) {
                    float sv[4];
                    Vec4<T>::load((const T*)a.dout + base + idx, dy[u][c]);
                    if (a.dout_add) {
                        float t[4];
                        Vec4<float>::load(a.dout_add + base + idx, t);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dy[u][c][i] += t[i];
                    }
                    load4<T>(a.src, a.src_f32, base + idx, sv);
                    if (a.res) load4<T>(a.res, a.res_f32, base + idx, r[u][c]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xh[u][c][i] = a.from_output ? (sv[i] - bet[c][i]) / gam[c][i] : (sv[i] - mu) * rs;
                        const float gh = dy[u][c][i] * gam[c][i];
                        s1[u] += gh;
                        s2[u] += gh * xh[u][c][i];
                        pg[c][i] += dy[u][c][i] * xh[u][c][i];
                        pb[c][i] += dy[u][c][i];
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = row0 + rr + u;
            if (row >= a.T) continue;
            const float mg = wave_sum(s1[u]) / (float)H;
            const float mgx = wave_sum(s2[u]) / (float)H;
            const size_t base = (size_t)row * H;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int idx = c * 256 + lane * 4;
                if (!col_ok<NC>(c, lane, H)) continue;
                float dx[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dx[i] = rsv[u] * (dy[u][c][i] * gam[c][i] - mg - xh[u][c][i] * mgx) + r[u][c][i];
                store4<T>(a.out, a.out_f32, base + idx, dx);
                if (a.drop_out) {
                    if (a.drop.thr) {
                        const uint32_t k = keep4(a.drop.rng, (base + idx) >> 2, a.drop.thr);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dx[i] = ((k >> i) & 1u) ? dx[i] * a.drop.scale : 0.0f;
                    }
                    Vec4<T>::store((T*)a.drop_out + base + idx, dx);
                }
            }
        }
    }
    for (int which = 0; which < 2; ++which) {
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[wave][c * 256 + lane * 4 + i] = which ? pb[c][i] : pg[c][i];
        __syncthreads();
        for (int j = threadIdx.x; j < H; j += 256) {
            const float v = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
            (which ? a.part_b : a.part_g)[(size_t)blockIdx.x * H + j] = v;
        }
        __syncthreads();
    }
}

// out[n] = sum_p part[p][n]: 32 columns x 8 row phases per workgroup; phase
// j sums rows j, j+8, j+16, ... in order, then the 8 phase sums are added in
// order -- a fixed summation order, independent of scheduling.
template <typename T>
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* part, int P, int N, T* out) {
    __shared__ float red[8][33];
    const int cl = threadIdx.x & 31, ph = threadIdx.x >> 5;
    const int n = blockIdx.x * 32 + cl;
    float s = 0.0f;
    if (n < N) {
        int p = ph;
        for (; p + 24 < P; p += 32) {
            const float a0 = part[(size_t)p * N + n], a1 = part[(size_t)(p + 8) * N + n];
            const float a2 = part[(size_t)(p + 16) * N + n], a3 = part[(size_t)(p + 24) * N + n];
            s += a0; s += a1; s += a2; s += a3;
        }
        for (; p < P; p += 8) s += part[(size_t)p * N + n];
    }
    red[ph][cl] = s;
    __syncthreads();
    if (ph == 0 && n < N) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) t += red[j][cl];
        out[n] = from_f<T>(t);
    }
}

constexpr int CS_ROWS = 64;  // rows per partial in colsum_partial

template <typename T>
__global__ __launch_bounds__(256) void colsum_partial_kernel(const T* in, int rows, int N, float* part) {
    const int n4 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (n4 >= N) return;
    const int r0 = blockIdx.y * CS_ROWS;
    const int r1 = min(rows, r0 + CS_ROWS);
    float s[4] = {0, 0, 0, 0};
    for (int r = r0; r < r1; ++r) {
        float v[4];
        Vec4<T>::load(in + (size_t)r * N + n4, v);
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] += v[i];
    }
    Vec4<float>::store(part + (size_t)blockIdx.y * N + n4, s);
}

template <typename T>
__global__ __launch_bounds__(256) void dropout_apply_kernel(const T* in, T* out, size_t n, Drop d) {
    const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= n) return;
    float v[4];
    Vec4<T>::load(in + i4, v);
    if (d.thr) {
        const uint32_t k = keep4(d.rng, i4 >> 2, d.thr);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = ((k >> i) & 1u) ? v[i] * d.scale : 0.0f;
    }
    Vec4<T>::store(out + i4, v);
}

__global__ __launch_bounds__(256) void mask_dump_kernel(Drop d, uint8_t* out, size_t n) {
    const size_t i4 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (i4 >= n) return;
    const uint32_t k = d.thr ? keep4(d.rng, i4 >> 2, d.thr) : 0xFu;
    uchar4 v = make_uchar4(k & 1u, (k >> 1) & 1u, (k >> 2) & 1u, (k >> 3) & 1u);
    *reinterpret_cast<uchar4*>(out + i4) = v;
}

// ------------------------------------------------------------------ launchers
template <typename T>
static hipError_t ln_forward_t(const LnFwdArgs& a, hipStream_t st) {
    dim3 grid((a.T + 3) / 4), blk(256);
    switch ((a.H + 255) / 256) {
        case 1: hipLaunchKernelGGL((ln_fwd_kernel<T, 1>), grid, blk, 0, st, a); break;
        case 2: hipLaunchKernelGGL((ln_fwd_kernel<T, 2>), grid, blk, 0, st, a); break;
        case 3: hipLaunchKernelGGL((ln_fwd_kernel<T, 3>), grid, blk, 0, st, a); break;
        case 4: hipLaunchKernelGGL((ln_fwd_kernel<T, 4>), grid, blk, 0, st, a); break;
        case 5: case 6: hipLaunchKernelGGL((ln_fwd_kernel<T, 6>), grid, blk, 0, st, a); break;
        case 7: case 8: hipLaunchKernelGGL((ln_fwd_kernel<T, 8>), grid, blk, 0, st, a); break;
        default: hipLaunchKernelGGL((ln_fwd_kernel<T, 16>), grid, blk, 0, st, a); break;
    }
    return hipGetLastError();
}

hipError_t ln_forward(const LnFwdArgs& a, hipStream_t st) {
    switch (a.dtype) {
        case 0: return ln_forward_t<float>(a, st);
        case 1: return ln_forward_t<f16>(a, st);
        case 2: return ln_forward_t<bf16>(a, st);
    }
    return hipErrorInvalidValue;
}

int ln_backward_parts(int T) { return (T + 4 * LN_RPW - 1) / (4 * LN_RPW); }

template <typename T>
static hipError_t ln_backward_t(const LnBwdArgs& a, hipStream_t st) {
    dim3 grid(ln_backward_parts(a.T)), blk(256);
    switch ((a.H + 255) / 256) {
        case 1: hipLaunchKernelGGL((ln_bwd_kernel<T, 1>), grid, blk, 0, st, a); break;
        case 2: hipLaunchKernelGGL((ln_bwd_kernel<T, 2>), grid, blk, 0, st, a); break;
        case 3: hipLaunchKernelGGL((ln_bwd_kernel<T, 3>), grid, blk, 0, st, a); break;
        case 4: hipLaunchKernelGGL((ln_bwd_kernel<T, 4>), grid, blk, 0, st, a); break;
        case 5: case 6: hipLaunchKernelGGL((ln_bwd_kernel<T, 6>), grid, blk, 0, st, a); break;
        case 7: case 8: hipLaunchKernelGGL((ln_bwd_kernel<T, 8>), grid, blk, 0, st, a); break;
        default: return hipErrorInvalidValue;  // H <= 2048 (LDS of the partial reduction)
    }
    return hipGetLastError();
}

hipError_t ln_backward(const LnBwdArgs& a, hipStream_t st) {
    switch (a.dtype) {
        case 0: return ln_backward_t<float>(a, st);
        case 1: return ln_backward_t<f16>(a, st);
        case 2: return ln_backward_t<bf16>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t colsum_finalize(int dtype, const float* part, int P, int N, void* out, hipStream_t st) {
    dim3 grid((N + 31) / 32);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(colsum_finalize_kernel<float>, grid, dim3(256), 0, st, part, P, N, (float*)out); break;
        case 1: hipLaunchKernelGGL(colsum_finalize_kernel<f16>, grid, dim3(256), 0, st, part, P, N, (f16*)out); break;
        case 2: hipLaunchKernelGGL(colsum_finalize_kernel<bf16>, grid, dim3(256), 0, st, part, P, N, (bf16*)out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int colsum_parts(int rows) { return (rows + CS_ROWS - 1) / CS_ROWS; }

hipError_t colsum_partial(int dtype, const void* in, int rows, int N, float* part, hipStream_t st) {
    dim3 grid((N / 4 + 255) / 256, colsum_parts(rows));
    switch (dtype) {
        case 0: hipLaunchKernelGGL(colsum_partial_kernel<float>, grid, dim3(256), 0, st, (const float*)in, rows, N, part); break;
        case 1: hipLaunchKernelGGL(colsum_partial_kernel<f16>, grid, dim3(256), 0, st, (const f16*)in, rows, N, part); break;
        case 2: hipLaunchKernelGGL(colsum_partial_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)in, rows, N, part); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t dropout_apply(int dtype, const void* in, void* out, size_t n, const Drop& d, hipStream_t st) {
    dim3 grid((unsigned)((n / 4 + 255) / 256));
    switch (dtype) {
        case 0: hipLaunchKernelGGL(dropout_apply_kernel<float>, grid, dim3(256), 0, st, (const float*)in, (float*)out, n, d); break;
        case 1: hipLaunchKernelGGL(dropout_apply_kernel<f16>, grid, dim3(256), 0, st, (const f16*)in, (f16*)out, n, d); break;
        case 2: hipLaunchKernelGGL(dropout_apply_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)in, (bf16*)out, n, d); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t dropout_mask_dump(const Drop& d, uint8_t* out, size_t n, hipStream_t st) {
    dim3 grid((unsigned)((n / 4 + 255) / 256));
    hipLaunchKernelGGL(mask_dump_kernel, grid, dim3(256), 0, st, d, out, n);
    return hipGetLastError();
}

}  // namespace tel
