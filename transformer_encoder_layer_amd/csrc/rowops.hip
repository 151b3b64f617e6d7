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

constexpr int LN_MAXC = 16;   // H <= 64 lanes * 4 * 16 = 4096
constexpr int LN_RPW = 4;     // rows per wave in the backward

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

template <typename T>
__global__ __launch_bounds__(256) void ln_fwd_kernel(LnFwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.T) return;
    const int H = a.H;
    const size_t base = (size_t)row * H;
    float v[LN_MAXC][4];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < LN_MAXC; ++c) {
        const int idx = c * 256 + lane * 4;
        if (idx < H) {
            load4<T>(a.x, a.x_f32, base + idx, v[c]);
            s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
        }
    }
    const float mean = wave_sum(s) / (float)H;
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < LN_MAXC; ++c) {
        const int idx = c * 256 + lane * 4;
        if (idx < H) {
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
    for (int c = 0; c < LN_MAXC; ++c) {
        const int idx = c * 256 + lane * 4;
        if (idx < H) {
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

template <typename T>
__global__ __launch_bounds__(256) void ln_bwd_kernel(LnBwdArgs a) {
    __shared__ float red[4][LN_MAXC * 256 / 4 > 1024 ? 1024 : LN_MAXC * 256 / 4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H;
    float pg[LN_MAXC][4], pb[LN_MAXC][4];
#pragma unroll
    for (int c = 0; c < LN_MAXC; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) { pg[c][i] = 0.0f; pb[c][i] = 0.0f; }

    for (int rr = 0; rr < LN_RPW; ++rr) {
        const int row = (blockIdx.x * 4 + wave) * LN_RPW + rr;
        if (row >= a.T) break;
        const size_t base = (size_t)row * H;
        const float rs = a.rstd[row];
        const float mu = a.from_output ? 0.0f : a.mu[row];
        float dy[LN_MAXC][4], xh[LN_MAXC][4];
        float sg = 0.0f, sgx = 0.0f;
#pragma unroll
        for (int c = 0; c < LN_MAXC; ++c) {
            const int idx = c * 256 + lane * 4;
            if (idx < H) {
                float g[4], sv[4];
                Vec4<T>::load((const T*)a.dout + base + idx, dy[c]);
                if (a.dout_add) {
                    float t[4];
                    Vec4<float>::load(a.dout_add + base + idx, t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dy[c][i] += t[i];
                }
                Vec4<T>::load((const T*)a.gamma + idx, g);
                load4<T>(a.src, a.src_f32, base + idx, sv);
                if (a.from_output) {
                    float bt[4];
                    Vec4<T>::load((const T*)a.beta + idx, bt);
#pragma unroll
                    for (int i = 0; i < 4; ++i) xh[c][i] = (sv[i] - bt[i]) / g[i];
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) xh[c][i] = (sv[i] - mu) * rs;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float gh = dy[c][i] * g[i];
                    sg += gh;
                    sgx += gh * xh[c][i];
                    pg[c][i] += dy[c][i] * xh[c][i];
                    pb[c][i] += dy[c][i];
                }
            }
        }
        const float mg = wave_sum(sg) / (float)H;
        const float mgx = wave_sum(sgx) / (float)H;
#pragma unroll
        for (int c = 0; c < LN_MAXC; ++c) {
            const int idx = c * 256 + lane * 4;
            if (idx < H) {
                float g[4], dx[4];
                Vec4<T>::load((const T*)a.gamma + idx, g);
#pragma unroll
                for (int i = 0; i < 4; ++i) dx[i] = rs * (dy[c][i] * g[i] - mg - xh[c][i] * mgx);
                if (a.res) {
                    float r[4];
                    load4<T>(a.res, a.res_f32, base + idx, r);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dx[i] += r[i];
                }
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
    // block reduction of the dgamma / dbeta partials over the 4 waves
    for (int which = 0; which < 2; ++which) {
        for (int c0 = 0; c0 < LN_MAXC; c0 += 4) {
            // chunks c0..c0+3 cover columns [c0*256, c0*256 + 1024)
            if (c0 * 256 >= H) break;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                const int c = c0 + cc;
                const int idx = c * 256 + lane * 4;
                if (c < LN_MAXC && idx < H) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) red[wave][cc * 256 + lane * 4 + i] = which ? pb[c][i] : pg[c][i];
                }
            }
            __syncthreads();
            for (int j = threadIdx.x; j < 1024; j += 256) {
                const int col = c0 * 256 + j;
                if (col < H) {
                    const float v = (red[0][j] + red[1][j]) + (red[2][j] + red[3][j]);
                    (which ? a.part_b : a.part_g)[(size_t)blockIdx.x * H + col] = v;
                }
            }
            __syncthreads();
        }
    }
}

template <typename T>
__global__ void colsum_finalize_kernel(const float* part, int P, int N, T* out) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    float s = 0.0f;
    for (int p = 0; p < P; ++p) s += part[(size_t)p * N + n];
    out[n] = from_f<T>(s);
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
hipError_t ln_forward(const LnFwdArgs& a, hipStream_t st) {
    dim3 grid((a.T + 3) / 4);
    switch (a.dtype) {
        case 0: hipLaunchKernelGGL(ln_fwd_kernel<float>, grid, dim3(256), 0, st, a); break;
        case 1: hipLaunchKernelGGL(ln_fwd_kernel<f16>, grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL(ln_fwd_kernel<bf16>, grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int ln_backward_parts(int T) { return (T + 4 * LN_RPW - 1) / (4 * LN_RPW); }

hipError_t ln_backward(const LnBwdArgs& a, hipStream_t st) {
    dim3 grid(ln_backward_parts(a.T));
    switch (a.dtype) {
        case 0: hipLaunchKernelGGL(ln_bwd_kernel<float>, grid, dim3(256), 0, st, a); break;
        case 1: hipLaunchKernelGGL(ln_bwd_kernel<f16>, grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL(ln_bwd_kernel<bf16>, grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t colsum_finalize(int dtype, const float* part, int P, int N, void* out, hipStream_t st) {
    dim3 grid((N + 255) / 256);
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
