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

// LayerNorm backward: one workgroup per LN_ROWS rows, one thread per 4
// consecutive columns (H/4 threads).  Rows are processed LN_RB at a time; the
// two per-row sums (of g*gamma and g*gamma*xhat) are reduced across the
// workgroup in a fixed order.  Each thread keeps the dgamma/dbeta partial
// sums of its own 4 columns over the workgroup's rows, so the per-workgroup
// partial rows need no further reduction inside the kernel.
constexpr int LN_ROWS = 32;
constexpr int LN_RB = 4;

template <typename T>
__global__ __launch_bounds__(1024) void ln_bwd_kernel(LnBwdArgs a) {
    __shared__ float red[2][16][LN_RB];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int H = a.H;
    const int c4 = tid * 4;
    const bool act = c4 < H;
    float gam[4] = {0, 0, 0, 0}, bet[4] = {0, 0, 0, 0};
    if (act) {
        Vec4<T>::load((const T*)a.gamma + c4, gam);
        if (a.from_output) Vec4<T>::load((const T*)a.beta + c4, bet);
    }
    float pg[4] = {0, 0, 0, 0}, pb[4] = {0, 0, 0, 0};
    const int rbeg = blockIdx.x * LN_ROWS;
    const int rend = min(a.T, rbeg + LN_ROWS);
    for (int r0 = rbeg; r0 < rend; r0 += LN_RB) {
        float dy[LN_RB][4], xh[LN_RB][4], s1[LN_RB], s2[LN_RB];
#pragma unroll
        for (int rb = 0; rb < LN_RB; ++rb) {
            const int row = r0 + rb;
            s1[rb] = 0.0f;
            s2[rb] = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) { dy[rb][i] = 0.0f; xh[rb][i] = 0.0f; }
            if (row < rend && act) {
                const size_t off = (size_t)row * H + c4;
                float sv[4];
                Vec4<T>::load((const T*)a.dout + off, dy[rb]);
                if (a.dout_add) {
                    float t[4];
                    Vec4<float>::load(a.dout_add + off, t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dy[rb][i] += t[i];
                }
                load4<T>(a.src, a.src_f32, off, sv);
                const float rs = a.rstd[row];
                const float mu = a.from_output ? 0.0f : a.mu[row];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    xh[rb][i] = a.from_output ? (sv[i] - bet[i]) / gam[i] : (sv[i] - mu) * rs;
                    const float gh = dy[rb][i] * gam[i];
                    s1[rb] += gh;
                    s2[rb] += gh * xh[rb][i];
                    pg[i] += dy[rb][i] * xh[rb][i];
                    pb[i] += dy[rb][i];
                }
            }
        }
#pragma unroll
        for (int rb = 0; rb < LN_RB; ++rb) {
            s1[rb] = wave_sum(s1[rb]);
            s2[rb] = wave_sum(s2[rb]);
        }
        if (lane == 0) {
#pragma unroll
            for (int rb = 0; rb < LN_RB; ++rb) {
                red[0][wave][rb] = s1[rb];
                red[1][wave][rb] = s2[rb];
            }
        }
        __syncthreads();
        float mg[LN_RB], mgx[LN_RB];
#pragma unroll
        for (int rb = 0; rb < LN_RB; ++rb) {
            float t1 = 0.0f, t2 = 0.0f;
            for (int w = 0; w < nw; ++w) {
                t1 += red[0][w][rb];
                t2 += red[1][w][rb];
            }
            mg[rb] = t1 / (float)H;
            mgx[rb] = t2 / (float)H;
        }
        __syncthreads();
#pragma unroll
        for (int rb = 0; rb < LN_RB; ++rb) {
            const int row = r0 + rb;
            if (row < rend && act) {
                const size_t off = (size_t)row * H + c4;
                const float rs = a.rstd[row];
                float dx[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) dx[i] = rs * (dy[rb][i] * gam[i] - mg[rb] - xh[rb][i] * mgx[rb]);
                if (a.res) {
                    float r[4];
                    load4<T>(a.res, a.res_f32, off, r);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dx[i] += r[i];
                }
                store4<T>(a.out, a.out_f32, off, dx);
                if (a.drop_out) {
                    if (a.drop.thr) {
                        const uint32_t k = keep4(a.drop.rng, off >> 2, a.drop.thr);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dx[i] = ((k >> i) & 1u) ? dx[i] * a.drop.scale : 0.0f;
                    }
                    Vec4<T>::store((T*)a.drop_out + off, dx);
                }
            }
        }
    }
    if (act) {
        Vec4<float>::store(a.part_g + (size_t)blockIdx.x * H + c4, pg);
        Vec4<float>::store(a.part_b + (size_t)blockIdx.x * H + c4, pb);
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

int ln_backward_parts(int T) { return (T + LN_ROWS - 1) / LN_ROWS; }

hipError_t ln_backward(const LnBwdArgs& a, hipStream_t st) {
    dim3 grid(ln_backward_parts(a.T));
    const int thr = ((a.H / 4 + 63) / 64) * 64;
    if (thr > 1024) return hipErrorInvalidValue;
    switch (a.dtype) {
        case 0: hipLaunchKernelGGL(ln_bwd_kernel<float>, grid, dim3(thr), 0, st, a); break;
        case 1: hipLaunchKernelGGL(ln_bwd_kernel<f16>, grid, dim3(thr), 0, st, a); break;
        case 2: hipLaunchKernelGGL(ln_bwd_kernel<bf16>, grid, dim3(thr), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
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
