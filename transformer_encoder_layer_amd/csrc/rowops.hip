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
#include <type_traits>

namespace tel {


// Lane layout shared by the LayerNorm kernels: one 64-lane wave per row;
// lane l holds the NC groups of 4 consecutive columns c*256 + 4l .. +3
// (c < NC, NC = ceil(H / 256)), so each load or store of a group is one
// 8- or 16-byte access and a wave covers 256 contiguous columns per group.
// FULL: H is exactly NC * 256, every group is in range and no mask is
// needed (the kernels are instantiated both ways and picked at launch).
template <bool FULL>
__device__ __forceinline__ bool col_ok(int c, int lane, int H) { return FULL || c * 256 + lane * 4 < H; }

// Every load of a row is issued unconditionally so that they are all in
// flight together: a lane whose column group lies beyond H (H need not be a
// multiple of 256) reads the row's last group instead and its values are
// masked to zero; rows past T read row T-1 and store nothing.  (Loads under
// per-lane or per-flag branches would each be followed by a full memory
// wait at the branch join.)
template <bool FULL>
__device__ __forceinline__ int col_clamped(int c, int lane, int H) {
    return FULL ? c * 256 + lane * 4 : min(c * 256 + lane * 4, H - 4);
}

template <typename T, bool F32>
__device__ __forceinline__ void load4k(const void* p, size_t off, float v[4]) {
    if constexpr (F32) Vec4<float>::load((const float*)p + off, v);
    else Vec4<T>::load((const T*)p + off, v);
}
// store4k with a non-temporal hint: the LayerNorm backward's gradient output
// is read next only after several other kernels (the next LayerNorm
// backward, or the layer below's), so it should not displace the lines the
// kernels in between read.
template <typename T, bool F32>
__device__ __forceinline__ void store4k_nt(void* p, size_t off, const float v[4]) {
    if constexpr (F32 || sizeof(T) == 4) {
        typedef float f4 __attribute__((ext_vector_type(4)));
        const f4 q = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(q, reinterpret_cast<f4*>((float*)p + off));
    } else {
        typedef T t4 __attribute__((ext_vector_type(4)));
        const t4 q = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
        __builtin_nontemporal_store(q, reinterpret_cast<t4*>((T*)p + off));
    }
}
template <typename T, bool F32>
__device__ __forceinline__ void store4k(void* p, size_t off, const float v[4]) {
    if constexpr (F32) Vec4<float>::store((float*)p + off, v);
    else Vec4<T>::store((T*)p + off, v);
}

// x passed through an empty register barrier: a product feeding a rounding
// to fp16/bf16 stays an fp32 product, so two kernels that scale the same
// stored values round the same way (a mixed-precision fma would round once).
__device__ __forceinline__ float fp32_barrier(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Sum over the 64 lanes of a wave, the same value in every lane: DPP adds
// within each row of 16 lanes (quad swaps, then rotations by 4 and 8), then
// the four row sums read from lanes 0, 16, 32 and 48 -- no LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum64(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x124>(v);  // row_ror:4
    v += dpp_f32<0x128>(v);  // row_ror:8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

template <typename T, int NC, bool XF32, bool FULL>
__global__ __launch_bounds__(256) void ln_fwd_kernel(LnFwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int H = a.H;
    const int rowc = min(row, a.T - 1);
    const size_t base = (size_t)rowc * H;
    float v[NC][4], g[NC][4], bt[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int idx = col_clamped<FULL>(c, lane, H);
        load4k<T, XF32>(a.x, base + idx, v[c]);
        Vec4<T>::load((const T*)a.gamma + idx, g[c]);
        Vec4<T>::load((const T*)a.beta + idx, bt[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (!col_ok<FULL>(c, lane, H)) v[c][0] = v[c][1] = v[c][2] = v[c][3] = 0.0f;
        s += (v[c][0] + v[c][1]) + (v[c][2] + v[c][3]);
    }
    const float mean = wave_sum64(s) * (1.0f / (float)H);
    float s2 = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        if (col_ok<FULL>(c, lane, H)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float dlt = v[c][i] - mean;
                s2 += dlt * dlt;
            }
        }
    }
    const float var = wave_sum64(s2) * (1.0f / (float)H);
    const float rs = 1.0f / sqrtf(var + a.eps);
    if (row >= a.T) return;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int idx = c * 256 + lane * 4;
        if (col_ok<FULL>(c, lane, H)) {
            float y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) y[i] = (v[c][i] - mean) * rs * g[c][i] + bt[c][i];
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
// one partial row per workgroup.  The tensor layout is a compile-time mode:
//   bit 0 LN source fp32, bit 1 source is the LN output (invertible),
//   bits 2-3 residual term added to dx (0 none, 1 dtype, 2 fp32),
//   bit 4 fp32 term added to dy, bit 5 dx stored fp32, bit 6 drop(dx) stored.
constexpr int LN_RPW = 4;
enum : int {
    LNB_SRC_F32 = 1, LNB_FROM_OUT = 2, LNB_RES_LOWP = 4, LNB_RES_F32 = 8, LNB_ADD = 16, LNB_OUT_F32 = 32,
    LNB_DROP = 64
};

template <typename T, int NC, int MODE, bool FULL>
__global__ __launch_bounds__(256) void ln_bwd_kernel(LnBwdArgs a) {
    constexpr bool SRC_F32 = MODE & LNB_SRC_F32, FROM_OUT = MODE & LNB_FROM_OUT, ADD = MODE & LNB_ADD;
    constexpr bool OUT_F32 = MODE & LNB_OUT_F32, DROP = MODE & LNB_DROP;
    constexpr int RES = (MODE & LNB_RES_F32) ? 2 : (MODE & LNB_RES_LOWP) ? 1 : 0;
    __shared__ float red[4][NC * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int H = a.H;
    float gam[NC][4], bet[NC][4], pg[NC][4], pb[NC][4];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int idx = col_clamped<FULL>(c, lane, H);
        Vec4<T>::load((const T*)a.gamma + idx, gam[c]);
        if constexpr (FROM_OUT) Vec4<T>::load((const T*)a.beta + idx, bet[c]);
#pragma unroll
        for (int i = 0; i < 4; ++i) { pg[c][i] = 0.0f; pb[c][i] = 0.0f; }
    }
    const int row0 = (blockIdx.x * 4 + wave) * LN_RPW;
    for (int rr = 0; rr < LN_RPW; rr += 2) {
        float dy[2][NC][4], sv[2][NC][4], r[2][NC][4], xh[2][NC][4];
        float rsv[2], muv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int rowc = min(row0 + rr + u, a.T - 1);
            const size_t base = (size_t)rowc * H;
            rsv[u] = a.rstd[rowc];
            muv[u] = FROM_OUT ? 0.0f : a.mu[rowc];
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int idx = col_clamped<FULL>(c, lane, H);
                Vec4<T>::load((const T*)a.dout + base + idx, dy[u][c]);
                if constexpr (ADD) {
                    float t[4];
                    Vec4<float>::load(a.dout_add + base + idx, t);
#pragma unroll
                    for (int i = 0; i < 4; ++i) dy[u][c][i] += t[i];
                }
                load4k<T, SRC_F32>(a.src, base + idx, sv[u][c]);
                if constexpr (RES != 0) load4k<T, RES == 2>(a.res, base + idx, r[u][c]);
            }
        }
        float s1[2] = {0, 0}, s2[2] = {0, 0};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bool rok = row0 + rr + u < a.T;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bool ok = rok && col_ok<FULL>(c, lane, H);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d = ok ? dy[u][c][i] : 0.0f;
                    const float x = FROM_OUT ? (sv[u][c][i] - bet[c][i]) / gam[c][i] : (sv[u][c][i] - muv[u]) * rsv[u];
                    dy[u][c][i] = d;
                    xh[u][c][i] = ok ? x : 0.0f;
                    const float gh = d * gam[c][i];
                    s1[u] += gh;
                    s2[u] += gh * xh[u][c][i];
                    pg[c][i] += d * xh[u][c][i];
                    pb[c][i] += d;
                }
            }
        }
        // Dropout keep bits: lanes 2j and 2j+1 hold the two halves of one
        // 8-column Philox block of each of the two rows, so each draws the
        // block of one row and they swap halves (one Philox call per 8
        // elements).  Every lane draws, before any row or column is skipped.
        uint32_t kn[2][NC];
        if constexpr (DROP) {
            if (a.drop.thr) {
                const int odd = lane & 1;
                const int urow = min(row0 + rr + odd, a.T - 1);  // the row this lane draws for
                const size_t tok = a.row_map ? (size_t)max(a.row_map[urow], 0) : (size_t)urow;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const uint32_t k8 = keep8(a.drop.rng, (tok * H + c * 256 + (lane & ~1) * 4) >> 3, a.drop.thr);
                    const uint32_t o8 = __shfl_xor(k8, 1, 64);
                    kn[0][c] = odd ? (o8 >> 4) : (k8 & 0xFu);
                    kn[1][c] = odd ? (k8 >> 4) : (o8 & 0xFu);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int row = row0 + rr + u;
            const float mg = wave_sum64(s1[u]) * (1.0f / (float)H);
            const float mgx = wave_sum64(s2[u]) * (1.0f / (float)H);
            if (row >= a.T) continue;
            const size_t base = (size_t)row * H;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int idx = c * 256 + lane * 4;
                if (!col_ok<FULL>(c, lane, H)) continue;
                float dx[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dx[i] = rsv[u] * (dy[u][c][i] * gam[c][i] - mg - xh[u][c][i] * mgx);
                    if constexpr (RES != 0) dx[i] += r[u][c][i];
                }
                store4k_nt<T, OUT_F32>(a.out, base + idx, dx);
                if constexpr (DROP) {
                    // the mask applies to dx as stored (rounded to T when
                    // stored in T), exactly as a separate dropout pass over
                    // the stored tensor would
                    if constexpr (!OUT_F32) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) dx[i] = round_through<T>(dx[i]);
                    }
                    if (a.drop.thr) {
                        const uint32_t k = kn[u][c];
#pragma unroll
                        for (int i = 0; i < 4; ++i) dx[i] = ((k >> i) & 1u) ? fp32_barrier(dx[i] * a.drop.scale) : 0.0f;
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

// out_v[n] = sum_p part_v[p][n] for up to two vectors v (blockIdx.y),
// kColsumCols columns per workgroup, in the fixed order of colsum_block.
template <typename T>
__global__ __launch_bounds__(256) void colsum_finalize_kernel(const float* part0, const float* part1, int P, int N,
                                                              T* out0, T* out1) {
    __shared__ float red[256 / kColsumCols][kColsumCols + 1];
    colsum_block<T>(blockIdx.y ? part1 : part0, P, N, blockIdx.y ? out1 : out0, blockIdx.x * kColsumCols, red);
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

// Elementwise dropout, 8 elements (one Philox block) per thread; n % 4 == 0.
template <typename T>
__global__ __launch_bounds__(256) void dropout_apply_kernel(const T* in, T* out, size_t n, Drop d,
                                                            const int32_t* row_map, int H) {
    const size_t i8 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i8 >= n) return;
    const bool two = i8 + 4 < n;
    float v[8];
    Vec4<T>::load(in + i8, v);
    if (two) Vec4<T>::load(in + i8 + 4, v + 4);
    if (d.thr) {
        size_t e = i8;  // element id of the first of the 8 (a multiple of 8)
        if (row_map) {
            const size_t r = i8 / H;
            e = (size_t)max(row_map[r], 0) * H + (i8 - r * H);
        }
        const uint32_t k = keep8(d.rng, e >> 3, d.thr);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = ((k >> i) & 1u) ? fp32_barrier(v[i] * d.scale) : 0.0f;
    }
    Vec4<T>::store(out + i8, v);
    if (two) Vec4<T>::store(out + i8 + 4, v + 4);
}

__global__ __launch_bounds__(256) void mask_dump_kernel(Drop d, uint8_t* out, size_t n) {
    const size_t i8 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i8 >= n) return;
    const uint32_t k = d.thr ? keep8(d.rng, i8 >> 3, d.thr) : 0xFFu;
    *reinterpret_cast<uchar4*>(out + i8) = make_uchar4(k & 1u, (k >> 1) & 1u, (k >> 2) & 1u, (k >> 3) & 1u);
    if (i8 + 4 < n)
        *reinterpret_cast<uchar4*>(out + i8 + 4) =
            make_uchar4((k >> 4) & 1u, (k >> 5) & 1u, (k >> 6) & 1u, (k >> 7) & 1u);
}

// ------------------------------------------------------------------ launchers
template <typename T, int NC, bool XF32>
static void ln_fwd_launch(const LnFwdArgs& a, dim3 grid, dim3 blk, hipStream_t st) {
    if (a.H == NC * 256) hipLaunchKernelGGL((ln_fwd_kernel<T, NC, XF32, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((ln_fwd_kernel<T, NC, XF32, false>), grid, blk, 0, st, a);
}
template <typename T, bool XF32>
static hipError_t ln_forward_x(const LnFwdArgs& a, hipStream_t st) {
    dim3 grid((a.T + 3) / 4), blk(256);
    switch ((a.H + 255) / 256) {
        case 1: ln_fwd_launch<T, 1, XF32>(a, grid, blk, st); break;
        case 2: ln_fwd_launch<T, 2, XF32>(a, grid, blk, st); break;
        case 3: ln_fwd_launch<T, 3, XF32>(a, grid, blk, st); break;
        case 4: ln_fwd_launch<T, 4, XF32>(a, grid, blk, st); break;
        case 5: case 6: ln_fwd_launch<T, 6, XF32>(a, grid, blk, st); break;
        case 7: case 8: ln_fwd_launch<T, 8, XF32>(a, grid, blk, st); break;
        default: return hipErrorInvalidValue;  // H <= 2048
    }
    return hipGetLastError();
}
template <typename T>
static hipError_t ln_forward_t(const LnFwdArgs& a, hipStream_t st) {
    return a.x_f32 ? ln_forward_x<T, true>(a, st) : ln_forward_x<T, false>(a, st);
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

template <typename T, int NC, int MODE>
static void ln_bwd_launch(const LnBwdArgs& a, dim3 grid, dim3 blk, hipStream_t st) {
    if (a.H == NC * 256) hipLaunchKernelGGL((ln_bwd_kernel<T, NC, MODE, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((ln_bwd_kernel<T, NC, MODE, false>), grid, blk, 0, st, a);
}
template <typename T, int MODE>
static hipError_t ln_backward_m(const LnBwdArgs& a, hipStream_t st) {
    dim3 grid(ln_backward_parts(a.T)), blk(256);
    switch ((a.H + 255) / 256) {
        case 1: ln_bwd_launch<T, 1, MODE>(a, grid, blk, st); break;
        case 2: ln_bwd_launch<T, 2, MODE>(a, grid, blk, st); break;
        case 3: ln_bwd_launch<T, 3, MODE>(a, grid, blk, st); break;
        case 4: ln_bwd_launch<T, 4, MODE>(a, grid, blk, st); break;
        case 5: case 6: ln_bwd_launch<T, 6, MODE>(a, grid, blk, st); break;
        case 7: case 8: ln_bwd_launch<T, 8, MODE>(a, grid, blk, st); break;
        default: return hipErrorInvalidValue;  // H <= 2048 (LDS of the partial reduction)
    }
    return hipGetLastError();
}

// The tensor layouts the layer's four LayerNorm backward passes use, each
// with and without the invertible (from-output) form.
template <typename T>
static hipError_t ln_backward_t(const LnBwdArgs& a, hipStream_t st) {
    const int mode = (a.src_f32 ? LNB_SRC_F32 : 0) | (a.from_output ? LNB_FROM_OUT : 0) |
                     (a.res ? (a.res_f32 ? LNB_RES_F32 : LNB_RES_LOWP) : 0) | (a.dout_add ? LNB_ADD : 0) |
                     (a.out_f32 ? LNB_OUT_F32 : 0) | (a.drop_out ? LNB_DROP : 0);
    switch (mode) {
#define TEL_LNB(M) case (M): return ln_backward_m<T, (M)>(a, st);
        // Pre-LN, LN2: dx1 = dy + LN2'(da2), drop(dx1) for the attention branch; x1
        // and dx1 in fp32 (bf16 and fp32 layers) or fp16 (fp16 layers); or the LN output
        TEL_LNB(LNB_SRC_F32 | LNB_RES_LOWP | LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_FROM_OUT | LNB_RES_LOWP | LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_RES_LOWP | LNB_DROP)
        TEL_LNB(LNB_FROM_OUT | LNB_RES_LOWP | LNB_DROP)
        // Pre-LN, LN1: dx = dx1 + LN1'(da1), dx1 in fp32 or fp16 as above;
        // in a chained stack also the layer below's drop2(dx) (the fp16
        // forms with the drop are the LN2 ones above)
        TEL_LNB(LNB_RES_F32)
        TEL_LNB(LNB_FROM_OUT | LNB_RES_F32)
        TEL_LNB(LNB_RES_LOWP)
        TEL_LNB(LNB_FROM_OUT | LNB_RES_LOWP)
        TEL_LNB(LNB_RES_F32 | LNB_DROP)
        TEL_LNB(LNB_FROM_OUT | LNB_RES_F32 | LNB_DROP)
        // Post-LN, LN2: dz2 = LN2'(dy) in fp32, drop(dz2) for the FFN branch
        // (source z2 in fp32 or fp16, or the output y)
        TEL_LNB(LNB_SRC_F32 | LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_FROM_OUT | LNB_OUT_F32 | LNB_DROP)
        // Post-LN, LN1: dz1 = LN1'(da1 + dz2) in fp32, drop(dz1) for the attention branch
        // (source z1 or the output x1, in fp32 or, for fp16 layers, fp16)
        TEL_LNB(LNB_SRC_F32 | LNB_ADD | LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_SRC_F32 | LNB_FROM_OUT | LNB_ADD | LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_ADD | LNB_OUT_F32 | LNB_DROP)
        TEL_LNB(LNB_FROM_OUT | LNB_ADD | LNB_OUT_F32 | LNB_DROP)
#undef TEL_LNB
    }
    return hipErrorNotSupported;
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
    return colsum_finalize2(dtype, part, nullptr, P, N, out, nullptr, st);
}

hipError_t colsum_finalize2(int dtype, const float* part0, const float* part1, int P, int N, void* out0, void* out1,
                            hipStream_t st) {
    dim3 grid((N + kColsumCols - 1) / kColsumCols, part1 ? 2 : 1);
    switch (dtype) {
        case 0: hipLaunchKernelGGL(colsum_finalize_kernel<float>, grid, dim3(256), 0, st, part0, part1, P, N, (float*)out0, (float*)out1); break;
        case 1: hipLaunchKernelGGL(colsum_finalize_kernel<f16>, grid, dim3(256), 0, st, part0, part1, P, N, (f16*)out0, (f16*)out1); break;
        case 2: hipLaunchKernelGGL(colsum_finalize_kernel<bf16>, grid, dim3(256), 0, st, part0, part1, P, N, (bf16*)out0, (bf16*)out1); break;
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

hipError_t dropout_apply(int dtype, const void* in, void* out, size_t n, const Drop& d, hipStream_t st,
                         const int32_t* row_map, int H) {
    if (row_map && (H <= 0 || H % 8 || n % H)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(((n + 7) / 8 + 255) / 256));
    switch (dtype) {
        case 0: hipLaunchKernelGGL(dropout_apply_kernel<float>, grid, dim3(256), 0, st, (const float*)in, (float*)out, n, d, row_map, H); break;
        case 1: hipLaunchKernelGGL(dropout_apply_kernel<f16>, grid, dim3(256), 0, st, (const f16*)in, (f16*)out, n, d, row_map, H); break;
        case 2: hipLaunchKernelGGL(dropout_apply_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)in, (bf16*)out, n, d, row_map, H); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// ------------------------------------------------------------------ token packing
// One thread per token t (and per filler row): the packed row of t is the
// number of valid tokens of the sequences before b plus s.  B is small, so
// each thread sums the lengths it needs directly.
__global__ __launch_bounds__(256) void build_row_maps_kernel(const int32_t* len, int B, int S, int P, int32_t* map,
                                                             int32_t* inv) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    const int T = B * S;
    if (i < T) {
        const int b = i / S, s = i - b * S;
        int off = 0;
        for (int j = 0; j < b; ++j) off += min(max(len[j], 0), S);
        const int p = off + s;
        const bool valid = s < min(max(len[b], 0), S) && p < P;
        inv[i] = valid ? p : -1;
        if (valid) map[p] = i;
    }
    if (i < P) {
        int total = 0;
        for (int j = 0; j < B; ++j) total += min(max(len[j], 0), S);
        if (i >= total) map[i] = -1;
    }
}

// 8 elements (16 bytes for 16-bit types) per thread; W % 8 == 0.
template <typename T>
__global__ __launch_bounds__(256) void move_rows_kernel(const T* src, T* dst, const int32_t* idx, int rows, int W) {
    const size_t i8 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    if (i8 >= (size_t)rows * W) return;
    const int r = (int)(i8 / W), c = (int)(i8 - (size_t)r * W);
    const int from = idx ? idx[r] : -1;
    float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (from >= 0) {
        Vec4<T>::load(src + (size_t)from * W + c, v);
        Vec4<T>::load(src + (size_t)from * W + c + 4, v + 4);
    }
    Vec4<T>::store(dst + i8, v);
    Vec4<T>::store(dst + i8 + 4, v + 4);
}

// Rows s >= len[b] of [G][B][NH][S][d]: one thread per 8 elements.
template <typename T>
__global__ __launch_bounds__(256) void zero_padded_heads_kernel(T* buf, int G, int B, int NH, int S, int d,
                                                                const int32_t* len) {
    const size_t i8 = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
    const size_t n = (size_t)G * B * NH * S * d;
    if (i8 >= n) return;
    const size_t row = i8 / d;
    const int s = (int)(row % S);
    const int b = (int)((row / S / NH) % B);
    if (s < len[b]) return;
    const float z[4] = {0, 0, 0, 0};
    Vec4<T>::store(buf + i8, z);
    Vec4<T>::store(buf + i8 + 4, z);
}

template <typename F>
static hipError_t by_dtype(int dtype, F&& f) {
    switch (dtype) {
        case 0: return f((float*)nullptr);
        case 1: return f((f16*)nullptr);
        case 2: return f((bf16*)nullptr);
    }
    return hipErrorInvalidValue;
}

hipError_t build_row_maps(const int32_t* len, int B, int S, int P, int32_t* map, int32_t* inv, hipStream_t st) {
    const int n = B * S > P ? B * S : P;
    hipLaunchKernelGGL(build_row_maps_kernel, dim3((n + 255) / 256), dim3(256), 0, st, len, B, S, P, map, inv);
    return hipGetLastError();
}

hipError_t gather_rows(int dtype, const void* src, void* dst, const int32_t* map, int P, int H, hipStream_t st) {
    if (H % 8) return hipErrorInvalidValue;
    const size_t n8 = (size_t)P * H / 8;
    return by_dtype(dtype, [&](auto* tp) {
        using T = std::remove_pointer_t<decltype(tp)>;
        hipLaunchKernelGGL(move_rows_kernel<T>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           (const T*)src, (T*)dst, map, P, H);
        return hipGetLastError();
    });
}

hipError_t scatter_rows(int dtype, const void* src, void* dst, const int32_t* inv, int T, int H, hipStream_t st) {
    return gather_rows(dtype, src, dst, inv, T, H, st);  // the same move with the inverse map
}

hipError_t zero_rows(int dtype, void* buf, int r0, int r1, int W, hipStream_t st) {
    if (r1 <= r0) return hipSuccess;
    if (W % 8) return hipErrorInvalidValue;
    const size_t n8 = (size_t)(r1 - r0) * W / 8;
    return by_dtype(dtype, [&](auto* tp) {
        using T = std::remove_pointer_t<decltype(tp)>;
        hipLaunchKernelGGL(move_rows_kernel<T>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           (const T*)nullptr, (T*)buf + (size_t)r0 * W, (const int32_t*)nullptr, r1 - r0, W);
        return hipGetLastError();
    });
}

hipError_t zero_padded_heads(int dtype, void* buf, int G, int B, int NH, int S, int d, const int32_t* len,
                             hipStream_t st) {
    if (d % 8) return hipErrorInvalidValue;
    const size_t n8 = (size_t)G * B * NH * S * d / 8;
    return by_dtype(dtype, [&](auto* tp) {
        using T = std::remove_pointer_t<decltype(tp)>;
        hipLaunchKernelGGL(zero_padded_heads_kernel<T>, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, st,
                           (T*)buf, G, B, NH, S, d, len);
        return hipGetLastError();
    });
}

hipError_t dropout_mask_dump(const Drop& d, uint8_t* out, size_t n, hipStream_t st) {
    dim3 grid((unsigned)(((n + 7) / 8 + 255) / 256));
    hipLaunchKernelGGL(mask_dump_kernel, grid, dim3(256), 0, st, d, out, n);
    return hipGetLastError();
}

}  // namespace tel
