// gemm.hip -- GEMMs of the encoder layer on gfx950 with fused epilogues.
//
// Fast path: fp16/bf16 MFMA (v_mfma_f32_32x32x16_{f16,bf16}, fp32
// accumulation) with LDS double buffering.  A k-major operand tile is kept
// in LDS as [rows][64 k] with 16-byte chunks XOR-swizzled by row and read
// with 128-bit LDS loads; an m/n-major operand tile is kept as
// [64 k][rows + pad] exactly as in global memory and read with the gfx950
// transposing LDS load (ds_read_b64_tr_b16), so no layout needs a separate
// transpose pass.  The MFMA "A" operand is the B tile and the "B" operand
// the A tile, so each lane ends with four consecutive output columns of one
// row: epilogues (bias, GELU, dropout, residual, head split) work on
// 4-wide vectors and store 8 or 16 bytes.
//
// Generic path: a SIMT fp32-FMA tiled GEMM with bounds checks for every
// shape and dtype (the fp32 configuration and shapes the MFMA tiles do not
// divide).  Both paths share the epilogue code.
#include "gemm.h"
#include "mfma_common.h"
#include <type_traits>
#include <algorithm>

namespace tel {

// ------------------------------------------------------------------ epilogue
// out[0..1] += (v0, v1) rounded to T, as one packed atomic add (the pair
// must be 4-byte aligned).
__device__ __forceinline__ void atomic_add2(float* out, float v0, float v1) {
    atomicAdd(out, v0);
    atomicAdd(out + 1, v1);
}
__device__ __forceinline__ void atomic_add2(f16* out, float v0, float v1) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_global_atomic_fadd_v2f16((h2 __attribute__((address_space(1)))*)out, (h2){(f16)v0, (f16)v1});
}
__device__ __forceinline__ void atomic_add2(bf16* out, float v0, float v1) {
    typedef short s2 __attribute__((ext_vector_type(2)));
    const bf16 a = (bf16)v0, b = (bf16)v1;
    __builtin_amdgcn_global_atomic_fadd_v2bf16((s2 __attribute__((address_space(1)))*)out,
                                               (s2){__builtin_bit_cast(short, a), __builtin_bit_cast(short, b)});
}

// Non-temporal forms, for data whose next reader is far away (the
// backward, the optimizer) or that is read for the last time: they do not
// displace cache lines that the kernels in between still use.
template <typename T>
__device__ __forceinline__ void store4_nt(T* p, const float v[4]) {
    typedef T t4 __attribute__((ext_vector_type(4)));
    const t4 q = {(T)v[0], (T)v[1], (T)v[2], (T)v[3]};
    __builtin_nontemporal_store(q, reinterpret_cast<t4*>(p));
}
__device__ __forceinline__ void load4f_nt(const float* p, float v[4]) {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 q = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
    v[0] = q[0]; v[1] = q[1]; v[2] = q[2]; v[3] = q[3];
}
__device__ __forceinline__ uint2 load8_nt(const void* p) {
    typedef unsigned u2 __attribute__((ext_vector_type(2)));
    const u2 q = __builtin_nontemporal_load(reinterpret_cast<const u2*>(p));
    return make_uint2(q[0], q[1]);
}

// Each epilogue works on 4 consecutive columns n..n+3 of row m.  It is split
// into loads (per-column bias, per-element residual / GELU input) and the
// compute-and-store, so that a kernel can issue every load of a block of
// outputs before its first store: otherwise the compiler must assume a store
// may alias the next load and serialises each load's full latency.
template <typename T, int EPI>
struct Epi {
    static constexpr bool kBias = EPI == EPI_QKV || EPI == EPI_BIAS_DROP_RES || EPI == EPI_BIAS_GELU;
    static constexpr bool kElem =
        EPI == EPI_BIAS_DROP_RES || EPI == EPI_GELU_BWD || EPI == EPI_ADD_RES || EPI == EPI_MUL_AUX;

    static __device__ __forceinline__ void load_bias(const EpiArgs& e, int n, float b[4]) {
        if constexpr (kBias) Vec4<T>::load((const T*)e.bias + n, b);
    }
    static __device__ __forceinline__ void load_elem(const EpiArgs& e, int m, int n, float r[4]) {
        const size_t off = (size_t)m * e.ldo + n;
        if constexpr (EPI == EPI_BIAS_DROP_RES) {
            if (e.res_f32) Vec4<float>::load((const float*)e.res + off, r);
            else Vec4<T>::load((const T*)e.res + off, r);
        } else if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_MUL_AUX) {
            Vec4<T>::load((const T*)e.aux + off, r);
        } else if constexpr (EPI == EPI_ADD_RES) {
            Vec4<float>::load((const float*)e.res + off, r);
        }
    }
    // The same element inputs as raw bits, so that many loads can be in flight
    // before any is converted: a 16-byte load of fp32 sources; for dtype
    // sources the 8 bytes are loaded twice (low and high halves alike) so
    // that the source type, a runtime flag, selects an address, not a branch.
    static __device__ __forceinline__ uint4 load_elem_raw(const EpiArgs& e, int m, int n) {
        const size_t off = (size_t)m * e.ldo + n;
        const void* src = nullptr;
        bool f32 = false;
        if constexpr (EPI == EPI_BIAS_DROP_RES) {
            f32 = e.res_f32 != 0;
            src = f32 ? (const void*)((const float*)e.res + off) : (const void*)((const T*)e.res + off);
        } else if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_MUL_AUX) {
            src = (const T*)e.aux + off;
        } else if constexpr (EPI == EPI_ADD_RES) {
            f32 = true;
            src = (const float*)e.res + off;
        }
        const uint2* q = reinterpret_cast<const uint2*>(src);
        if constexpr (EPI == EPI_GELU_BWD || EPI == EPI_MUL_AUX) {
            // GELU'(u) or u: this is its last read
            const uint2 lo = load8_nt(q);
            return make_uint4(lo.x, lo.y, lo.x, lo.y);
        }
        const uint2 lo = q[0];
        const uint2 hi = q[f32 ? 1 : 0];
        return make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
    static __device__ __forceinline__ void elem_from_raw(const EpiArgs& e, uint4 raw, float r[4]) {
        bool f32 = false;
        if constexpr (EPI == EPI_BIAS_DROP_RES) f32 = e.res_f32 != 0;
        if constexpr (EPI == EPI_ADD_RES) f32 = true;
        if (f32) {
            r[0] = __uint_as_float(raw.x); r[1] = __uint_as_float(raw.y);
            r[2] = __uint_as_float(raw.z); r[3] = __uint_as_float(raw.w);
        } else {
            Vec4<T>::load(reinterpret_cast<const T*>(&raw), r);
        }
    }
    // Dropout element index of (row m, column n): token * ldo + column; PK:
    // packed rows, the token comes from row_map (filler rows use token 0).
    template <bool PK>
    static __device__ __forceinline__ uint64_t drop_element(const EpiArgs& e, int m, int n) {
        const int t = PK ? max(e.row_map[m], 0) : m;
        return (uint64_t)t * e.ldo + n;
    }
    // EPI_BIAS_DROP_RES with the keep bits of the 4 elements given (bit i:
    // column n + i; all set without dropout).
    static __device__ __forceinline__ void finish_drop(const EpiArgs& e, int m, int n, float v[4], const float b[4],
                                                       const float r[4], uint32_t k) {
        const size_t off = (size_t)m * e.ldo + n;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += b[i];
        if (e.drop.thr) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = ((k >> i) & 1u) ? v[i] * e.drop.scale : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += r[i];
        if (e.out_f32) Vec4<float>::store((float*)e.out + off, v);
        else Vec4<T>::store((T*)e.out + off, v);
    }
    template <bool PK = false>
    static __device__ __forceinline__ void finish(const EpiArgs& e, int m, int n, float v[4], const float b[4],
                                                  const float r[4]) {
        const size_t off = (size_t)m * e.ldo + n;
        if constexpr (EPI == EPI_STORE) {
            if (e.out_f32) Vec4<float>::store((float*)e.out + off, v);
            else Vec4<T>::store((T*)e.out + off, v);
        } else if constexpr (EPI == EPI_QKV) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += b[i];
            const int t = PK ? e.row_map[m] : m;
            if (PK && t < 0) return;
            const int which = (int)e.fH.div(n), rem = n - which * e.H;
            const int h = (int)e.fd.div(rem), c = rem - h * e.d;
            const int bb = (int)e.fS.div(t), s = t - bb * e.S;
            const size_t o = ((((size_t)which * e.B + bb) * e.NH + h) * e.S + s) * e.d + c;
            Vec4<T>::store((T*)e.out + o, v);
        } else if constexpr (EPI == EPI_BIAS_DROP_RES) {
            uint32_t k = 0xFu;
            if (e.drop.thr) k = keep4(e.drop.rng, drop_element<PK>(e, m, n) >> 2, e.drop.thr);
            finish_drop(e, m, n, v, b, r, k);
        } else if constexpr (EPI == EPI_BIAS_GELU) {
            // u is rounded to the storage type first, so GELU(u) and GELU'(u)
            // are those of the stored u (what a recompute from u would give)
            float g[4], d[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float u = round_through<T>(v[i] + b[i]);
                float cdf, pdf;
                normal_cdf_pdf(u, cdf, pdf);
                g[i] = __fmul_rn(u, cdf);               // GELU(u)
                d[i] = e.gelu_grad_out ? __fmaf_rn(u, pdf, cdf) : u;  // GELU'(u) or u
            }
            // GELU'(u) (or u) is next read in the backward: a non-temporal
            // store; GELU(u) feeds the next GEMM and stays cacheable
            store4_nt<T>((T*)e.out + off, d);
            if (e.out2) Vec4<T>::store((T*)e.out2 + off, g);
        } else if constexpr (EPI == EPI_GELU_BWD) {
            // GELU'(u) rounded to the storage type, exactly as the forward
            // stores it when GELU is not checkpointed (EPI_MUL_AUX path); with
            // out2, also GELU(u) (the W2 weight gradient's operand), the same
            // bits as the forward's stored GELU(u)
            float g[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float cdf, pdf;
                normal_cdf_pdf(r[i], cdf, pdf);
                v[i] *= round_through<T>(__fmaf_rn(r[i], pdf, cdf));  // GELU'(u)
                g[i] = __fmul_rn(r[i], cdf);                          // GELU(u)
            }
            Vec4<T>::store((T*)e.out + off, v);
            if (e.out2) Vec4<T>::store((T*)e.out2 + off, g);
        } else if constexpr (EPI == EPI_MUL_AUX) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] *= r[i];
            Vec4<T>::store((T*)e.out + off, v);
        } else if constexpr (EPI == EPI_HEADSPLIT) {
            const int t = PK ? e.row_map[m] : m;
            if (PK && t < 0) return;
            const int bb = (int)e.fS.div(t), s = t - bb * e.S, h = (int)e.fd.div(n), c = n - h * e.d;
            const size_t o = (((size_t)bb * e.NH + h) * e.S + s) * e.d + c;
            Vec4<T>::store((T*)e.out + o, v);
        } else if constexpr (EPI == EPI_ADD_RES) {
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] += r[i];
            Vec4<T>::store((T*)e.out + off, v);
        } else if constexpr (EPI == EPI_ATOMIC_ADD) {
            atomic_add2((T*)e.out + off, v[0], v[1]);
            atomic_add2((T*)e.out + off + 2, v[2], v[3]);
        }
    }
};

template <typename T, int EPI>
__device__ __forceinline__ void epilogue4(const EpiArgs& e, int m, int n, float v[4]) {
    float b[4] = {0, 0, 0, 0}, r[4] = {0, 0, 0, 0};
    Epi<T, EPI>::load_bias(e, n, b);
    Epi<T, EPI>::load_elem(e, m, n, r);
    if (e.row_map) Epi<T, EPI>::template finish<true>(e, m, n, v, b, r);
    else Epi<T, EPI>::template finish<false>(e, m, n, v, b, r);
}

struct GemmParams {
    const void* A;
    const void* B;
    int lda, ldb;
    int M, N, K;
    int k_per_split;  // multiple of the k tile
    EpiArgs ea;
    float* ws;        // split-K partials, [splits][M][N]
    void* rsum;       // row sums of A: dtype [M] (one split) or fp32 [splits][M] after ws
    void* rsum_out = nullptr;  // dtype [M] row sums, for splits that add into it atomically
};

// One or two GEMMs of the same tile shape run by one persistent launch: the
// work units are problem 0's (split, tile) pairs, then problem 1's.
struct GemmGroup {
    GemmParams p[2];
    int splits[2];
    int units0;  // units of problem 0 (its tiles x splits)
    int units;   // all units
    // Relaxed-determinism weight gradients: every k-split adds its partial
    // tile (and row sums) to the zeroed outputs with packed dtype atomics
    // instead of writing fp32 partials for a separate reduction.
    int atomic;
};

// ------------------------------------------------------------------ MFMA path
constexpr int KT = 64;  // k granularity the MFMA kernels need of K

// Map the linear workgroup id to an output tile.  Consecutive ids are
// dispatched round-robin over the 8 XCDs; the remap gives each XCD one
// contiguous range of tiles, walked in groups of GM tile rows so that the
// tiles resident on one XCD share A rows and B columns in its L2.
#ifndef GEMM_XCD_REMAP
#define GEMM_XCD_REMAP 1
#endif
#ifndef GEMM_GM
#define GEMM_GM 8
#endif
__device__ __forceinline__ int xcd_range(int u, int total) {
    return (GEMM_XCD_REMAP && (total & 7) == 0) ? (u & 7) * (total >> 3) + (u >> 3) : u;
}
template <bool REMAP = true>
__device__ __forceinline__ void tile_of(int pid, int tm, int tn, int& im, int& in_) {
    if (REMAP) pid = xcd_range(pid, tm * tn);
    constexpr int GM = GEMM_GM;
    const int group = pid / (GM * tn);
    const int first = group * GM;
    const int gm = min(tm - first, GM);
    const int r = pid - group * GM * tn;
    im = first + r % gm;
    in_ = r / gm;
}

// Epilogue shared by the GEMM kernels (acc layout of the 32x32x16 MFMA with
// the operand roles swapped: lane holds 4 consecutive columns of one row).
template <typename T, int EPI, int BM, int BN, int WGM, int WGN, bool PK>
__device__ __forceinline__ void gemm_epilogue_impl(const GemmParams& p, f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                                   unsigned char* smem_raw, int m0, int n0, int wm, int wn, int wave,
                                                   int lane, int split, int nsplit) {
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int MI = WM / 32, NI = WN / 32;
    // acc[i][j][g*4 + r]: row m = m0 + wm*WM + i*32 + (lane & 31),
    // columns n .. n+3 with n = n0 + wn*WN + j*32 + g*8 + (lane >> 5)*4.
    if (nsplit > 1) {  // split-K partial: fp32 to the workspace slice of this split
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int m = m0 + wm * WM + i * 32 + (lane & 31);
                    const int n = n0 + wn * WN + j * 32 + g * 8 + (lane >> 5) * 4;
                    float v[4] = {acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2],
                                  acc[i][j][g * 4 + 3]};
                    Vec4<float>::store(p.ws + ((size_t)split * p.M + m) * p.N + n, v);
                }
        return;
    }
    // Epilogue, staged through LDS (free after the main loop): for each
    // 32-row block, the wave writes its 32 x WN fp32 tile to a private LDS
    // region in the accumulator layout, then reads it back with each lane
    // holding 4 consecutive columns and consecutive lanes consecutive column
    // groups, so global loads (residual, GELU input) and stores run over
    // contiguous rows.  Element inputs are loaded PB blocks ahead, all rows of
    // a block at once, so that a wave keeps up to 128 registers' worth of
    // loads in flight instead of waiting out each load's latency.
    typedef Epi<T, EPI> E;
    constexpr int ELD = WN + 4;  // fp32 row stride: 16 rows of a column group hit distinct banks
    float* est = reinterpret_cast<float*>(smem_raw) + wave * 32 * ELD;
    constexpr int GPR = WN / 4;           // 4-column groups per row
    constexpr int RPI = 64 / GPR;         // rows per lane-iteration
    constexpr int NIT = 32 / RPI;         // lane-iterations per block
    // lanes in use: all 64 unless GPR does not divide 64 (WN = 96: 48 lanes
    // cover two rows of 24 groups; the other 16 follow row 0's addresses and
    // store nothing)
    constexpr int LANES = RPI * GPR;
    static_assert(32 % RPI == 0, "whole lane-iterations per 32-row block");
    constexpr int BUDGET = EPI == EPI_BIAS_DROP_RES ? 64 : 128;  // dropout's Philox needs registers too
    constexpr int PBMAX = BUDGET / (NIT * 4) < 1 ? 1 : BUDGET / (NIT * 4);
    constexpr int PB = E::kElem ? (MI < PBMAX ? MI : PBMAX) : 1;
    const bool lane_on = LANES == 64 || lane < LANES;
    const int cg = lane % GPR, r0 = lane_on ? lane / GPR : 0;
    const int n = n0 + wn * WN + cg * 4;
    const int mrow0 = m0 + wm * WM + r0;  // this lane's first row of block 0
    float b[4] = {0, 0, 0, 0};
    E::load_bias(p.ea, n, b);
    uint4 el[PB][NIT];
    if constexpr (E::kElem) {
#pragma unroll
        for (int pb = 0; pb < PB; ++pb)
#pragma unroll
            for (int it = 0; it < NIT; ++it) el[pb][it] = E::load_elem_raw(p.ea, mrow0 + pb * 32 + it * RPI, n);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = j * 32 + g * 8 + (lane >> 5) * 4;
                *reinterpret_cast<float4*>(est + (lane & 31) * ELD + col) =
                    make_float4(acc[i][j][g * 4 + 0], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]);
            }
        // Dropout keep bits of this lane's rows: lanes 2c and 2c+1 hold the
        // two halves of one 8-column Philox block, so for each pair of rows
        // each draws the block of one row and they swap the results (half
        // the Philox calls of one per 4 elements).
        uint32_t kn[NIT];
        if constexpr (EPI == EPI_BIAS_DROP_RES) {
            static_assert(NIT % 2 == 0 && GPR % 2 == 0, "row pairs and column-group pairs");
            const int odd = cg & 1;
#pragma unroll
            for (int t = 0; t < NIT / 2; ++t) {
                uint32_t k8 = 0xFFu;
                if (p.ea.drop.thr) {
                    const int m = m0 + wm * WM + i * 32 + (2 * t + odd) * RPI + r0;
                    k8 = keep8(p.ea.drop.rng, E::template drop_element<PK>(p.ea, m, n - odd * 4) >> 3, p.ea.drop.thr);
                }
                const uint32_t o8 = __shfl_xor(k8, 1, 64);
                kn[2 * t] = odd ? (o8 >> 4) : (k8 & 0xFu);
                kn[2 * t + 1] = odd ? (k8 >> 4) : (o8 & 0xFu);
            }
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
            const int rr = it * RPI + r0;
            const float4 q = *reinterpret_cast<const float4*>(est + rr * ELD + cg * 4);
            float v[4] = {q.x, q.y, q.z, q.w};
            float r[4] = {0, 0, 0, 0};
            if constexpr (E::kElem) E::elem_from_raw(p.ea, el[i % PB][it], r);
            if (lane_on) {
                if constexpr (EPI == EPI_BIAS_DROP_RES)
                    E::finish_drop(p.ea, m0 + wm * WM + i * 32 + rr, n, v, b, r, kn[it]);
                else
                    E::template finish<PK>(p.ea, m0 + wm * WM + i * 32 + rr, n, v, b, r);
            }
        }
        if constexpr (E::kElem) {
            if (i + PB < MI) {
#pragma unroll
                for (int it = 0; it < NIT; ++it)
                    el[i % PB][it] = E::load_elem_raw(p.ea, mrow0 + (i + PB) * 32 + it * RPI, n);
            }
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// Packed rows (row_map set) change only the head-split scatters and the
// dropout element index; the choice is made once per kernel so that the
// unpacked epilogue keeps its row arithmetic free of per-row loads.
template <typename T, int EPI, int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void gemm_epilogue(const GemmParams& p, f32x16 (&acc)[BM / WGM / 32][BN / WGN / 32],
                                              unsigned char* smem_raw, int m0, int n0, int wm, int wn, int wave,
                                              int lane, int split, int nsplit) {
    if constexpr (EPI == EPI_QKV || EPI == EPI_HEADSPLIT || EPI == EPI_BIAS_DROP_RES) {
        if (p.ea.row_map) {
            gemm_epilogue_impl<T, EPI, BM, BN, WGM, WGN, true>(p, acc, smem_raw, m0, n0, wm, wn, wave, lane, split,
                                                              nsplit);
            return;
        }
    }
    gemm_epilogue_impl<T, EPI, BM, BN, WGM, WGN, false>(p, acc, smem_raw, m0, n0, wm, wn, wave, lane, split, nsplit);
}

// ------------------------------------------------------------------ direct-load path
// Tiles of 32 k per stage, 4 stages in LDS.  Operand data goes from global
// memory straight into LDS (global_load_lds_dwordx4: lane i of a wave writes
// 16 bytes at the wave's LDS base + 16 i), so no registers stage it and no
// LDS-store instructions sit in the MFMA stream; loads run three k-tiles
// ahead.  Both operand layouts are stored unpadded with an XOR swizzle of
// their 16-byte chunks, chosen so the fragment reads are bank-conflict free
// (k-major rows of 64 bytes: chunk ^ ((row >> 2) & 3); m/n-major rows of
// R >= 128 elements: chunk ^ 4 (k & 3)).
constexpr int DKT = 32;    // k per stage
constexpr int DNS = 4;     // stages

__device__ __forceinline__ int kmaj32_off(int row, int k) {
    return row * 32 + (((k >> 3) ^ ((row >> 2) & 3)) << 3) + (k & 7);
}
// Chunk swizzle of an m/n-major row k of R elements.  R a multiple of 128:
// chunk ^ 4 (k & 3), so the four k rows of a transposing read (whose bases
// fall on one bank) take four distinct 16-dword windows.  R = 192 (24 chunks,
// rows 96 dwords apart: rows k and k+2 share banks): chunk ^ 4 ((k >> 1) & 1),
// which keeps every chunk inside its aligned group of 8 and moves rows k+2
// and k+3 16 dwords away from rows k and k+1.
template <int R>
__device__ __forceinline__ int mn_swz(int k) {
    static_assert(R % 128 == 0 || R == 192, "m/n-major tile width");
    return R % 128 == 0 ? 4 * (k & 3) : 4 * ((k >> 1) & 1);
}
template <int R>
__device__ __forceinline__ int mn32_off(int k, int col) {
    return k * R + (((col >> 3) ^ mn_swz<R>(k)) << 3) + (col & 7);
}

// One wave-wide direct load: lane i copies the 16 bytes at sbase + voff to
// LDS byte address m0v + 16 i (m0v wave-uniform).  The scalar-base form
// keeps the per-lane offset fixed over the k loop: advancing to the next k
// tile is one scalar add on sbase, and the LDS address is scalar arithmetic,
// so a load costs two instructions.  Written as inline asm on purpose: the
// compiler would otherwise treat every later LDS read as dependent on every
// direct load in flight and wait for all of them, serialising the stage
// ring.  The instruction has no result registers (its inputs are read at
// issue); its completion is ordered explicitly with s_waitcnt vmcnt and the
// workgroup barrier before any wave reads the stage.  M0 is written and
// consumed inside the same statement, and nothing else in these kernels
// uses it.
__device__ __forceinline__ void dl_load16(const void* sbase, uint32_t voff, uint32_t m0v) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "s"(m0v)
                 : "memory");
}

// Direct-load plan of one operand tile (R rows of m or n, 32 of k) for one
// wave: the wave issues PER of the tile's NQ wave-loads (q = wave + j*NW);
// voff[j] is this lane's source byte offset from the tile origin (row0, k0).
template <typename T, bool KMAJ, int R, int NW>
struct DlPlan {
    static constexpr int NQ = R * DKT * (int)sizeof(T) / 1024;
    static constexpr int PER = NQ / NW;
    static_assert(NQ % NW == 0, "tile/wave mismatch");
    uint32_t voff[PER];

    __device__ __forceinline__ DlPlan(int ld, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int slot = (wave + j * NW) * 64 + lane;  // 16-byte slot of the tile this lane fills
            if constexpr (KMAJ) {
                const int row = slot >> 2, p = slot & 3;
                const int c = p ^ ((row >> 2) & 3);
                voff[j] = (uint32_t)((row * ld + c * 8) * (int)sizeof(T));
            } else {
                constexpr int CPR = R / 8;
                const int k = slot / CPR, p = slot % CPR;
                const int ch = p ^ mn_swz<R>(k);
                voff[j] = (uint32_t)((k * ld + ch * 8) * (int)sizeof(T));
            }
        }
    }
    // tile whose origin is at byte address `origin`, into LDS bytes lds_bytes
    __device__ __forceinline__ void issue(const char* origin, uint32_t lds_bytes, int wave) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) issue_one(origin, lds_bytes, wave, j);
    }
    __device__ __forceinline__ void issue_one(const char* origin, uint32_t lds_bytes, int wave, int j) const {
        dl_load16(origin, voff[j], lds_bytes + (uint32_t)(wave + j * NW) * 1024u);
    }
};

template <typename T, bool KMAJ, int R>
__device__ __forceinline__ typename MfmaOp<T>::v8 dl_frag(const T* lds, int rb, int ks, int lane) {
    if constexpr (KMAJ) {
        typedef typename MfmaOp<T>::v8 v8;
        const int row = rb + (lane & 31);
        return *reinterpret_cast<const v8*>(lds + kmaj32_off(row, ks * 16 + (lane >> 5) * 8));
    } else {
        const int i = lane & 15, G = lane >> 4;
        const int k0 = ks * 16 + (G >> 1) * 8 + (i >> 2);
        const int col = rb + (G & 1) * 16 + (i & 3) * 4;
        const i16x4 lo = ds_read_tr16(lds + mn32_off<R>(k0, col));
        const i16x4 hi = ds_read_tr16(lds + mn32_off<R>(k0 + 4, col));
        return join8<T>(lo, hi);
    }
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <typename T, int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(WGM* WGN * 64) void gemm_dl_kernel(GemmParams p) {
    constexpr int NW = WGM * WGN, NT = NW * 64;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int MI = WM / 32, NI = WN / 32;
    constexpr int AEL = BM * DKT, BEL = BN * DKT, STAGE = AEL + BEL;
    constexpr int LPW = (AEL + BEL) * (int)sizeof(T) / 1024 / NW;  // direct loads per wave per stage
    typedef typename MfmaOp<T>::v8 v8;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* smem = reinterpret_cast<T*>(smem_raw);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave % WGN;
    const int tm = p.M / BM, tn = p.N / BN;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const DlPlan<T, AK, BM, NW> pa(p.lda, wave_s, lane);
    const DlPlan<T, BKM, BN, NW> pb(p.ldb, wave_s, lane);
    // Persistent over tiles: a workgroup takes tiles blockIdx.x, +gridDim.x,
    // ...; the stores of one tile's epilogue drain while the next tile's
    // loads and MFMAs run.
    for (int pid = blockIdx.x; pid < tm * tn; pid += gridDim.x) {
        if (pid != (int)blockIdx.x) __syncthreads();  // the last epilogue is done with LDS
        int im, in_;
        tile_of(pid, tm, tn, im, in_);
        const int m0 = im * BM, n0 = in_ * BN;
        const int kbeg = blockIdx.z * p.k_per_split;
        const int kend = min(p.K, kbeg + p.k_per_split);
        const int nk = (kend - kbeg) / DKT;
        const T* A = (const T*)p.A;
        const T* B = (const T*)p.B;

        // bias gradient fused into a weight gradient (tile column 0 only): each
        // thread sums a fixed 8-row chunk of A over the k rows it reads from LDS
        const bool do_rsum = !AK && p.rsum != nullptr && in_ == 0;
        float rs[8] = {0, 0, 0, 0, 0, 0, 0, 0};

        f32x16 acc[MI][NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        // scalar tile origins (advanced by one k tile per issue) and LDS byte addresses
        const char* oa = reinterpret_cast<const char*>(A + (AK ? (size_t)m0 * p.lda + kbeg : (size_t)kbeg * p.lda + m0));
        const char* ob = reinterpret_cast<const char*>(B + (BKM ? (size_t)n0 * p.ldb + kbeg : (size_t)kbeg * p.ldb + n0));
        const size_t sta = (size_t)(AK ? DKT : DKT * p.lda) * sizeof(T);
        const size_t stb = (size_t)(BKM ? DKT : DKT * p.ldb) * sizeof(T);
        const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem_raw;
        int issued = 0;  // k tiles issued so far
        auto issue_next = [&]() {
            const uint32_t st = lds0 + (uint32_t)((issued % DNS) * STAGE * (int)sizeof(T));
            pa.issue(oa, st, wave_s);
            pb.issue(ob, st + AEL * (uint32_t)sizeof(T), wave_s);
            oa += sta;
            ob += stb;
            ++issued;
        };
        // fragments of one 16-wide k-step of a stage
        auto read_ks = [&](int kt, int ks, v8 (&fa)[MI], v8 (&fb)[NI]) {
            const T* sa = smem + (kt % DNS) * STAGE;
            const T* sb = sa + AEL;
#pragma unroll
            for (int i = 0; i < MI; ++i) fa[i] = dl_frag<T, AK, BM>(sa, wm * WM + i * 32, ks, lane);
#pragma unroll
            for (int j = 0; j < NI; ++j) fb[j] = dl_frag<T, BKM, BN>(sb, wn * WN + j * 32, ks, lane);
        };
        auto rowsums = [&](int kt) {
            if constexpr (!AK) {
                if (do_rsum) {
                    const T* sa = smem + (kt % DNS) * STAGE;
                    constexpr int CPR = BM / 8;
#pragma unroll
                    for (int c = tid; c < DKT * CPR; c += NT) {
                        const int k = c / CPR;
                        typedef T t8 __attribute__((ext_vector_type(8)));
                        const t8 x = *reinterpret_cast<const t8*>(sa + mn32_off<BM>(k, (c % CPR) * 8));
#pragma unroll
                        for (int e = 0; e < 8; ++e) rs[e] += to_f(x[e]);
                    }
                }
            }
        };
        auto mfmas = [&](const v8 (&fa)[MI], const v8 (&fb)[NI]) {
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NI; ++j) acc[i][j] = MfmaOp<T>::mma(fb[j], fa[i], acc[i][j]);
        };
        // the same MFMAs with the next tile's direct loads spread over them
        // (one after every NQ/LPW-th MFMA) rather than issued together
        constexpr int NQ = MI * NI;
        static_assert(LPW <= NQ, "loads per MFMA block");
        auto mfmas_issue = [&](const v8 (&fa)[MI], const v8 (&fb)[NI]) {
            const uint32_t st = lds0 + (uint32_t)((issued % DNS) * STAGE * (int)sizeof(T));
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                acc[q / NI][q % NI] = MfmaOp<T>::mma(fb[q % NI], fa[q / NI], acc[q / NI][q % NI]);
                if (q % (NQ / LPW) == 0 && q / (NQ / LPW) < LPW) {
                    const int l = q / (NQ / LPW);
                    if (l < DlPlan<T, AK, BM, NW>::PER) pa.issue_one(oa, st, wave_s, l);
                    else pb.issue_one(ob, st + AEL * (uint32_t)sizeof(T), wave_s, l - DlPlan<T, AK, BM, NW>::PER);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            oa += sta;
            ob += stb;
            ++issued;
        };

#pragma unroll
        for (int s0 = 0; s0 < DNS - 1; ++s0)
            if (s0 < nk) issue_next();
        // tile 0 landed: the tiles issued after it may still be in flight
        if (nk >= DNS - 1) wait_vmcnt<(DNS - 2) * LPW>();
        else if (nk == 2) wait_vmcnt<LPW>();
        else wait_vmcnt<0>();
        __syncthreads();
        // Per k-tile kt (fragments of its first k-step already in f0):
        //   read its second k-step -> f1; MFMAs on f0;
        //   make tile kt+1 visible (its loads landed on every wave; every wave is
        //   past tile kt-1, whose stage the loads of tile kt+3 now overwrite);
        //   read tile kt+1's first k-step -> f0; MFMAs on f1.
        // The steady state (a tile still to issue) is one branch-free block, so
        // the scheduling fences hold; the last DNS-1 tiles run in a peeled loop.
        v8 fa0[MI], fb0[NI], fa1[MI], fb1[NI];
        read_ks(0, 0, fa0, fb0);
        int kt = 0;
        for (; kt < nk - (DNS - 1); ++kt) {
            read_ks(kt, 1, fa1, fb1);
            rowsums(kt);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            wait_vmcnt<(DNS - 3) * LPW>();
            __syncthreads();
            read_ks(kt + 1, 0, fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            mfmas_issue(fa1, fb1);  // tile kt+3 into the stage tile kt-1 left
            __builtin_amdgcn_sched_barrier(0);
        }
        for (; kt < nk; ++kt) {
            read_ks(kt, 1, fa1, fb1);
            rowsums(kt);
            __builtin_amdgcn_sched_barrier(0);
            mfmas(fa0, fb0);
            __builtin_amdgcn_sched_barrier(0);
            if (kt + 1 < nk) {
                if (kt + 2 < nk) wait_vmcnt<LPW>();
                else wait_vmcnt<0>();
                __syncthreads();
                read_ks(kt + 1, 0, fa0, fb0);
            }
            __builtin_amdgcn_sched_barrier(0);
            mfmas(fa1, fb1);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();

        if constexpr (!AK) {
            if (do_rsum) {
                // threads tid, tid + CPR, ... hold the same 8 rows: add in that order
                constexpr int CPR = BM / 8;
                float* red = reinterpret_cast<float*>(smem_raw);
#pragma unroll
                for (int e = 0; e < 8; ++e) red[tid * 8 + e] = rs[e];
                __syncthreads();
                if (tid < CPR) {
                    float t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    for (int q = tid; q < NT; q += CPR)
#pragma unroll
                        for (int e = 0; e < 8; ++e) t[e] += red[q * 8 + e];
                    const int mrow = m0 + tid * 8;
                    if (gridDim.z > 1) {
                        float* out = reinterpret_cast<float*>(p.rsum) + (size_t)blockIdx.z * p.M + mrow;
#pragma unroll
                        for (int e = 0; e < 8; ++e) out[e] = t[e];
                    } else {
                        T* out = reinterpret_cast<T*>(p.rsum) + mrow;
#pragma unroll
                        for (int e = 0; e < 8; ++e) out[e] = from_f<T>(t[e]);
                    }
                }
                __syncthreads();
            }
        }
        gemm_epilogue<T, EPI, BM, BN, WGM, WGN>(p, acc, smem_raw, m0, n0, wm, wn, wave, lane, blockIdx.z, gridDim.z);
    }
}

// ------------------------------------------------- 256x256 tiles, one wave per SIMD
// Four waves in a 2 x 2 grid of 128x128 wave tiles; k tiles 64 deep in as
// many LDS stages as fit (two of 64 KB at 256x256, three of 48 KB at
// 256x128, so that loads run two k tiles ahead where the k tile is short).  Compared with two waves per SIMD on 128x64 wave
// tiles: 8 fragment reads feed 16 MFMAs (a third fewer LDS bytes per MFMA,
// and LDS traffic is what bounds the loop), k-major rows are 128 bytes so
// every direct load fetches whole cache lines, and there is one barrier per
// 64 k instead of per 32.  No second wave on a SIMD covers waits, so the k
// loop is software pipelined by hand: each MFMA is paired with at most two
// memory instructions (a fragment read for the next k-step, a direct load of
// the tile after next), fenced so that the pairing survives scheduling.
constexpr int QKT = 64;  // k per stage
// LDS stages of a BM x BN tile: three where they fit in the 160 KB, else two
// (128x128 keeps two, so that two workgroups share a CU)
constexpr int dl4_stages(int BM, int BN, int esz) {
    return BM + BN >= 384 && 3 * (BM + BN) * QKT * esz <= 160 * 1024 ? 3 : 2;
}

// k-major rows of 64 k (128 bytes): 16-byte chunk c of row r is stored at
// chunk c ^ ((r >> 1) & 7), so the 16 rows read by each quarter of a wave's
// 128-bit fragment load fall in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int kmaj64_off(int row, int k) {
    return row * 64 + (((k >> 3) ^ ((row >> 1) & 7)) << 3) + (k & 7);
}

// Direct-load plan of one 256-row operand tile, 64 k deep, for one of four
// waves: PER wave-loads each (q = wave + 4 j); voff[j] is this lane's
// source byte offset from the tile origin.
template <typename T, bool KMAJ, int R>
struct Dl4Plan {
    static constexpr int NQ = R * QKT * (int)sizeof(T) / 1024;
    static constexpr int PER = NQ / 4;
    uint32_t voff[PER];
    __device__ __forceinline__ Dl4Plan(int ld, int wave, int lane) {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int slot = (wave + j * 4) * 64 + lane;
            if constexpr (KMAJ) {
                const int row = slot >> 3, c = (slot & 7) ^ ((row >> 1) & 7);
                voff[j] = (uint32_t)((row * ld + c * 8) * (int)sizeof(T));
            } else {
                constexpr int CPR = R / 8;
                const int k = slot / CPR, ch = (slot % CPR) ^ mn_swz<R>(k);
                voff[j] = (uint32_t)((k * ld + ch * 8) * (int)sizeof(T));
            }
        }
    }
    __device__ __forceinline__ void issue_one(const char* origin, uint32_t lds_bytes, int wave, int j) const {
        dl_load16(origin, voff[j], lds_bytes + (uint32_t)(wave + j * 4) * 1024u);
    }
};

template <typename T, bool KMAJ, int R>
__device__ __forceinline__ typename MfmaOp<T>::v8 dl4_frag(const T* lds, int rb, int ks, int lane) {
    if constexpr (KMAJ) {
        typedef typename MfmaOp<T>::v8 v8;
        const int row = rb + (lane & 31);
        return *reinterpret_cast<const v8*>(lds + kmaj64_off(row, ks * 16 + (lane >> 5) * 8));
    } else {
        return dl_frag<T, false, R>(lds, rb, ks, lane);  // [k][R] layout, any k depth
    }
}

// acc + the sum of the 8 elements of an operand fragment: packed dot
// products against (1, 1), exact products summed in fp32.
__device__ __forceinline__ float frag_sum8(f16x8 x, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < 8; e += 2) acc = __builtin_amdgcn_fdot2((h2){x[e], x[e + 1]}, (h2){1, 1}, acc, false);
    return acc;
}
__device__ __forceinline__ float frag_sum8(bf16x8 x, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int e = 0; e < 8; e += 2)
        acc = __builtin_amdgcn_fdot2_f32_bf16((b2){x[e], x[e + 1]}, (b2){1, 1}, acc, false);
    return acc;
}

template <typename T, int BM, int BN, bool AK, bool BKM, int EPI>
__global__ __launch_bounds__(256) void gemm_dl4_kernel(GemmGroup G) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MI = WM / 32, NI = WN / 32;  // A and B fragments per k-step
    constexpr int NF = MI + NI;                // fragments per k-step: MI A, NI B
    constexpr int NQ = MI * NI;                // MFMAs per k-step
    constexpr int LA = BM * QKT * (int)sizeof(T) / 1024 / 4;  // direct loads per wave per stage: A
    constexpr int LPW = LA + BN * QKT * (int)sizeof(T) / 1024 / 4;  // A and B
    constexpr int AEL = BM * QKT, STAGE = (BM + BN) * QKT;
    constexpr int NS = dl4_stages(BM, BN, (int)sizeof(T));
    static_assert(NS == 2 || NS == 3, "stage count");
    typedef typename MfmaOp<T>::v8 v8;

    extern __shared__ __align__(16) unsigned char smem_raw[];
    T* smem = reinterpret_cast<T*>(smem_raw);
    // The accumulators (up to 256 per lane) must live in the accumulation
    // registers; the compiler gives MFMAs that operand form only in kernels
    // that it sees using those registers.
    asm volatile("; accumulation registers in use" ::: "a0");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)smem_raw;
    for (int u = blockIdx.x; u < G.units; u += gridDim.x) {
        if (u != (int)blockIdx.x) __syncthreads();  // the last epilogue is done with LDS
        // each XCD takes one contiguous range of the units (whole k-splits
        // of one problem where they divide evenly), so the A and B panels
        // its L2 fetches serve every tile of that range
        const int v = xcd_range(u, G.units);
        const int g = v >= G.units0 ? 1 : 0;
        const GemmParams& p = g ? G.p[1] : G.p[0];
        const int nsplit = g ? G.splits[1] : G.splits[0];
        const int tm = p.M / BM, tn = p.N / BN;
        const int lu = v - (g ? G.units0 : 0);
        const int split = lu / (tm * tn), pid = lu - split * (tm * tn);
        const Dl4Plan<T, AK, BM> pa(p.lda, wave_s, lane);
        const Dl4Plan<T, BKM, BN> pb(p.ldb, wave_s, lane);
        int im, in_;
        tile_of<false>(pid, tm, tn, im, in_);
        const int m0 = im * BM, n0 = in_ * BN;
        const int kbeg = split * p.k_per_split;
        const int kend = min(p.K, kbeg + p.k_per_split);
        const int nk = (kend - kbeg) / QKT;
        const T* A = (const T*)p.A;
        const T* B = (const T*)p.B;
        // bias gradient fused into a weight gradient: every lane sums the A
        // (= dY^T) fragments it feeds to the MFMAs, row (lane & 31) of each
        // 32-row block over its half of each k-step; tile column 0 stores.
        float rsa[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i) rsa[i] = 0.0f;

        f32x16 acc[MI][NI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NI; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

        const char* oa = reinterpret_cast<const char*>(A + (AK ? (size_t)m0 * p.lda + kbeg : (size_t)kbeg * p.lda + m0));
        const char* ob = reinterpret_cast<const char*>(B + (BKM ? (size_t)n0 * p.ldb + kbeg : (size_t)kbeg * p.ldb + n0));
        const size_t sta = (size_t)(AK ? QKT : QKT * p.lda) * sizeof(T);
        const size_t stb = (size_t)(BKM ? QKT : QKT * p.ldb) * sizeof(T);
        // direct load q of the current origins (0..LA-1 A, then B) into stage st
        auto load_q = [&](int st, int q) {
            const uint32_t base = lds0 + (uint32_t)(st * STAGE * (int)sizeof(T));
            if (q < LA) pa.issue_one(oa, base, wave_s, q);
            else pb.issue_one(ob, base + AEL * (uint32_t)sizeof(T), wave_s, q - LA);
        };
        auto frag = [&](const T* st, int ks, int q) -> v8 {
            if (q < MI) return dl4_frag<T, AK, BM>(st, wm * WM + q * 32, ks, lane);
            return dl4_frag<T, BKM, BN>(st + AEL, wn * WN + (q - MI) * 32, ks, lane);
        };
        v8 fr[2][NF];  // fragment sets: [0..MI-1] A, [MI..] B
        // NQ MFMAs on fragment set S, paired with reads of k-step RKS of stage
        // RST into set S^1 (if RD) and the direct loads L0 .. L1-1 of the
        // current origins into stage LST (if the wave-uniform LOK holds),
        // spread over the MFMAs; RD, L0 and L1 are literals
#define TEL_DL4_BLOCK_IF(S, RD, RST, RKS, LST, L0, L1, LOK)                                              \
    _Pragma("unroll") for (int q = 0; q < NQ; ++q) {                                                     \
        acc[q / NI][q % NI] = MfmaOp<T>::mma(fr[S][MI + q % NI], fr[S][q / NI], acc[q / NI][q % NI]);    \
        if (!AK && q < MI) rsa[q] = frag_sum8(fr[S][q], rsa[q]);                                         \
        if (RD && q < NF) fr[(S) ^ 1][q] = frag((RST), (RKS), q);                                         \
        _Pragma("unroll") for (int l = (L0) + q * ((L1) - (L0)) / NQ; l < (L0) + (q + 1) * ((L1) - (L0)) / NQ; \
                               ++l) if (LOK) load_q((LST), l);                                           \
        __builtin_amdgcn_sched_barrier(0);                                                               \
    }
#define TEL_DL4_BLOCK(S, RD, RST, RKS, LST, L0, L1) TEL_DL4_BLOCK_IF(S, RD, RST, RKS, LST, L0, L1, true)

        int kt = 0, sc = 0;  // sc = kt % NS
        if constexpr (NS == 3) {
            // Loads of tile kt+2 are spread over the whole of k tile kt-1's
            // last k-step (the first L4, into the stage tile kt-1 just freed)
            // and k tile kt's first three (the rest), so that no k-step issues
            // more than a quarter of a tile's loads: bunched together they
            // back up the load path and stall the MFMA issue behind them.
            constexpr int LQ = LPW / 4, L4 = LPW - 3 * LQ;
            // prologue: tiles 0 and 1 whole, the first L4 loads of tile 2
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                if (t < nk) {
#pragma unroll
                    for (int q = 0; q < LPW; ++q) load_q(t, q);
                    oa += sta;
                    ob += stb;
                }
            }
            if (nk > 2) {
#pragma unroll
                for (int q = 0; q < L4; ++q) load_q(2, q);
                wait_vmcnt<LPW + L4>();  // tile 0 landed
            } else if (nk == 2) {
                wait_vmcnt<LPW>();
            } else {
                wait_vmcnt<0>();
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < NF; ++q) fr[0][q] = frag(smem, 0, q);
            // steady state: tile kt+2 is completed, tile kt+3 begun
            for (; kt < nk - 3; ++kt) {
                const int sn = sc == 2 ? 0 : sc + 1, sp = sn == 2 ? 0 : sn + 1;  // stages of kt+1, kt+2
                const T* cur = smem + sc * STAGE;
                const T* nxt = smem + sn * STAGE;
                __builtin_amdgcn_sched_barrier(0);
                TEL_DL4_BLOCK(0, 1, cur, 1, sp, L4, L4 + LQ)
                TEL_DL4_BLOCK(1, 1, cur, 2, sp, L4 + LQ, L4 + 2 * LQ)
                TEL_DL4_BLOCK(0, 1, cur, 3, sp, L4 + 2 * LQ, LPW)
                oa += sta;
                ob += stb;
                wait_vmcnt<LPW>();  // tile kt+1 landed; tile kt+2 may be in flight
                __syncthreads();
                TEL_DL4_BLOCK(1, 1, nxt, 0, sc, 0, L4)
                sc = sn;
            }
            for (; kt < nk; ++kt) {
                const int sn = sc == 2 ? 0 : sc + 1, sp = sn == 2 ? 0 : sn + 1;
                const T* cur = smem + sc * STAGE;
                const T* nxt = smem + sn * STAGE;
                // tile kt+2, when it exists, is the last one: complete it
                const bool more = kt + 2 < nk;
                __builtin_amdgcn_sched_barrier(0);
                TEL_DL4_BLOCK_IF(0, 1, cur, 1, sp, L4, L4 + LQ, more)
                TEL_DL4_BLOCK_IF(1, 1, cur, 2, sp, L4 + LQ, L4 + 2 * LQ, more)
                TEL_DL4_BLOCK_IF(0, 1, cur, 3, sp, L4 + 2 * LQ, LPW, more)
                if (more) wait_vmcnt<LPW>();
                else wait_vmcnt<0>();
                if (kt + 1 < nk) {
                    __syncthreads();
#pragma unroll
                    for (int q = 0; q < NF; ++q) fr[0][q] = frag(nxt, 0, q);
                }
                __builtin_amdgcn_sched_barrier(0);
                TEL_DL4_BLOCK(1, 0, cur, 0, 0, 0, 0)
                sc = sn;
            }
        } else {
            // Two stages: the loads of tile kt+1 go out half in k tile
            // kt-1's last k-step (into the stage tile kt-1 just freed) and
            // half in k tile kt's first, two k-steps before the wait for them.
            constexpr int H1 = LPW / 2;
            // prologue: tile 0 whole, the first H1 loads of tile 1
#pragma unroll
            for (int q = 0; q < LPW; ++q) load_q(0, q);
            oa += sta;
            ob += stb;
            if (nk > 1) {
#pragma unroll
                for (int q = 0; q < H1; ++q) load_q(1, q);
                wait_vmcnt<H1>();  // tile 0 landed
            } else {
                wait_vmcnt<0>();
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < NF; ++q) fr[0][q] = frag(smem, 0, q);
            // Per k tile kt (stage kt & 1; k-step 0 fragments already in set
            // 0): k-steps 0..2 each read the next k-step of the stage (the
            // first also completes tile kt+1's loads); then tile kt+1 is made
            // visible (its loads landed on every wave, and every wave has read
            // all of tile kt, whose stage tile kt+2 now takes), and k-step 3
            // reads tile kt+1's first k-step while tile kt+2's first loads go
            // out.  The steady state is one branch-free block; the last two
            // tiles are peeled.
            for (; kt < nk - 2; ++kt) {
                const int sn = sc ^ 1;
                const T* cur = smem + sc * STAGE;
                const T* nxt = smem + sn * STAGE;
                __builtin_amdgcn_sched_barrier(0);
                TEL_DL4_BLOCK(0, 1, cur, 1, sn, H1, LPW)
                oa += sta;
                ob += stb;
                TEL_DL4_BLOCK(1, 1, cur, 2, 0, 0, 0)
                TEL_DL4_BLOCK(0, 1, cur, 3, 0, 0, 0)
                wait_vmcnt<0>();
                __syncthreads();
                TEL_DL4_BLOCK(1, 1, nxt, 0, sc, 0, H1)
                sc = sn;
            }
            for (; kt < nk; ++kt) {
                const int sn = sc ^ 1;
                const T* cur = smem + sc * STAGE;
                const T* nxt = smem + sn * STAGE;
                const bool more = kt + 1 < nk;  // tile kt+1 (begun) is the last one: complete it
                __builtin_amdgcn_sched_barrier(0);
                TEL_DL4_BLOCK_IF(0, 1, cur, 1, sn, H1, LPW, more)
                TEL_DL4_BLOCK(1, 1, cur, 2, 0, 0, 0)
                TEL_DL4_BLOCK(0, 1, cur, 3, 0, 0, 0)
                if (more) {
                    wait_vmcnt<0>();
                    __syncthreads();
#pragma unroll
                    for (int q = 0; q < NF; ++q) fr[0][q] = frag(nxt, 0, q);
                }
                __builtin_amdgcn_sched_barrier(0);
                TEL_DL4_BLOCK(1, 0, cur, 0, 0, 0, 0)
                sc = sn;
            }
        }
#undef TEL_DL4_BLOCK
#undef TEL_DL4_BLOCK_IF
        __syncthreads();

        const bool atomic = !AK && EPI == EPI_STORE && nsplit > 1 && G.atomic;
        if constexpr (!AK) {
            if (p.rsum != nullptr && in_ == 0) {
                // lanes l and l + 32 hold the two k halves of row l; waves with
                // wn = 1 computed the same sums
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const float t = rsa[i] + __shfl_xor(rsa[i], 32, 64);
                    const float t1 = __shfl_down(t, 1, 64);  // row l + 1's sum, for the packed add
                    if (wn == 0 && lane < 32) {
                        const int mrow = m0 + wm * WM + i * 32 + lane;
                        if (atomic) {
                            if (!(lane & 1)) atomic_add2(reinterpret_cast<T*>(p.rsum_out) + mrow, t, t1);
                        } else if (nsplit > 1) {
                            reinterpret_cast<float*>(p.rsum)[(size_t)split * p.M + mrow] = t;
                        } else {
                            reinterpret_cast<T*>(p.rsum)[mrow] = from_f<T>(t);
                        }
                    }
                }
            }
        }
        if constexpr (!AK && EPI == EPI_STORE) {
            if (atomic) {
                // staged through LDS like a plain store, so that each packed
                // atomic instruction covers contiguous row segments
                gemm_epilogue_impl<T, EPI_ATOMIC_ADD, BM, BN, 2, 2, false>(p, acc, smem_raw, m0, n0, wm, wn, wave,
                                                                          lane, 0, 1);
                continue;
            }
        }
        gemm_epilogue<T, EPI, BM, BN, 2, 2>(p, acc, smem_raw, m0, n0, wm, wn, wave, lane, split, nsplit);
    }
}

// Deterministic split-K reduction: out[m][n] = sum_z ws[z][m][n] in z order.
// The first M/4 threads also add the per-split row sums (bias gradients).
template <typename T>
__device__ __forceinline__ void splitk_reduce_body(size_t i4, const float* ws, int splits, int M, int N,
                                                   const EpiArgs& ea, const float* rs_part, T* rs_out) {
    const size_t MN = (size_t)M * N;
    if (rs_out && i4 < (size_t)M) {
        float r[4] = {0, 0, 0, 0};
        for (int z = 0; z < splits; ++z) {
            float t[4];
            Vec4<float>::load(rs_part + (size_t)z * M + i4, t);
#pragma unroll
            for (int i = 0; i < 4; ++i) r[i] += t[i];
        }
        Vec4<T>::store(rs_out + i4, r);
    }
    if (i4 >= MN) return;
    // the partials are read once and the weight gradient is next read by the
    // caller's optimizer: non-temporal both ways
    float v[4] = {0, 0, 0, 0};
    for (int z = 0; z < splits; ++z) {
        float t[4];
        load4f_nt(ws + z * MN + i4, t);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] += t[i];
    }
    const int m = (int)(i4 / N), n = (int)(i4 - (size_t)m * N);
    const size_t off = (size_t)m * ea.ldo + n;
    if (ea.out_f32) store4_nt<float>((float*)ea.out + off, v);
    else store4_nt<T>((T*)ea.out + off, v);
}

template <typename T>
__global__ void splitk_reduce_kernel(const float* ws, int splits, int M, int N, EpiArgs ea, const float* rs_part,
                                     T* rs_out) {
    splitk_reduce_body<T>(((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4, ws, splits, M, N, ea, rs_part, rs_out);
}

// The reductions of a weight-gradient pair in one launch (a launch of this
// size costs about its own fixed overhead): blocks below `blocks0` reduce the
// first GEMM, the rest the second.
struct ReduceJob {
    const float* ws;
    int M, N;
    EpiArgs ea;
    const float* rs_part;
    void* rs_out;
};
struct ColsumJobs {
    ColsumJob j[kMaxColsumJobs];
    int n;
    int blocks;  // workgroups per job: N / kColsumCols (rounded up) of the widest job
};
// The first cs.n * cs.blocks workgroups each sum kColsumCols columns of one
// column-sum job (first, so that their latency-bound loads overlap the
// reduction); then blocks0 workgroups reduce problem a and the rest problem b.
template <typename T>
__global__ __launch_bounds__(256) void splitk_reduce_pair_kernel(ReduceJob a, ReduceJob b, int splits,
                                                                 unsigned blocks0, ColsumJobs cs) {
    const unsigned extra = (unsigned)(cs.n * cs.blocks);
    if (blockIdx.x < extra) {
        __shared__ float red[256 / kColsumCols][kColsumCols + 1];
        const int job = (int)(blockIdx.x / (unsigned)cs.blocks), n0 = (int)(blockIdx.x % (unsigned)cs.blocks) * kColsumCols;
        const ColsumJob& c = cs.j[job];
        if (n0 < c.N) colsum_block<T>(c.part, c.P, c.N, reinterpret_cast<T*>(c.out), n0, red);  // block-uniform
        return;
    }
    const unsigned bid = blockIdx.x - extra;
    const bool second = bid >= blocks0;
    const ReduceJob& j = second ? b : a;
    const size_t i4 = ((size_t)(bid - (second ? blocks0 : 0u)) * blockDim.x + threadIdx.x) * 4;
    splitk_reduce_body<T>(i4, j.ws, splits, j.M, j.N, j.ea, j.rs_part, reinterpret_cast<T*>(j.rs_out));
}

// Relaxed-determinism pairs: zero the outputs the k-splits add into (regions
// of 16-byte multiples), then the column sums riding along, in one launch
// before the grouped weight-gradient launch.
struct ZeroJobs {
    void* p[4];
    size_t n16[4];  // 16-byte units
    int n;
};
template <typename T>
__global__ __launch_bounds__(256) void zero_colsum_kernel(ZeroJobs z, unsigned zero_blocks, ColsumJobs cs) {
    if (blockIdx.x < zero_blocks) {
        const size_t stride = (size_t)zero_blocks * 256;
        for (int r = 0; r < z.n; ++r) {
            uint4* q = reinterpret_cast<uint4*>(z.p[r]);
            for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < z.n16[r]; i += stride)
                q[i] = make_uint4(0u, 0u, 0u, 0u);
        }
        return;
    }
    __shared__ float red[256 / kColsumCols][kColsumCols + 1];
    const unsigned bid = blockIdx.x - zero_blocks;
    const int job = (int)(bid / (unsigned)cs.blocks), n0 = (int)(bid % (unsigned)cs.blocks) * kColsumCols;
    const ColsumJob& c = cs.j[job];
    if (n0 < c.N) colsum_block<T>(c.part, c.P, c.N, reinterpret_cast<T*>(c.out), n0, red);  // block-uniform
}

// ------------------------------------------------------------------ SIMT path
template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_simt_kernel(GemmParams p, int a_kmajor, int b_kmajor) {
    constexpr int TB = 64, TK = 16;
    __shared__ float As[TK][TB + 1];
    __shared__ float Bs[TK][TB + 1];
    const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
    const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
    const T* A = (const T*)p.A;
    const T* B = (const T*)p.B;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < p.K; k0 += TK) {
        for (int e = tid; e < TB * TK; e += 256) {
            const int r = e / TK, kk = e % TK;  // r: row in tile, kk: k in tile
            const int m = m0 + r, n = n0 + r, k = k0 + kk;
            float av = 0.f, bv = 0.f;
            if (m < p.M && k < p.K) av = to_f(a_kmajor ? A[(size_t)m * p.lda + k] : A[(size_t)k * p.lda + m]);
            if (n < p.N && k < p.K) bv = to_f(b_kmajor ? B[(size_t)n * p.ldb + k] : B[(size_t)k * p.ldb + n]);
            As[kk][r] = av;
            Bs[kk][r] = bv;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
    const int n = n0 + tx * 4;
    if (n >= p.N) return;  // N % 4 == 0: a 4-group is wholly in or out
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = m0 + ty + 16 * i;
        if (m < p.M) epilogue4<T, EPI>(p.ea, m, n, acc[i]);
    }
}

// ------------------------------------------------------------------ dispatch
struct TileCfg {
    int BM, BN;
};

static bool mfma_ok(const GemmDesc& g, int BM, int BN) {
    return g.M % BM == 0 && g.N % BN == 0 && g.K % KT == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0;
}

// Split-K count for a weight-gradient GEMM whose tile grid is too small to
// fill 256 CUs; 1 otherwise.
static int splitk_for(const GemmDesc& g, int BM, int BN) {
    if (g.epi != EPI_STORE || g.splitk_ws == nullptr) return 1;
    const int tiles = (g.M / BM) * (g.N / BN);
    const int ksteps = g.K / KT;
    int s = 1;
    while (tiles * s < 256 && s * 2 <= ksteps / 8 && ksteps % (s * 2) == 0) s *= 2;
    if ((size_t)s * g.M * g.N + (size_t)s * g.M > g.splitk_ws_elems) s = 1;
    return s;
}

static TileCfg pick_tiles(const GemmDesc& g) {
    // largest tile whose grid still yields >= 256 workgroups, else 128x128;
    // a weight gradient with at least 64 tiles of 256x256 takes them and
    // fills the chip with a split-K of at most 4 (smaller ones measured
    // faster on 128x128 tiles)
    const TileCfg cands[] = {{256, 256}, {256, 128}, {128, 128}};
    if (!g.a_kmajor && !g.b_kmajor && g.epi == EPI_STORE && g.splitk_ws && mfma_ok(g, 256, 256) &&
        (g.M / 256) * (g.N / 256) >= 64)
        return {256, 256};
    // Projections (QKV head split, bias + dropout + residual) and input
    // gradients (store, head split, residual add): 256x192 tiles when their
    // whole waves of 256 finish sooner than those of 256x128 tiles (a 256x192
    // tile is 1.5 times the work) -- widths in multiples of 768 (768 = 4 x
    // 192, a 1.5-wave grid on 256x128 tiles)
    const bool fwd192 = (g.epi == EPI_QKV || g.epi == EPI_BIAS_DROP_RES) && g.b_kmajor;
    const bool dgrad192 = (g.epi == EPI_STORE || g.epi == EPI_HEADSPLIT || g.epi == EPI_ADD_RES) && !g.b_kmajor;
    if ((fwd192 || dgrad192) && g.a_kmajor && mfma_ok(g, 256, 192) && mfma_ok(g, 256, 128)) {
        const int w192 = ((g.M / 256) * (g.N / 192) + 255) / 256;
        const int w128 = ((g.M / 256) * (g.N / 128) + 255) / 256;
        if (3 * w192 < 2 * w128) return {256, 192};
    }
    for (const TileCfg& c : cands) {
        if (!mfma_ok(g, c.BM, c.BN)) continue;
        const int tiles = (g.M / c.BM) * (g.N / c.BN);
        if (c.BM == 256 && c.BN == 256 && tiles >= 256 && tiles % 256 != 0 && mfma_ok(g, 256, 128)) {
            // one workgroup per CU: a partly filled last wave of 256x256
            // tiles idles CUs; half-width tiles (about 12 % slower per flop)
            // take over when their whole waves finish clearly sooner
            const int w256 = (tiles + 255) / 256, w128 = (2 * tiles + 255) / 256;
            if (w128 * 1.12 < 0.9 * 2 * w256) return {256, 128};
        }
        if (tiles >= 256 || (c.BM == 128 && c.BN == 128)) return c;
    }
    return {0, 0};
}

template <typename Kern>
static hipError_t set_lds(Kern k, size_t bytes) {
    return hipFuncSetAttribute(reinterpret_cast<const void*>(k), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int BM, int BN, int WGM, int WGN>
constexpr size_t epilogue_lds_bytes() {
    return (size_t)(WGM * WGN) * 32 * (BN / WGN + 4) * 4;  // every wave: 32 rows x (WN + 4) floats
}

template <typename T, int BM, int BN, int WGM, int WGN, bool AK, bool BKM, int EPI>
static hipError_t launch_dl(const GemmDesc& g, hipStream_t st, int splits) {
    float* rs_part = splits > 1 ? g.splitk_ws + (size_t)splits * g.M * g.N : nullptr;
    void* rsum = g.rowsum_out == nullptr || AK ? nullptr : (splits > 1 ? (void*)rs_part : g.rowsum_out);
    GemmParams p{g.A, g.B, g.lda, g.ldb, g.M, g.N, g.K, g.K / splits, g.ea, g.splitk_ws, rsum};
    auto kern = gemm_dl_kernel<T, BM, BN, WGM, WGN, AK, BKM, EPI>;
    size_t lds = (size_t)DNS * (BM + BN) * DKT * sizeof(T);
    lds = std::max(lds, epilogue_lds_bytes<BM, BN, WGM, WGN>());
    lds = std::max(lds, (size_t)WGM * WGN * 64 * 8 * 4);
    static int slots = 0;  // workgroups of this kernel resident on the whole device
    if (!slots) {
        hipError_t e = set_lds(kern, lds);
        if (e != hipSuccess) return e;
        int per_cu = 0, dev = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, WGM * WGN * 64, lds);
        if (e != hipSuccess) return e;
        e = hipGetDevice(&dev);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        slots = std::max(1, per_cu) * std::max(1, cus);
    }
    const int tiles = (g.M / BM) * (g.N / BN);
    // persistent grid: at most one resident wave of workgroups, a multiple of
    // the 8 XCDs so each workgroup's tiles stay on its XCD's range
    int gx = std::min(tiles, std::max(8, slots / splits / 8 * 8));
    dim3 grid(gx, 1, splits);
    hipLaunchKernelGGL(kern, grid, dim3(WGM * WGN * 64), lds, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const size_t n4 = (size_t)g.M * g.N / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                       (const float*)g.splitk_ws, splits, g.M, g.N, g.ea, rs_part,
                       rsum ? reinterpret_cast<T*>(g.rowsum_out) : (T*)nullptr);
    return hipGetLastError();
}

// Kernel parameters of one GEMM of a launch with `splits` k-splits whose
// partials (and per-split row sums) go to ws.
template <bool AK>
static GemmParams dl4_params(const GemmDesc& g, int splits, float* ws) {
    float* rs_part = splits > 1 ? ws + (size_t)splits * g.M * g.N : nullptr;
    void* rsum = g.rowsum_out == nullptr || AK ? nullptr : (splits > 1 ? (void*)rs_part : g.rowsum_out);
    // k tiles per split rounded up: the last split may be shorter
    const int kps = (g.K / QKT + splits - 1) / splits * QKT;
    return GemmParams{g.A, g.B, g.lda, g.ldb, g.M, g.N, g.K, kps, g.ea, ws, rsum};
}

// Resident workgroups of a dl4 instantiation on the device (0 on failure).
template <typename T, int BM, int BN, bool AK, bool BKM, int EPI>
static int dl4_slots(size_t lds) {
    static int slots = 0;
    if (!slots) {
        auto kern = gemm_dl4_kernel<T, BM, BN, AK, BKM, EPI>;
        if (set_lds(kern, lds) != hipSuccess) return 0;
        int per_cu = 0, dev = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess) return 0;
        if (hipGetDevice(&dev) != hipSuccess) return 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        slots = std::max(1, per_cu) * std::max(1, cus);
    }
    return slots;
}

template <int BM, int BN>
constexpr size_t dl4_lds_bytes(size_t esz) {
    return std::max(std::max((size_t)dl4_stages(BM, BN, (int)esz) * (BM + BN) * QKT * esz,
                             epilogue_lds_bytes<BM, BN, 2, 2>()),
                    (size_t)256 * 8 * 4);
}

// Deterministic reduction of one GEMM's split-K partials (and row sums).
template <typename T>
static hipError_t splitk_reduce(const GemmDesc& g, int splits, const float* ws, hipStream_t st) {
    const float* rs_part = ws + (size_t)splits * g.M * g.N;
    const bool rsum = g.rowsum_out != nullptr && !g.a_kmajor;
    const size_t n4 = (size_t)g.M * g.N / 4;
    hipLaunchKernelGGL(splitk_reduce_kernel<T>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st, ws, splits,
                       g.M, g.N, g.ea, rsum ? rs_part : nullptr, rsum ? reinterpret_cast<T*>(g.rowsum_out) : (T*)nullptr);
    return hipGetLastError();
}

template <typename T, int BM, int BN, bool AK, bool BKM, int EPI>
static hipError_t launch_dl4(const GemmDesc& g, hipStream_t st, int splits) {
    auto kern = gemm_dl4_kernel<T, BM, BN, AK, BKM, EPI>;
    const size_t lds = dl4_lds_bytes<BM, BN>(sizeof(T));
    const int slots = dl4_slots<T, BM, BN, AK, BKM, EPI>(lds);  // workgroups resident on the device
    if (!slots) return hipErrorInvalidConfiguration;
    GemmGroup G{};
    G.p[0] = G.p[1] = dl4_params<AK>(g, splits, g.splitk_ws);
    G.splits[0] = G.splits[1] = splits;
    G.units0 = G.units = (g.M / BM) * (g.N / BN) * splits;
    // persistent grid: at most one resident wave of workgroups, a multiple of
    // the 8 XCDs so each workgroup's tiles stay on its XCD's range
    const int gx = std::min(G.units, std::max(8, slots / 8 * 8));
    hipLaunchKernelGGL(kern, dim3(gx), dim3(256), lds, st, G);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    return splitk_reduce<T>(g, splits, g.splitk_ws, st);
}

// Two weight gradients in one launch (256x256 tiles, A and B m/n-major,
// plain store with fused row sums): the split count fills the chip with the
// tiles of both; partials of the second follow those of the first in ws.
// Split count of a pair on 256x256 tiles, one workgroup per CU.  Its cost is
// modelled as the waves of 256 units times the k tiles of the longest unit
// (the critical path), plus the split-K partials the reduction reads (one
// 256x256x64 k tile, ~2 us at the sustained rate, against ~0.7 ps per fp32
// partial element): the cheapest count in 1..8 wins.  Splits may be unequal
// (k tiles rounded up per split) so that shapes in multiples of 768 fill
// whole waves (BERT-Base: 72 tiles x 7 splits = 504 units); every split
// keeps at least 8 k tiles.  0: the pair does not fit.
static int group_splits(const GemmDesc& a, const GemmDesc& b) {
    auto ok = [](const GemmDesc& g) {
        return g.dtype != 0 && !g.a_kmajor && !g.b_kmajor && g.epi == EPI_STORE &&
               g.M % 256 == 0 && g.N % 256 == 0 && g.K % QKT == 0 && g.lda % 8 == 0 && g.ldb % 8 == 0;
    };
    if (!ok(a) || !ok(b) || a.dtype != b.dtype) return 0;
    const int tiles = (a.M / 256) * (a.N / 256) + (b.M / 256) * (b.N / 256);
    const double elems = (double)a.M * a.N + (double)b.M * b.N;
    auto splits_fit = [](int K, int s) {  // every split of K gets >= 8 k tiles
        const int kt = K / QKT, per = (kt + s - 1) / s;
        return per >= 8 && kt - (s - 1) * per >= 8;
    };
    int best = 0;
    double best_cost = 0.0;
    for (int s = 1; s <= 8; ++s) {
        if (!splits_fit(a.K, s) || !splits_fit(b.K, s)) continue;
        const int waves = (tiles * s + 255) / 256;
        const int per = (std::max(a.K, b.K) / QKT + s - 1) / s;
        const double cost = (double)waves * per + (s > 1 ? s * elems * 3.2e-7 : 0.0);
        if (!best || cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    // a pair that would leave over a quarter of the chip idle runs apart
    if (!best || (double)tiles * best / (((tiles * best + 255) / 256) * 256) < 0.75) return 0;
    return best;
}

size_t gemm_splitk_group_elems(const GemmDesc& a, const GemmDesc& b) {
    const int s = group_splits(a, b);
    if (s <= 1) return 0;
    return (size_t)s * ((size_t)a.M * a.N + a.M + (size_t)b.M * b.N + b.M);
}

bool gemm_group_ok(const GemmDesc& a, const GemmDesc& b) {
    const int s = group_splits(a, b);
    if (s == 0) return false;
    if (a.splitk_atomic != b.splitk_atomic) return false;
    if (a.splitk_atomic) {
        // packed adds need 4-byte aligned pairs and whole 16-byte outputs to zero
        auto ok = [](const GemmDesc& g) {
            return g.ea.ldo == g.N && ((uintptr_t)g.ea.out & 15) == 0 && (g.rowsum_out == nullptr ||
                   (((uintptr_t)g.rowsum_out & 15) == 0 && (g.M * 2) % 16 == 0));
        };
        return ok(a) && ok(b);
    }
    if (s > 1 && (a.splitk_ws == nullptr || gemm_splitk_group_elems(a, b) > a.splitk_ws_elems)) return false;
    return true;
}

template <typename T>
static hipError_t launch_group_tail(const GemmDesc& a, const GemmDesc& b, hipStream_t st, const ColsumJobs& cs,
                                    int splits, float* ws_a, float* ws_b);
template <typename T>
static hipError_t launch_dl4_group(const GemmDesc& a, const GemmDesc& b, hipStream_t st, const ColsumJobs& cs,
                                   const GroupEvents& ev) {
    auto mark = [&](hipEvent_t e) { return e ? hipEventRecord(e, st) : hipSuccess; };
    constexpr int BM = 256, BN = 256;
    const int splits = group_splits(a, b);
    auto kern = gemm_dl4_kernel<T, BM, BN, false, false, EPI_STORE>;
    const size_t lds = dl4_lds_bytes<BM, BN>(sizeof(T));
    const int slots = dl4_slots<T, BM, BN, false, false, EPI_STORE>(lds);
    if (!slots) return hipErrorInvalidConfiguration;
    float* ws_a = a.splitk_ws;
    float* ws_b = splits > 1 ? ws_a + (size_t)splits * ((size_t)a.M * a.N + a.M) : nullptr;
    GemmGroup G{};
    G.p[0] = dl4_params<false>(a, splits, ws_a);
    G.p[1] = dl4_params<false>(b, splits, ws_b);
    G.splits[0] = G.splits[1] = splits;
    G.units0 = (a.M / BM) * (a.N / BN) * splits;
    G.units = G.units0 + (b.M / BM) * (b.N / BN) * splits;
    const int gx = std::min(G.units, std::max(8, slots / 8 * 8));
    if (splits > 1 && a.splitk_atomic) {
        // the k-splits add into the zeroed outputs; the column sums ride with the zeroing
        G.atomic = 1;
        G.p[0].rsum_out = a.rowsum_out;
        G.p[1].rsum_out = b.rowsum_out;
        ZeroJobs z{};
        auto add = [&](void* ptr, size_t bytes) {
            if (ptr) {
                z.p[z.n] = ptr;
                z.n16[z.n++] = bytes / 16;
            }
        };
        add(a.ea.out, (size_t)a.M * a.N * sizeof(T));
        add(b.ea.out, (size_t)b.M * b.N * sizeof(T));
        add(a.rowsum_out, (size_t)a.M * sizeof(T));
        add(b.rowsum_out, (size_t)b.M * sizeof(T));
        const unsigned zb = 512;
        hipLaunchKernelGGL(zero_colsum_kernel<T>, dim3(zb + (unsigned)(cs.n * cs.blocks)), dim3(256), 0, st, z, zb, cs);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        if ((e = mark(ev.gemm_start)) != hipSuccess) return e;
        hipLaunchKernelGGL(kern, dim3(gx), dim3(256), lds, st, G);
        if ((e = hipGetLastError()) != hipSuccess || (e = mark(ev.gemm_stop)) != hipSuccess) return e;
        if ((e = mark(ev.red_start)) != hipSuccess) return e;
        return mark(ev.red_stop);
    }
    hipError_t e = mark(ev.gemm_start);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(gx), dim3(256), lds, st, G);
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(ev.gemm_stop)) != hipSuccess) return e;
    if ((e = mark(ev.red_start)) != hipSuccess) return e;
    e = launch_group_tail<T>(a, b, st, cs, splits, ws_a, ws_b);
    if (e != hipSuccess) return e;
    return mark(ev.red_stop);
}

// The launch after a grouped GEMM: the split-K reduction of both problems
// with the column sums riding along, the column sums alone, or nothing.
template <typename T>
static hipError_t launch_group_tail(const GemmDesc& a, const GemmDesc& b, hipStream_t st, const ColsumJobs& cs,
                                    int splits, float* ws_a, float* ws_b) {
    if (splits == 1 && cs.n == 0) return hipSuccess;
    const unsigned extra = (unsigned)(cs.n * cs.blocks);
    if (splits == 1) {  // no partials to reduce: the column sums alone
        hipLaunchKernelGGL(splitk_reduce_pair_kernel<T>, dim3(extra), dim3(256), 0, st, ReduceJob{}, ReduceJob{}, 1,
                           0u, cs);
        return hipGetLastError();
    }
    auto job = [&](const GemmDesc& g, const float* ws) {
        const bool rsum = g.rowsum_out != nullptr;  // fused row sums (A is m-major here)
        return ReduceJob{ws, g.M, g.N, g.ea, rsum ? ws + (size_t)splits * g.M * g.N : nullptr,
                         rsum ? g.rowsum_out : nullptr};
    };
    const unsigned blocks0 = (unsigned)(((size_t)a.M * a.N / 4 + 255) / 256);
    const unsigned blocks1 = (unsigned)(((size_t)b.M * b.N / 4 + 255) / 256);
    hipLaunchKernelGGL(splitk_reduce_pair_kernel<T>, dim3(extra + blocks0 + blocks1), dim3(256), 0, st, job(a, ws_a),
                       job(b, ws_b), splits, blocks0, cs);
    return hipGetLastError();
}

hipError_t gemm_launch_group(const GemmDesc& a, const GemmDesc& b, hipStream_t st, const ColsumJob* colsums,
                             int n_colsums, const GroupEvents* events) {
    const GroupEvents ev = events ? *events : GroupEvents{};
    if (!gemm_group_ok(a, b) || n_colsums < 0 || n_colsums > kMaxColsumJobs || (n_colsums && !colsums))
        return hipErrorInvalidValue;
    ColsumJobs cs{};
    cs.n = n_colsums;
    for (int i = 0; i < n_colsums; ++i) {
        const ColsumJob& c = colsums[i];
        if (!c.part || !c.out || c.P <= 0 || c.N <= 0) return hipErrorInvalidValue;
        cs.j[i] = c;
        cs.blocks = std::max(cs.blocks, (c.N + kColsumCols - 1) / kColsumCols);
    }
    switch (a.dtype) {
        case 1: return launch_dl4_group<f16>(a, b, st, cs, ev);
        case 2: return launch_dl4_group<bf16>(a, b, st, cs, ev);
    }
    return hipErrorInvalidValue;
}

// Tiles run the four-wave kernel (2 x 2 waves of BM/2 x BN/2, 64-deep k
// tiles), except under the GELU forward epilogue and the short-k dropout
// epilogue, whose VALU work hides better with two waves per SIMD: the
// eight-wave kernel in a 2 x 4 grid of 128x64 wave tiles (256x256), a 4 x 2
// grid of 64x64 (256x128), or the four-wave 2 x 2 grid of 64x64 with 32-deep
// k tiles (128x128).
#ifndef GEMM_W256N
#define GEMM_W256N 2
#endif
constexpr int W256N = GEMM_W256N;
constexpr int W128M = 4;
template <typename T, int EPI, bool AK, bool BKM>
static hipError_t dispatch_tiles(const GemmDesc& g, hipStream_t st, TileCfg c) {
    // operands stream straight from global memory into LDS
    if (c.BM == 256 && c.BN == 256) {
        // the GELU epilogue's VALU work runs better with two waves per SIMD
        if constexpr (W256N == 2 && EPI != EPI_BIAS_GELU)
            return launch_dl4<T, 256, 256, AK, BKM, EPI>(g, st, splitk_for(g, 256, 256));
        else
            return launch_dl<T, 256, 256, 2, 4, AK, BKM, EPI>(g, st, splitk_for(g, 256, 256));
    }
    if (c.BM == 256 && c.BN == 192) {
        if constexpr ((EPI == EPI_QKV || EPI == EPI_BIAS_DROP_RES) && AK && BKM)
            return launch_dl4<T, 256, 192, AK, BKM, EPI>(g, st, 1);
        if constexpr ((EPI == EPI_STORE || EPI == EPI_HEADSPLIT || EPI == EPI_ADD_RES) && AK && !BKM)
            return launch_dl4<T, 256, 192, AK, BKM, EPI>(g, st, 1);
        return hipErrorNotSupported;
    }
    if (c.BM == 256 && c.BN == 128) {
        // the dropout epilogue's Philox work, like GELU's, favours two waves
        // per SIMD unless the k loop is long enough to dominate
        if constexpr (EPI != EPI_BIAS_GELU) {
            if (EPI != EPI_BIAS_DROP_RES || g.K >= 2048)
                return launch_dl4<T, 256, 128, AK, BKM, EPI>(g, st, splitk_for(g, 256, 128));
        }
        return launch_dl<T, 256, 128, W128M, 2, AK, BKM, EPI>(g, st, splitk_for(g, 256, 128));
    }
    if constexpr (EPI != EPI_BIAS_GELU) {
        if (EPI != EPI_BIAS_DROP_RES || g.K >= 2048)
            return launch_dl4<T, 128, 128, AK, BKM, EPI>(g, st, splitk_for(g, 128, 128));
    }
    return launch_dl<T, 128, 128, 2, 2, AK, BKM, EPI>(g, st, splitk_for(g, 128, 128));
}

// Operand layouts the layer uses with each epilogue: projections (A, B
// k-major) end in QKV / bias+dropout+residual / bias+GELU; input gradients
// (B n-major) in GELU' / store / head split / residual add; weight gradients
// (A m-major, B n-major) in store.  Other combinations take the SIMT path.
template <int EPI, bool AK, bool BKM>
constexpr bool mfma_combo() {
    if (AK && BKM) return EPI == EPI_QKV || EPI == EPI_BIAS_DROP_RES || EPI == EPI_BIAS_GELU || EPI == EPI_STORE;
    if (AK && !BKM)
        return EPI == EPI_GELU_BWD || EPI == EPI_MUL_AUX || EPI == EPI_STORE || EPI == EPI_HEADSPLIT ||
               EPI == EPI_ADD_RES;
    if (!AK && !BKM) return EPI == EPI_STORE;
    return false;
}

template <typename T, int EPI>
static hipError_t dispatch_mfma(const GemmDesc& g, hipStream_t st, TileCfg c) {
    if (g.a_kmajor && g.b_kmajor) {
        if constexpr (mfma_combo<EPI, true, true>()) return dispatch_tiles<T, EPI, true, true>(g, st, c);
    } else if (g.a_kmajor && !g.b_kmajor) {
        if constexpr (mfma_combo<EPI, true, false>()) return dispatch_tiles<T, EPI, true, false>(g, st, c);
    } else if (!g.a_kmajor && !g.b_kmajor) {
        if constexpr (mfma_combo<EPI, false, false>()) return dispatch_tiles<T, EPI, false, false>(g, st, c);
    }
    return hipErrorNotSupported;
}

template <typename T, int EPI>
static hipError_t launch_simt(const GemmDesc& g, hipStream_t st) {
    GemmParams p{g.A, g.B, g.lda, g.ldb, g.M, g.N, g.K, g.K, g.ea, nullptr, nullptr};
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64);
    hipLaunchKernelGGL((gemm_simt_kernel<T, EPI>), grid, dim3(256), 0, st, p, (int)g.a_kmajor, (int)g.b_kmajor);
    return hipGetLastError();
}

template <typename T, int EPI>
static hipError_t dispatch_epi(const GemmDesc& g, hipStream_t st, bool force_simt) {
    constexpr bool lowp = !std::is_same<T, float>::value;
    if constexpr (lowp) {
        if (!force_simt) {
            TileCfg c = pick_tiles(g);
            if (c.BM) {
                const hipError_t e = dispatch_mfma<T, EPI>(g, st, c);
                if (e != hipErrorNotSupported) return e;
            }
        }
    }
    return launch_simt<T, EPI>(g, st);
}

template <typename T>
static hipError_t dispatch_type(const GemmDesc& g, hipStream_t st, bool force_simt) {
    switch (g.epi) {
        case EPI_STORE: return dispatch_epi<T, EPI_STORE>(g, st, force_simt);
        case EPI_QKV: return dispatch_epi<T, EPI_QKV>(g, st, force_simt);
        case EPI_BIAS_DROP_RES: return dispatch_epi<T, EPI_BIAS_DROP_RES>(g, st, force_simt);
        case EPI_BIAS_GELU: return dispatch_epi<T, EPI_BIAS_GELU>(g, st, force_simt);
        case EPI_GELU_BWD: return dispatch_epi<T, EPI_GELU_BWD>(g, st, force_simt);
        case EPI_HEADSPLIT: return dispatch_epi<T, EPI_HEADSPLIT>(g, st, force_simt);
        case EPI_ADD_RES: return dispatch_epi<T, EPI_ADD_RES>(g, st, force_simt);
        case EPI_MUL_AUX: return dispatch_epi<T, EPI_MUL_AUX>(g, st, force_simt);
    }
    return hipErrorInvalidValue;
}

hipError_t gemm_launch(const GemmDesc& g_in, hipStream_t st, bool force_simt) {
    if (g_in.M <= 0 || g_in.N <= 0 || g_in.K <= 0) return hipSuccess;
    GemmDesc g = g_in;
    if (g.epi == EPI_QKV || g.epi == EPI_HEADSPLIT) {
        // the scatters divide row and column indices (< 2^31) by S, H and d
        if (g.ea.S < 1 || g.ea.H < 1 || g.ea.d < 1) return hipErrorInvalidValue;
        g.ea.fS = FastDiv((uint32_t)g.ea.S);
        g.ea.fH = FastDiv((uint32_t)g.ea.H);
        g.ea.fd = FastDiv((uint32_t)g.ea.d);
    }
    switch (g.dtype) {
        case 0: return dispatch_type<float>(g, st, true);
        case 1: return dispatch_type<f16>(g, st, force_simt);
        case 2: return dispatch_type<bf16>(g, st, force_simt);
    }
    return hipErrorInvalidValue;
}

size_t gemm_splitk_elems(const GemmDesc& g) {
    if (g.dtype == 0) return 0;
    // decide tiles and splits exactly as a launch with a workspace will
    GemmDesc h = g;
    h.splitk_ws = reinterpret_cast<float*>(16);
    h.splitk_ws_elems = (size_t)-1;
    TileCfg c = pick_tiles(h);
    if (!c.BM) return 0;
    const int s = splitk_for(h, c.BM, c.BN);
    return s > 1 ? (size_t)s * g.M * g.N + (size_t)s * g.M : 0;
}

bool gemm_rowsum_fused(const GemmDesc& g) {
    if (g.dtype == 0 || g.a_kmajor || g.b_kmajor || g.epi != EPI_STORE) return false;
    return pick_tiles(g).BM != 0;
}

}  // namespace tel
