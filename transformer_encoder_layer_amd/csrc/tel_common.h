// tel_common.h -- device-side helpers shared by the gfx950 kernels of the
// fused encoder layer: storage types, conversions, vector access, the
// counter-based dropout generator and the exact GELU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tel {

typedef _Float16 f16;
typedef __bf16 bf16;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- types
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ f16 from_f<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// round a float through storage type T and back (value the stored tensor holds)
template <typename T> __device__ __forceinline__ float round_through(float x) { return to_f(from_f<T>(x)); }

// 4 consecutive elements: load as float4, store from float4.
template <typename T> struct Vec4;
template <> struct Vec4<float> {
    static __device__ __forceinline__ void load(const float* p, float v[4]) {
        float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    static __device__ __forceinline__ void store(float* p, const float v[4]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <> struct Vec4<f16> {
    static __device__ __forceinline__ void load(const f16* p, float v[4]) {
        f16x4 q = *reinterpret_cast<const f16x4*>(p);
        v[0] = (float)q[0]; v[1] = (float)q[1]; v[2] = (float)q[2]; v[3] = (float)q[3];
    }
    static __device__ __forceinline__ void store(f16* p, const float v[4]) {
        f16x4 q = {(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        *reinterpret_cast<f16x4*>(p) = q;
    }
};
template <> struct Vec4<bf16> {
    static __device__ __forceinline__ void load(const bf16* p, float v[4]) {
        bf16x4 q = *reinterpret_cast<const bf16x4*>(p);
        v[0] = (float)q[0]; v[1] = (float)q[1]; v[2] = (float)q[2]; v[3] = (float)q[3];
    }
    static __device__ __forceinline__ void store(bf16* p, const float v[4]) {
        bf16x4 q = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        *reinterpret_cast<bf16x4*>(p) = q;
    }
};

// ---------------------------------------------------------------- RNG
// Philox4x32 with 10 rounds (Salmon et al., SC'11): per round the counter
// words 0 and 2 are multiplied by two odd constants; the high halves are
// mixed with the other two words and the key, and the key advances by two
// Weyl increments between rounds.
struct Rng {
    uint32_t key0, key1;  // seed mod 2^32, layer id
    uint32_t site, step;  // counter words 2 and 3
};

// a ^ b ^ k as one gfx950 three-input logic instruction (truth table 0x96:
// bit set iff an odd number of inputs are set).  k is read from a scalar
// register, so it must be wave-uniform -- the Philox key words are (seed,
// layer id) and their Weyl increments.
__device__ __forceinline__ uint32_t xor3_uniform(uint32_t a, uint32_t b, uint32_t k) {
    uint32_t r;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
    return r;
}

// k0 and k1 must be wave-uniform (see xor3_uniform).
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        // one 32 x 32 -> 64-bit product per multiplier (a single
        // v_mad_u64_u32) instead of separate low and high multiplies
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p2 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t a0 = (uint32_t)p0, b0 = (uint32_t)(p0 >> 32);
        const uint32_t a2 = (uint32_t)p2, b2 = (uint32_t)(p2 >> 32);
        uint32_t n0, n2;
        if (round == 0) {
            // counter words 1 and 3 (block high word, step) are often
            // uniform too: plain xors let their key mix stay scalar
            n0 = b2 ^ (c1 ^ k0);
            n2 = b0 ^ (c3 ^ k1);
        } else {
            n0 = xor3_uniform(b2, c1, k0);
            n2 = xor3_uniform(b0, c3, k1);
        }
        c0 = n0; c1 = a2; c2 = n2; c3 = a0;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return make_uint4(c0, c1, c2, c3);
}

// Dropout decisions: one Philox call (block g, counter (g low, g high,
// site, step), key (seed, layer)) serves the 8 elements 8g .. 8g+7; element
// e uses the 16-bit half (e mod 2) of word (e/2 mod 4) and is kept iff that
// value >= thr = floor(p * 2^16).
// Keep bits of the 8 elements of block g: bit j set iff element 8g+j is kept.
// Per 16-bit half of w: 1 if the half is below thr (element dropped), else
// 0 -- a saturating packed subtract thr - half (zero iff half >= thr)
// clamped to 1.  thr2 = thr in both halves, wave-uniform.
__device__ __forceinline__ uint32_t dropped2(uint32_t w, uint32_t thr2) {
    uint32_t d, r;
    asm("v_pk_sub_u16 %0, %1, %2 clamp" : "=v"(d) : "s"(thr2), "v"(w));
    asm("v_pk_min_u16 %0, %1, %2" : "=v"(r) : "v"(d), "s"(0x00010001u));
    return r;  // bit 0: low half, bit 16: high half
}
// Bits 0..7 of the keep mask from the four words' dropped2 results
// (element 2j at bit 2j of x, element 2j+1 at bit 2j+16).
__device__ __forceinline__ uint32_t keep_bits8(uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
    const uint32_t x = d0 | (d1 << 2) | (d2 << 4) | (d3 << 6);
    return ~(x | (x >> 15)) & 0xFFu;
}
__device__ __forceinline__ uint32_t keep8(const Rng& r, uint64_t g, uint32_t thr) {
    const uint4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), r.site, r.step, r.key0, r.key1);
    const uint32_t t2 = thr * 0x00010001u;
    return keep_bits8(dropped2(w.x, t2), dropped2(w.y, t2), dropped2(w.z, t2), dropped2(w.w, t2));
}
// The same bits as keep8 from per-half compares: more instructions, fewer
// registers live at once (for kernels at the edge of their register budget).
__device__ __forceinline__ uint32_t keep8_cmp(const Rng& r, uint64_t g, uint32_t thr) {
    const uint4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), r.site, r.step, r.key0, r.key1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
    uint32_t k = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) k |= (uint32_t)(((ws[j >> 1] >> (16 * (j & 1))) & 0xFFFFu) >= thr) << j;
    return k;
}
// Keep bits of the four elements 4q .. 4q+3 (half of block q/2): bit i set
// iff element 4q+i is kept.  Costs a whole Philox call; kernels that can
// use all 8 decisions of a block call keep8 instead.
__device__ __forceinline__ uint32_t keep4(const Rng& r, uint64_t q, uint32_t thr) {
    const uint64_t g = q >> 1;
    const uint4 w = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), r.site, r.step, r.key0, r.key1);
    const uint32_t a = (q & 1) ? w.z : w.x, b = (q & 1) ? w.w : w.y;
    const uint32_t t2 = thr * 0x00010001u;
    const uint32_t x = dropped2(a, t2) | (dropped2(b, t2) << 2);  // a: bits 0, 16; b: bits 2, 18
    return ~(x | (x >> 15)) & 0xFu;
}

// Dropout description passed to kernels: thr == 0 means "no dropout".
struct Drop {
    Rng rng;
    uint32_t thr;   // floor(p * 2^16)
    float scale;  // 1/(1-p) rounded to fp32
};

// ---------------------------------------------------------------- column sums
// out[n] = sum_p part[p][n] (fp32 [P][N] partial rows) for the 32 columns
// n0 .. n0+31, by one 256-thread block: thread (phase j = tid / 32, column
// tid % 32) adds rows j, j+8, ... in order, then the 8 phase sums are added
// in order -- a fixed summation order, independent of scheduling.  A wave's
// load covers two rows of 32 consecutive columns (whole 128-byte lines) and
// each thread keeps 8 loads in flight.  red: 8 x 33 floats of LDS; every
// thread of the block must call it.
constexpr int kColsumCols = 32;
template <typename T>
__device__ __forceinline__ void colsum_block(const float* part, int P, int N, T* out, int n0,
                                             float (*red)[kColsumCols + 1]) {
    const int cl = threadIdx.x & (kColsumCols - 1), ph = threadIdx.x / kColsumCols;
    const int n = n0 + cl;
    float s = 0.0f;
    if (n < N) {
        int p = ph;
        for (; p + 56 < P; p += 64) {
            float a[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a[i] = part[(size_t)(p + 8 * i) * N + n];
#pragma unroll
            for (int i = 0; i < 8; ++i) s += a[i];
        }
        for (; p < P; p += 8) s += part[(size_t)p * N + n];
    }
    red[ph][cl] = s;
    __syncthreads();
    if (ph == 0 && n < N) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < 256 / kColsumCols; ++j) t += red[j][cl];
        out[n] = from_f<T>(t);
    }
}

// ---------------------------------------------------------------- GELU
// Exact GELU u*Phi(u) and its derivative Phi(u) + u*phi(u) (AI-infra blog,
// section 2.3: the erf form, not the tanh approximation).  Phi comes from
// the complementary error function in the rational form of Abramowitz &
// Stegun, Handbook of Mathematical Functions, formula 7.1.26
// (|error| <= 1.5e-7 in erf), evaluated on |u|/sqrt(2) so that the left
// tail has no cancellation; phi shares the same exponential.  Every
// operation is explicitly rounded so that every epilogue that evaluates it
// (the FFN1 forward, the FFN2 input gradient under GELU checkpointing) gets
// the same bits: GELU(u) = u * cdf, GELU'(u) = cdf + u * pdf.
__device__ __forceinline__ void normal_cdf_pdf(float u, float& cdf, float& pdf) {
    const float x = __fmul_rn(fabsf(u), 0.70710678118654752f);
    const float t = __builtin_amdgcn_rcpf(__fmaf_rn(0.3275911f, x, 1.0f));
    const float e = __builtin_amdgcn_exp2f(__fmul_rn(__fmul_rn(u, u), -0.72134752044448170f));  // e^(-u^2/2)
    float poly = __fmaf_rn(1.061405429f, t, -1.453152027f);
    poly = __fmaf_rn(poly, t, 1.421413741f);
    poly = __fmaf_rn(poly, t, -0.284496736f);
    poly = __fmaf_rn(poly, t, 0.254829592f);
    poly = __fmul_rn(poly, t);
    const float half_erfc = __fmul_rn(__fmul_rn(0.5f, poly), e);
    cdf = u >= 0.0f ? __fadd_rn(1.0f, -half_erfc) : half_erfc;
    pdf = __fmul_rn(e, 0.39894228040143268f);
}

}  // namespace tel
