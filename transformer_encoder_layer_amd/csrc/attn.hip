// attn.hip -- scaled, key-masked softmax attention with dropout on the
// probabilities, forward and backward, for gfx950.
//
// Definition (deployment article, attention pseudo-code; AI-infra blog
// section 5.1 for the 1/sqrt(d) scale and inverted dropout):
//   s_ij = q_i . k_j / sqrt(d) for keys j < len[b], -inf otherwise
//   P_ij = softmax_j(s_ij);  O_i = sum_j P_ij * keep_ij / (1-p) * v_j
// The softmax normaliser runs over all valid keys before dropout.
//
// MFMA path (d = 64, S % 64 == 0): one workgroup = 4 waves x 32 queries
// of one (batch, head); keys stream through LDS in blocks of 64 with an
// online (running max / running sum) softmax, so only the per-row
// log-sum-exp is written -- never the S x S matrix.  Scores are produced
// transposed (keys x queries) so that each lane owns one query and four
// consecutive keys: the row max/sum needs one cross-lane exchange, and the
// two lanes of a query split the Philox calls (8 keys each) of every 32-key
// keep word and swap the results.  The probability
// tile feeds the P.V product straight from registers; V is read with the
// transposing LDS load using the same key permutation.
//
// Backward: a query-parallel kernel computes D_i = rowsum(dO_i * O_i) and
// dQ; a key-parallel kernel computes dK and dV (no atomics: every output
// row is owned by one wave).  Both recompute P from Q, K and the saved
// log-sum-exp, and regenerate the dropout bits from the counter-based RNG:
// at these lengths the forward keeps no per-score state at all.  For
// S <= 128 one workgroup does the whole backward of a (batch, head); its
// dropout bits come from the 1-bit-per-score mask the forward packed (one
// 32-bit word per query and 32 keys, B*N*S*S/8 bytes), or, when the caller
// chose not to keep it (attention-dropout checkpointing), from the RNG
// again -- the same bits either way.  The forward kernels write their keep
// words to a.bits whenever it is set (the S <= 128 mask, or a test's copy).
//
// SIMT path: one thread per row, any S and d in {16, 32, 64, 128}.
#include "attn.h"
#include "mfma_common.h"

namespace tel {

static constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bool keep1(const Rng& r, uint64_t e, uint32_t thr) {
    return (keep4(r, e >> 2, thr) >> (e & 3)) & 1u;
}

// Keep word of the 32 keys of one query row starting at element e0 (a
// multiple of 32), computed by the two lanes l and l^32 that share the row:
// each evaluates two of the four 8-key Philox blocks and they swap results.
// Bit j of the word is key j.  Every lane of the wave must call it.
__device__ __forceinline__ uint32_t keep_word32(const Rng& r, uint64_t e0, uint32_t thr, int lane) {
    const int hh = lane >> 5;
    const uint32_t m0 = keep8(r, (e0 >> 3) + hh, thr);      // block hh
    const uint32_t m1 = keep8(r, (e0 >> 3) + 2 + hh, thr);  // block 2 + hh
    const uint32_t o0 = __shfl_xor(m0, 32, 64), o1 = __shfl_xor(m1, 32, 64);
    const uint32_t b0 = hh ? o0 : m0, b1 = hh ? m0 : o0, b2 = hh ? o1 : m1, b3 = hh ? m1 : o1;
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// Row of token t in ctx / dqkv: t itself, or its packed row (-1: padding).
__device__ __forceinline__ int out_row(const AttnArgs& a, int t) { return a.packed ? a.packed[t] : t; }

// ------------------------------------------------------------------ MFMA fwd
// One workgroup = 4 waves x 32 queries of one (batch, head); 64-key blocks
// of K and V flow through two LDS buffers, the next block fetched into
// registers before the MFMAs of the current one (one barrier per block).
template <typename T>
__global__ __launch_bounds__(256, 2) void attn_fwd_mfma(AttnArgs a) {
    constexpr int D = 64, KB = 64, VLD = D + 32;  // V rows 192 B apart: conflict-free transposing reads
    typedef typename MfmaOp<T>::v8 v8;
    __shared__ __align__(16) T Ks[2][KB * D];
    __shared__ __align__(16) T Vs[2][KB * VLD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = a.S, NH = a.NH, B = a.B;
    const int q0 = blockIdx.x * 128 + wave * 32;
    const bool active = q0 < S;
    const int L = a.len ? a.len[b] : S;
    const int nkb = (L + KB - 1) / KB;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const float c = kLog2e * 0.125f;  // log2(e) / sqrt(64)
    const int ql = q0 + (lane & 31);
    const int qlc = ql < S ? ql : 0;

    v8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const v8*>(Q + (size_t)qlc * D + ks * 16 + (lane >> 5) * 8);
    float m_run = -INFINITY, l_run = 0.0f;
    f32x16 o[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = 0.0f;
    const uint64_t rowbase = ((uint64_t)(b * NH + h) * S + qlc) * (uint64_t)S;

    const int row0 = tid >> 3, row1 = row0 + 32, ch = tid & 7;
    uint4 pk0, pk1, pv0, pv1;
    auto fetch = [&](int kb) {
        pk0 = *reinterpret_cast<const uint4*>(K + (size_t)(kb * KB + row0) * D + ch * 8);
        pk1 = *reinterpret_cast<const uint4*>(K + (size_t)(kb * KB + row1) * D + ch * 8);
        pv0 = *reinterpret_cast<const uint4*>(V + (size_t)(kb * KB + row0) * D + ch * 8);
        pv1 = *reinterpret_cast<const uint4*>(V + (size_t)(kb * KB + row1) * D + ch * 8);
    };
    if (nkb > 0) fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        *reinterpret_cast<uint4*>(&Ks[buf][kmaj_off(row0, ch * 8)]) = pk0;
        *reinterpret_cast<uint4*>(&Ks[buf][kmaj_off(row1, ch * 8)]) = pk1;
        *reinterpret_cast<uint4*>(&Vs[buf][row0 * VLD + ch * 8]) = pv0;
        *reinterpret_cast<uint4*>(&Vs[buf][row1 * VLD + ch * 8]) = pv1;
        __syncthreads();
        if (kb + 1 < nkb) fetch(kb + 1);
        if (active) {
            f32x16 s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) s[kt] = MfmaOp<T>::mma(frag_kmaj<T>(Ks[buf], kt * 32, ks, lane), qf[ks], s[kt]);
            }
            // s[kt][r]: raw score q.k of key kb*64 + kt*32 + 8*(r>>2) +
            // 4*(lane>>5) + (r&3) and query ql; keys at or beyond L only
            // occur in the last block
            if (kb * KB + KB > L) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = kb * KB + kt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                        if (key >= L) s[kt][r] = -INFINITY;
                    }
            }
            float mloc = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kt][r]);
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
            // Lazy rescaling: the reference maximum m_run (raw units) moves
            // only when a block's maximum exceeds it by more than 8 / c, so
            // the unnormalised probabilities stay <= 2^8 and O and l are
            // rescaled only on those (rare, after the first block) blocks.
            // The result is the same softmax up to rounding: l and O share
            // the reference, and the log-sum-exp is m_run * c + log2(l).
            if (__any(mloc > m_run + 8.0f / c)) {
                const float m_new = mloc > m_run + 8.0f / c ? mloc : m_run;
                const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);  // 0 on the first block
                m_run = m_new;
                l_run *= alpha;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                    for (int r = 0; r < 16; ++r) o[ct][r] *= alpha;
            }
            const float mc = m_run * c;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(__fmaf_rn(s[kt][r], c, -mc));
                    s[kt][r] = p;
                    l_run += p;
                }
            if (a.drop.thr) {
#pragma unroll
                for (int kt = 0; kt < 2; ++kt) {
                    // keep bits of keys kb*64 + kt*32 + 0..31; this lane's
                    // keys 8g + 4*(lane>>5) + i are bits 8g + i of kbits
                    const uint32_t word = keep_word32(a.drop.rng, rowbase + kb * KB + kt * 32, a.drop.thr, lane);
                    if (a.bits && lane < 32) a.bits[(rowbase >> 5) + kb * 2 + kt] = word;
                    const uint32_t kbits = word >> ((lane >> 5) * 4);
#pragma unroll
                    for (int g = 0; g < 4; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // all ones if the bit is set, else zero (written
                            // out: the compiler turns the C form into a
                            // compare and a select)
                            uint32_t m;
                            asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(kbits), "s"(g * 8 + i));
                            s[kt][g * 4 + i] = __uint_as_float(__float_as_uint(s[kt][g * 4 + i]) & m);
                        }
                }
            }
#pragma unroll
            for (int ks2 = 0; ks2 < 4; ++ks2) {
                const int kt = ks2 >> 1, half = ks2 & 1;
                v8 pf;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pf[i] = from_f<T>(s[kt][(2 * half) * 4 + i]);
                    pf[4 + i] = from_f<T>(s[kt][(2 * half + 1) * 4 + i]);
                }
                const int kb0 = kt * 32 + (2 * half) * 8 + (lane >> 5) * 4;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    o[ct] = MfmaOp<T>::mma(frag_tr<T>(Vs[buf], VLD, ct * 32, kb0, kb0 + 8, lane), pf, o[ct]);
            }
        }
    }
    if (active) {
        const float l = l_run + __shfl_xor(l_run, 32, 64);
        const float inv = a.drop.scale / l;
        const int orow = out_row(a, b * S + ql);
        T* out = (T*)a.ctx + (size_t)max(orow, 0) * (NH * D) + h * D;
        if (orow >= 0) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = o[ct][g * 4 + i] * inv;
                    Vec4<T>::store(out + ct * 32 + g * 8 + (lane >> 5) * 4, v);
                }
        }
        if (lane < 32) a.lse[(size_t)(b * NH + h) * S + ql] = m_run * c + log2f(l);
    }
}

// ------------------------------------------------------------------ MFMA fwd, S <= 128
// When all S <= 128 keys of a (batch, head) fit in LDS, one workgroup loads
// K and V once (every load issued together) and each wave scores its 32
// queries against all keys at once: the softmax is a plain two-pass one
// (exact row maximum, then exp2 and sum), with no online rescaling.
template <typename T>
__global__ __launch_bounds__(256, 2) void attn_fwd_short_mfma(AttnArgs a) {
    constexpr int D = 64, SMAX = 128, VLD = D + 32;
    typedef typename MfmaOp<T>::v8 v8;
    __shared__ __align__(16) T Ks[SMAX * D];
    __shared__ __align__(16) T Vs[SMAX * VLD];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = a.S, NH = a.NH, B = a.B;
    const int L = a.len ? a.len[b] : S;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const float c = kLog2e * 0.125f;  // log2(e) / sqrt(64)

    constexpr int CPT = SMAX * 8 / 256;
    uint4 ck[CPT], cv[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cidx = tid + i * 256, row = cidx >> 3, ch = cidx & 7;
        const size_t g = (size_t)(row < S ? row : 0) * D + ch * 8;
        ck[i] = *reinterpret_cast<const uint4*>(K + g);
        cv[i] = *reinterpret_cast<const uint4*>(V + g);
    }
    const int q0 = wave * 32;
    const bool active = q0 < S;
    const int ql = q0 + (lane & 31);
    const int qlc = ql < S ? ql : 0;
    v8 qf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = *reinterpret_cast<const v8*>(Q + (size_t)qlc * D + ks * 16 + (lane >> 5) * 8);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {  // rows S .. SMAX-1 are never read
        const int cidx = tid + i * 256, row = cidx >> 3, ch = cidx & 7;
        *reinterpret_cast<uint4*>(Ks + kmaj_off(row, ch * 8)) = ck[i];
        *reinterpret_cast<uint4*>(Vs + row * VLD + ch * 8) = cv[i];
    }
    __syncthreads();
    if (!active) return;

    f32x16 s[SMAX / 32];
    float m = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < SMAX / 32; ++kt) {
        if (kt * 32 < S) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[kt][r] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) s[kt] = MfmaOp<T>::mma(frag_kmaj<T>(Ks, kt * 32, ks, lane), qf[ks], s[kt]);
            // s[kt][r]: raw score of key kt*32 + 8*(r>>2) + 4*(lane>>5) + (r&3)
            // and query ql; only a tile reaching L holds masked keys
            if (kt * 32 + 32 > L) {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (kt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) >= L) s[kt][r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) m = fmaxf(m, s[kt][r]);
        }
    }
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    const float mc = m * c;  // row maximum in log2 units
    float l = 0.0f;
#pragma unroll
    for (int kt = 0; kt < SMAX / 32; ++kt) {
        if (kt * 32 < S) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = __builtin_amdgcn_exp2f(__fmaf_rn(s[kt][r], c, -mc));
                s[kt][r] = p;
                l += p;
            }
        }
    }
    l += __shfl_xor(l, 32, 64);
    const uint64_t rowbase = ((uint64_t)(b * NH + h) * S + ql) * (uint64_t)S;
    if (a.drop.thr) {
#pragma unroll
        for (int kt = 0; kt < SMAX / 32; ++kt) {
            if (kt * 32 < S) {
                // keep bits of keys kt*32 + 0..31
                const uint32_t word = keep_word32(a.drop.rng, rowbase + kt * 32, a.drop.thr, lane);
                const uint32_t kbits = word >> ((lane >> 5) * 4);  // key 8g + 4*(lane>>5) + i -> bit 8g + i
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        uint32_t mk;  // all ones if kept, else zero
                        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(mk) : "v"(kbits), "s"(g * 8 + i));
                        s[kt][g * 4 + i] = __uint_as_float(__float_as_uint(s[kt][g * 4 + i]) & mk);
                    }
                if (a.bits && lane < 32) a.bits[(rowbase >> 5) + kt] = word;
            }
        }
    }
    f32x16 o[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[ct][r] = 0.0f;
#pragma unroll
    for (int kt = 0; kt < SMAX / 32; ++kt) {
        if (kt * 32 < S) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                v8 pf;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pf[i] = from_f<T>(s[kt][(2 * half) * 4 + i]);
                    pf[4 + i] = from_f<T>(s[kt][(2 * half + 1) * 4 + i]);
                }
                const int kb0 = kt * 32 + (2 * half) * 8 + (lane >> 5) * 4;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct)
                    o[ct] = MfmaOp<T>::mma(frag_tr<T>(Vs, VLD, ct * 32, kb0, kb0 + 8, lane), pf, o[ct]);
            }
        }
    }
    const float inv = a.drop.scale / l;
    const int orow = out_row(a, b * S + ql);
    T* out = (T*)a.ctx + (size_t)max(orow, 0) * (NH * D) + h * D;
    if (orow >= 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = o[ct][g * 4 + i] * inv;
                Vec4<T>::store(out + ct * 32 + g * 8 + (lane >> 5) * 4, v);
            }
    }
    if (lane < 32) a.lse[(size_t)(b * NH + h) * S + ql] = mc + log2f(l);
}

// ------------------------------------------------------------------ MFMA bwd: D and dQ
// Query-parallel: wave w of workgroup x owns queries 128x + 32w .. +31 and
// walks the 64-key blocks below len[b].  K and V blocks flow through two LDS
// buffers, the next block (and this lane's two keep words of it) fetched into
// registers before the MFMAs of the current one, one barrier per block.
template <typename T>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_mfma(AttnArgs a) {
    constexpr int D = 64, KB = 64;
    typedef typename MfmaOp<T>::v8 v8;
    __shared__ __align__(16) T Ks[2][KB * D];
    __shared__ __align__(16) T Vs[2][KB * D];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = a.S, NH = a.NH, B = a.B, H = NH * D;
    const int q0 = blockIdx.x * 128 + wave * 32;
    const bool active = q0 < S;
    const int L = a.len ? a.len[b] : S;
    const int nkb = (L + KB - 1) / KB;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const T* dO = (const T*)a.dout + ((size_t)b * NH + h) * head;
    const float c = kLog2e * 0.125f;
    const int ql = q0 + (lane & 31);
    const int qlc = ql < S ? ql : 0;

    v8 qf[4], df[4];
    float Dq, lse2;
    {
        const int orow = out_row(a, b * S + qlc);  // padding (packed rows): dO is zero there
        const T* O = (const T*)a.ctx + (size_t)max(orow, 0) * H + h * D;
        float part = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int off = ks * 16 + (lane >> 5) * 8;
            qf[ks] = *reinterpret_cast<const v8*>(Q + (size_t)qlc * D + off);
            df[ks] = *reinterpret_cast<const v8*>(dO + (size_t)qlc * D + off);
            const v8 ov = *reinterpret_cast<const v8*>(O + off);
#pragma unroll
            for (int i = 0; i < 8; ++i) part += to_f(df[ks][i]) * to_f(ov[i]);
        }
        Dq = part + __shfl_xor(part, 32, 64);
        lse2 = a.lse[(size_t)(b * NH + h) * S + qlc];
        if (active && lane < 32) a.dvec[(size_t)(b * NH + h) * S + ql] = Dq;
    }
    f32x16 dq[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) dq[ct][r] = 0.0f;
    const uint64_t rowbase = ((uint64_t)(b * NH + h) * S + qlc) * (uint64_t)S;

    const int row0 = tid >> 3, row1 = row0 + 32, ch = tid & 7;
    uint4 pk0, pk1, pv0, pv1;
    auto fetch = [&](int kb) {
        pk0 = *reinterpret_cast<const uint4*>(K + (size_t)(kb * KB + row0) * D + ch * 8);
        pk1 = *reinterpret_cast<const uint4*>(K + (size_t)(kb * KB + row1) * D + ch * 8);
        pv0 = *reinterpret_cast<const uint4*>(V + (size_t)(kb * KB + row0) * D + ch * 8);
        pv1 = *reinterpret_cast<const uint4*>(V + (size_t)(kb * KB + row1) * D + ch * 8);
    };
    if (nkb > 0) fetch(0);
    for (int kb = 0; kb < nkb; ++kb) {
        const int buf = kb & 1;
        *reinterpret_cast<uint4*>(&Ks[buf][kmaj_off(row0, ch * 8)]) = pk0;
        *reinterpret_cast<uint4*>(&Ks[buf][kmaj_off(row1, ch * 8)]) = pk1;
        *reinterpret_cast<uint4*>(&Vs[buf][kmaj_off(row0, ch * 8)]) = pv0;
        *reinterpret_cast<uint4*>(&Vs[buf][kmaj_off(row1, ch * 8)]) = pv1;
        __syncthreads();
        if (kb + 1 < nkb) fetch(kb + 1);
        if (active) {
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                f32x16 sc, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) { sc[r] = 0.0f; dp[r] = 0.0f; }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    sc = MfmaOp<T>::mma(frag_kmaj<T>(Ks[buf], kt * 32, ks, lane), qf[ks], sc);
                    dp = MfmaOp<T>::mma(frag_kmaj<T>(Vs[buf], kt * 32, ks, lane), df[ks], dp);
                }
                // sc[r]: key kb*64 + kt*32 + 8*(r>>2) + 4*(lane>>5) + (r&3), query ql;
                // keys at or beyond L only occur in the last block
                if (kb * KB + KB > L) {
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (kb * KB + kt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3) >= L) sc[r] = -INFINITY;
                }
                // keep bits regenerated from the counter-based RNG (the
                // forward kept none for sequences this long)
                uint32_t word = 0xFFFFFFFFu;
                if (a.drop.thr) word = keep_word32(a.drop.rng, rowbase + kb * KB + kt * 32, a.drop.thr, lane);
                const uint32_t kbits = word >> ((lane >> 5) * 4);  // key 8g + 4*(lane>>5) + i -> bit 8g + i
                const uint32_t scale_bits = __float_as_uint(a.drop.scale);
#pragma unroll
                for (int g = 0; g < 4; ++g)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = g * 4 + i;
                        const float p = __builtin_amdgcn_exp2f(__fmaf_rn(sc[r], c, -lse2));
                        // dropout factor: 1/(1-p) if kept, else 0
                        uint32_t m;
                        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(kbits), "s"(g * 8 + i));
                        const float f = __uint_as_float(m & scale_bits);
                        sc[r] = p * __fmaf_rn(dp[r], f, -Dq);
                    }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    v8 pf;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pf[i] = from_f<T>(sc[(2 * half) * 4 + i]);
                        pf[4 + i] = from_f<T>(sc[(2 * half + 1) * 4 + i]);
                    }
                    const int kb0 = kt * 32 + (2 * half) * 8 + (lane >> 5) * 4;
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct)
                        dq[ct] = MfmaOp<T>::mma(frag_tr_kmaj<T>(Ks[buf], ct * 32, kb0, kb0 + 8, lane), pf, dq[ct]);
                }
            }
        }
    }
    const int drow = out_row(a, b * S + qlc);
    if (active && drow >= 0) {
        T* out = (T*)a.dqkv + (size_t)drow * (3 * H) + h * D;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = dq[ct][g * 4 + i] * 0.125f;
                Vec4<T>::store(out + ct * 32 + g * 8 + (lane >> 5) * 4, v);
            }
    }
}

// ------------------------------------------------------------------ MFMA bwd: dK, dV
// Key-parallel: wave w of workgroup x owns keys 128x + 32w .. +31 and walks
// every 64-query block.  The blocks flow through two LDS buffers: the
// global loads of block qb+1 (Q, dO, log-sum-exp, D and the keep words) are
// issued into registers before the MFMAs of block qb, so one barrier per
// block suffices and the load latency hides behind the compute.  Keep words
// are always staged: regenerated per 32 keys with one Philox call per 8
// keys, or all ones without dropout.
template <typename T>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_mfma(AttnArgs a) {
    constexpr int D = 64, QB = 64;
    typedef typename MfmaOp<T>::v8 v8;
    __shared__ __align__(16) T Qs[2][QB * D];
    __shared__ __align__(16) T Os[2][QB * D];
    __shared__ __align__(16) float lse_s[2][QB], D_s[2][QB];
    __shared__ __align__(16) uint32_t bits_s[2][4][QB];  // keep words [32-key word][query] of this block's 128 keys
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = a.S, NH = a.NH, B = a.B, H = NH * D;
    const int key0 = blockIdx.x * 128 + wave * 32;
    const bool active = key0 < S;
    const int L = a.len ? a.len[b] : S;
    const bool live = active && key0 < L;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const T* dO = (const T*)a.dout + ((size_t)b * NH + h) * head;
    const float* lse = a.lse + (size_t)(b * NH + h) * S;
    const float* Dv = a.dvec + (size_t)(b * NH + h) * S;
    const float c = kLog2e * 0.125f;
    const int kl = key0 + (lane & 31);
    const int klc = kl < S ? kl : 0;
    const uint64_t bhbase = (uint64_t)(b * NH + h) * S;
    const int NW32 = S / 32;

    v8 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int off = ks * 16 + (lane >> 5) * 8;
        kf[ks] = *reinterpret_cast<const v8*>(K + (size_t)klc * D + off);
        vf[ks] = *reinterpret_cast<const v8*>(V + (size_t)klc * D + off);
    }
    f32x16 dk[2], dv[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[ct][r] = 0.0f; dv[ct][r] = 0.0f; }

    // per-thread share of one block: 2 chunks of Q and of dO, one of the
    // log-sum-exp / D values, one keep word (query tid/4, key word tid%4)
    uint4 pq0, pq1, po0, po1;
    float pld = 0.0f;
    const int wq = tid >> 2, ww = tid & 3;
    const int kwi = blockIdx.x * 4 + ww;  // 32-key word index of this thread's keep word
    const int row0 = tid >> 3, row1 = (tid + 256) >> 3, ch = tid & 7;
    auto fetch = [&](int qb) {
        pq0 = *reinterpret_cast<const uint4*>(Q + (size_t)(qb * QB + row0) * D + ch * 8);
        pq1 = *reinterpret_cast<const uint4*>(Q + (size_t)(qb * QB + row1) * D + ch * 8);
        po0 = *reinterpret_cast<const uint4*>(dO + (size_t)(qb * QB + row0) * D + ch * 8);
        po1 = *reinterpret_cast<const uint4*>(dO + (size_t)(qb * QB + row1) * D + ch * 8);
        if (tid < QB) pld = lse[qb * QB + tid];
        else if (tid < 2 * QB) pld = Dv[qb * QB + tid - QB];
    };
    auto stage = [&](int qb, int buf) {
        *reinterpret_cast<uint4*>(&Qs[buf][kmaj_off(row0, ch * 8)]) = pq0;
        *reinterpret_cast<uint4*>(&Qs[buf][kmaj_off(row1, ch * 8)]) = pq1;
        *reinterpret_cast<uint4*>(&Os[buf][kmaj_off(row0, ch * 8)]) = po0;
        *reinterpret_cast<uint4*>(&Os[buf][kmaj_off(row1, ch * 8)]) = po1;
        if (tid < QB) lse_s[buf][tid] = pld;
        else if (tid < 2 * QB) D_s[buf][tid - QB] = pld;
        uint32_t word = 0xFFFFFFFFu;
        if (a.drop.thr && kwi < NW32) {
            const uint64_t e0 = (bhbase + qb * QB + wq) * (uint64_t)S + kwi * 32;
            word = 0;
#pragma unroll
            for (int g = 0; g < 4; ++g) word |= keep8_cmp(a.drop.rng, (e0 >> 3) + g, a.drop.thr) << (8 * g);
        }
        bits_s[buf][ww][wq] = word;
    };

    const int nqb = S / QB;
    fetch(0);
    for (int qb = 0; qb < nqb; ++qb) {
        const int buf = qb & 1;
        stage(qb, buf);
        __syncthreads();
        if (qb + 1 < nqb) fetch(qb + 1);
        if (live) {
            // one 32-query tile at a time keeps only its scores and dP live
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
                f32x16 sc, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) { sc[r] = 0.0f; dp[r] = 0.0f; }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    sc = MfmaOp<T>::mma(frag_kmaj<T>(Qs[buf], qt * 32, ks, lane), kf[ks], sc);
                    dp = MfmaOp<T>::mma(frag_kmaj<T>(Os[buf], qt * 32, ks, lane), vf[ks], dp);
                }
                // sc[r]: query qb*64 + qt*32 + 8*(r>>2) + 4*(lane>>5) + (r&3), key kl.
                // Keys at or beyond L are not masked here: a lane's P and dS
                // only reach its own key's rows of dK and dV, which are
                // written as zero instead.
                const uint32_t scale_bits = __float_as_uint(a.drop.scale);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int qi0 = qt * 32 + 8 * g + 4 * (lane >> 5);
                    const float4 l4 = *reinterpret_cast<const float4*>(&lse_s[buf][qi0]);
                    const float4 d4 = *reinterpret_cast<const float4*>(&D_s[buf][qi0]);
                    const uint4 w4 = *reinterpret_cast<const uint4*>(&bits_s[buf][wave][qi0]);
                    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
                    const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = g * 4 + i;
                        const float p = __builtin_amdgcn_exp2f(__fmaf_rn(sc[r], c, -lv[i]));
                        // dropout factor: 1/(1-p) if key kl of this query is kept, else 0
                        uint32_t m;
                        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(wv[i]), "v"(kl & 31));
                        const float f = __uint_as_float(m & scale_bits);
                        const float dsv = p * __fmaf_rn(dp[r], f, -dvv[i]);
                        sc[r] = p * f;
                        dp[r] = dsv;
                    }
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    v8 pf, sf;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pf[i] = from_f<T>(sc[(2 * half) * 4 + i]);
                        pf[4 + i] = from_f<T>(sc[(2 * half + 1) * 4 + i]);
                        sf[i] = from_f<T>(dp[(2 * half) * 4 + i]);
                        sf[4 + i] = from_f<T>(dp[(2 * half + 1) * 4 + i]);
                    }
                    const int qb0 = qt * 32 + (2 * half) * 8 + (lane >> 5) * 4;
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        dv[ct] = MfmaOp<T>::mma(frag_tr_kmaj<T>(Os[buf], ct * 32, qb0, qb0 + 8, lane), pf, dv[ct]);
                        dk[ct] = MfmaOp<T>::mma(frag_tr_kmaj<T>(Qs[buf], ct * 32, qb0, qb0 + 8, lane), sf, dk[ct]);
                    }
                }
            }
        }
    }
    const int krow = active ? out_row(a, b * S + kl) : -1;
    if (krow >= 0) {
        T* outk = (T*)a.dqkv + (size_t)krow * (3 * H) + H + h * D;
        T* outv = outk + H;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                float vk[4], vv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // keys at or beyond L get no gradient
                    vk[i] = kl < L ? dk[ct][g * 4 + i] * 0.125f : 0.0f;
                    vv[i] = kl < L ? dv[ct][g * 4 + i] : 0.0f;
                }
                const int col = ct * 32 + g * 8 + (lane >> 5) * 4;
                Vec4<T>::store(outk + col, vk);
                Vec4<T>::store(outv + col, vv);
            }
    }
}

// ------------------------------------------------------------------ MFMA bwd, S <= 128
// The whole backward of one (batch, head) in one workgroup when S <= 128:
// Q, dO and K fit in LDS, P is recomputed once, and no intermediate leaves
// the chip.
//   load:    Q, dO, K -> LDS; D_i = rowsum(dO_i * O_i), the log-sum-exp and
//            the dropout keep words (stored bits, or regenerated) -> LDS.
//   phase 1: wave w owns keys 32w .. 32w+31 (lane = key, register = query,
//            as in the key-parallel kernel): S and dP for every query, then
//            dV += P~^T dO and dK += dS^T Q accumulate in registers.
//   phase 2: dS goes to LDS as [query][key] over the then-dead Q/dO tiles,
//            and wave w computes dQ = dS K for queries 32w .. 32w+31.
// Element (q, key) of the dS tile sits at q*S + ((key/8) ^ (q mod C))*8 +
// key mod 8 (C = S/8 chunks of 16 bytes per row), so the 16 rows a 16-lane
// group reads hit 16 distinct 16-byte bank groups.
template <typename T>
__global__ __launch_bounds__(256, 2) void attn_bwd_short_mfma(AttnArgs a) {
    constexpr int D = 64, SMAX = 128;
    typedef typename MfmaOp<T>::v8 v8;
    __shared__ __align__(16) T lds[3 * SMAX * D];  // Q | dO | K; dS [S][S] overlays Q and dO
    __shared__ __align__(16) float lse_s[SMAX], D_s[SMAX];
    __shared__ __align__(16) uint32_t bits_s[SMAX / 32][SMAX];  // keep words [32-key word][query]
    T* Qs = lds;
    T* dOs = lds + SMAX * D;
    T* Ks = lds + 2 * SMAX * D;
    T* dSs = lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = blockIdx.z, h = blockIdx.y;
    const int S = a.S, NH = a.NH, B = a.B, H = NH * D;
    const int L = a.len ? a.len[b] : S;
    const size_t head = (size_t)S * D;
    const size_t bh = (size_t)b * NH + h;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const T* dO = (const T*)a.dout + bh * head;
    const float c = kLog2e * 0.125f;
    const int NW32 = S / 32;       // 32-key words per query row
    const int CMASK = S / 8 - 1;   // dS row chunks - 1

    // ---- load: every global read of this phase is issued before the first
    // use (fixed-count loops; slots past S read row 0 and are not stored)
    constexpr int CPT = SMAX * 8 / 256;  // 16-byte chunks per thread and tensor
    uint4 cq[CPT], cdo[CPT], ck[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cidx = tid + i * 256, row = cidx >> 3, ch = cidx & 7;
        const size_t g = (size_t)(row < S ? row : 0) * D + ch * 8;
        cq[i] = *reinterpret_cast<const uint4*>(Q + g);
        cdo[i] = *reinterpret_cast<const uint4*>(dO + g);
        ck[i] = *reinterpret_cast<const uint4*>(K + g);
    }
    // D_q: two threads per query row, 32 columns each
    const int dq_row = tid >> 1, dq_half = tid & 1;
    const int dq_q = dq_row < S ? dq_row : 0;
    v8 ov[4], dv8[4];
    {
        const T* orow = (const T*)a.ctx + (size_t)max(out_row(a, b * S + dq_q), 0) * H + h * D + dq_half * 32;
        const T* drow = dO + (size_t)dq_q * D + dq_half * 32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ov[j] = *reinterpret_cast<const v8*>(orow + j * 8);
            dv8[j] = *reinterpret_cast<const v8*>(drow + j * 8);
        }
    }
    const float lse_v = a.lse[bh * S + dq_q];
    // keep words: S * S/32 <= 512 per workgroup, two per thread
    uint32_t kw[2] = {0u, 0u};
    const bool stored_bits = a.drop.thr && a.bits;
    if (stored_bits) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int cidx = tid + i * 256;
            kw[i] = a.bits[bh * S * NW32 + (cidx < S * NW32 ? cidx : 0)];
        }
    }
    // this wave's key and value rows as MFMA operands
    const int kw0 = wave * 32;
    const bool active = kw0 < S;
    const int kl = kw0 + (lane & 31);
    const int klc = kl < S ? kl : 0;
    v8 kf[4], vf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const int off = ks * 16 + (lane >> 5) * 8;
        kf[ks] = *reinterpret_cast<const v8*>(K + (size_t)klc * D + off);
        vf[ks] = *reinterpret_cast<const v8*>(V + (size_t)klc * D + off);
    }
    // (rows S .. SMAX-1 of the tiles are never read; storing them
    // unconditionally keeps the loads above from being sunk into branches)
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int cidx = tid + i * 256, row = cidx >> 3, ch = cidx & 7;
        *reinterpret_cast<uint4*>(Qs + kmaj_off(row, ch * 8)) = cq[i];
        *reinterpret_cast<uint4*>(dOs + kmaj_off(row, ch * 8)) = cdo[i];
        *reinterpret_cast<uint4*>(Ks + kmaj_off(row, ch * 8)) = ck[i];
    }
    {
        float part = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 8; ++i) part += to_f(dv8[j][i]) * to_f(ov[j][i]);
        part += __shfl_xor(part, 1, 64);
        if (dq_row < S && dq_half == 0) {
            D_s[dq_row] = part;
            lse_s[dq_row] = lse_v;
        }
    }
    {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int cidx = tid + i * 256;
            if (cidx < S * NW32) {
                const int q = cidx / NW32, w = cidx - q * NW32;
                uint32_t word = a.drop.thr ? kw[i] : 0xFFFFFFFFu;  // no dropout: keep all
                if (a.drop.thr && !stored_bits) {
                    const uint64_t e0 = (bh * S + q) * (uint64_t)S + w * 32;  // element of key w*32
                    word = 0;
#pragma unroll
                    for (int g = 0; g < 4; ++g) word |= keep8(a.drop.rng, (e0 >> 3) + g, a.drop.thr) << (8 * g);
                }
                bits_s[w][q] = word;
            }
        }
    }
    __syncthreads();

    // ---- phase 1: keys of this wave
    f32x16 dk[2], dv[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 16; ++r) { dk[ct][r] = 0.0f; dv[ct][r] = 0.0f; }
    v8 dsf[SMAX / 32][2];  // dS of each 32-query tile as MFMA operands, kept for phase 2
    if (active) {
#pragma unroll
        for (int qt = 0; qt < SMAX / 32; ++qt) {
            if (qt * 32 < S) {
                f32x16 sc, dp;
#pragma unroll
                for (int r = 0; r < 16; ++r) { sc[r] = 0.0f; dp[r] = 0.0f; }
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    sc = MfmaOp<T>::mma(frag_kmaj<T>(Qs, qt * 32, ks, lane), kf[ks], sc);
                    dp = MfmaOp<T>::mma(frag_kmaj<T>(dOs, qt * 32, ks, lane), vf[ks], dp);
                }
                // sc[r]: query qt*32 + 8*(r>>2) + 4*(lane>>5) + (r&3), key kl.
                // A key at or beyond L is not masked per element: its dS
                // operands are zeroed below (phase 2 reads them for dQ) and
                // its rows of dK and dV are written as zero.
                f32x16 ds;
                const uint32_t scale_bits = __float_as_uint(a.drop.scale);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int qi0 = qt * 32 + 8 * g + 4 * (lane >> 5);
                    const float4 l4 = *reinterpret_cast<const float4*>(&lse_s[qi0]);
                    const float4 d4 = *reinterpret_cast<const float4*>(&D_s[qi0]);
                    const uint4 w4 = *reinterpret_cast<const uint4*>(&bits_s[wave][qi0]);
                    const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
                    const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int r = g * 4 + i;
                        const float p = __builtin_amdgcn_exp2f(__fmaf_rn(sc[r], c, -lv[i]));
                        uint32_t mk;  // all ones if key kl of this query is kept, else zero
                        asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(mk) : "v"(wv[i]), "v"(kl & 31));
                        const float f = __uint_as_float(mk & scale_bits);
                        ds[r] = p * __fmaf_rn(dp[r], f, -dvv[i]);
                        sc[r] = p * f;
                    }
                }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    v8 pf, sf;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pf[i] = from_f<T>(sc[(2 * half) * 4 + i]);
                        pf[4 + i] = from_f<T>(sc[(2 * half + 1) * 4 + i]);
                        sf[i] = from_f<T>(ds[(2 * half) * 4 + i]);
                        sf[4 + i] = from_f<T>(ds[(2 * half + 1) * 4 + i]);
                    }
                    const int qb0 = qt * 32 + (2 * half) * 8 + (lane >> 5) * 4;
#pragma unroll
                    for (int ct = 0; ct < 2; ++ct) {
                        dv[ct] = MfmaOp<T>::mma(frag_tr_kmaj<T>(dOs, ct * 32, qb0, qb0 + 8, lane), pf, dv[ct]);
                        dk[ct] = MfmaOp<T>::mma(frag_tr_kmaj<T>(Qs, ct * 32, qb0, qb0 + 8, lane), sf, dk[ct]);
                    }
                    if (kl >= L) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) sf[e] = from_f<T>(0.0f);
                    }
                    dsf[qt][half] = sf;
                }
            }
        }
    }
    __syncthreads();  // every wave is done with Q and dO
    if (active) {
        // dsf[qt][half] element i (< 4): query qt*32 + 16*half + 4*(lane>>5) + i,
        // element 4 + i: the same + 8; key kl
#pragma unroll
        for (int qt = 0; qt < SMAX / 32; ++qt) {
            if (qt * 32 < S) {
#pragma unroll
                for (int half = 0; half < 2; ++half)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int q = qt * 32 + 16 * half + 4 * (lane >> 5) + (e & 3) + (e >> 2) * 8;
                        dSs[q * S + ((((kl >> 3) ^ (q & CMASK))) << 3) + (kl & 7)] = dsf[qt][half][e];
                    }
            }
        }
        const int krow = out_row(a, b * S + kl);
        T* outk = (T*)a.dqkv + (size_t)max(krow, 0) * (3 * H) + H + h * D;
        T* outv = outk + H;
        if (krow >= 0) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float vk[4], vv[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // keys at or beyond L get no gradient
                        vk[i] = kl < L ? dk[ct][g * 4 + i] * 0.125f : 0.0f;
                        vv[i] = kl < L ? dv[ct][g * 4 + i] : 0.0f;
                    }
                    const int col = ct * 32 + g * 8 + (lane >> 5) * 4;
                    Vec4<T>::store(outk + col, vk);
                    Vec4<T>::store(outv + col, vv);
                }
        }
    }
    __syncthreads();

    // ---- phase 2: dQ of queries 32w .. 32w+31
    if (active) {
        const int q = kw0 + (lane & 31);
        f32x16 dq[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int r = 0; r < 16; ++r) dq[ct][r] = 0.0f;
        for (int kb = 0; kb < S; kb += 16) {
            const int r0 = kb + 8 * (lane >> 5);
            const v8 bf = *reinterpret_cast<const v8*>(dSs + q * S + (((r0 >> 3) ^ (q & CMASK)) << 3));
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
                dq[ct] = MfmaOp<T>::mma(frag_tr_kmaj<T>(Ks, ct * 32, r0, r0 + 4, lane), bf, dq[ct]);
        }
        const int qrow = out_row(a, b * S + q);
        T* out = (T*)a.dqkv + (size_t)max(qrow, 0) * (3 * H) + h * D;
        if (qrow >= 0) {
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = dq[ct][g * 4 + i] * 0.125f;
                    Vec4<T>::store(out + ct * 32 + g * 8 + (lane >> 5) * 4, v);
                }
        }
    }
}

// ------------------------------------------------------------------ SIMT
template <typename T, int D>
__global__ __launch_bounds__(128) void attn_fwd_simt(AttnArgs a) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int S = a.S, NH = a.NH, B = a.B, H = NH * D;
    if (idx >= B * NH * S) return;
    const int q = idx % S, bh = idx / S, b = bh / NH, h = bh % NH;
    const int L = a.len ? a.len[b] : S;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const float c = kLog2e / sqrtf((float)D);
    float qv[D], o[D];
#pragma unroll
    for (int i = 0; i < D; ++i) { qv[i] = to_f(Q[(size_t)q * D + i]); o[i] = 0.0f; }
    float m = -INFINITY, l = 0.0f;
    const uint64_t rowbase = ((uint64_t)bh * S + q) * (uint64_t)S;
    for (int j = 0; j < L; ++j) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) s += qv[i] * to_f(K[(size_t)j * D + i]);
        s *= c;
        const float mn = fmaxf(m, s);
        const float alpha = exp2f(m - mn), p = exp2f(s - mn);
        l = l * alpha + p;
        m = mn;
        const float pk = (a.drop.thr && !keep1(a.drop.rng, rowbase + j, a.drop.thr)) ? 0.0f : p;
#pragma unroll
        for (int i = 0; i < D; ++i) o[i] = o[i] * alpha + pk * to_f(V[(size_t)j * D + i]);
    }
    T* out = (T*)a.ctx + (size_t)(b * S + q) * H + h * D;
    const float inv = a.drop.scale / l;
#pragma unroll
    for (int i = 0; i < D; ++i) out[i] = from_f<T>(o[i] * inv);
    a.lse[idx] = m + log2f(l);
}

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_bwd_dq_simt(AttnArgs a) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int S = a.S, NH = a.NH, B = a.B, H = NH * D;
    if (idx >= B * NH * S) return;
    const int q = idx % S, bh = idx / S, b = bh / NH, h = bh % NH;
    const int L = a.len ? a.len[b] : S;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const T* dO = (const T*)a.dout + (size_t)bh * head;
    const T* O = (const T*)a.ctx + (size_t)(b * S + q) * H + h * D;
    const float c = kLog2e / sqrtf((float)D);
    float qv[D], dov[D], dq[D];
    float Dq = 0.0f;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        qv[i] = to_f(Q[(size_t)q * D + i]);
        dov[i] = to_f(dO[(size_t)q * D + i]);
        Dq += dov[i] * to_f(O[i]);
        dq[i] = 0.0f;
    }
    a.dvec[idx] = Dq;
    const float lse2 = a.lse[idx];
    const uint64_t rowbase = ((uint64_t)bh * S + q) * (uint64_t)S;
    for (int j = 0; j < L; ++j) {
        float s = 0.0f, dp = 0.0f;
#pragma unroll
        for (int i = 0; i < D; ++i) {
            s += qv[i] * to_f(K[(size_t)j * D + i]);
            dp += dov[i] * to_f(V[(size_t)j * D + i]);
        }
        const float p = exp2f(s * c - lse2);
        float f = 1.0f;
        if (a.drop.thr) f = keep1(a.drop.rng, rowbase + j, a.drop.thr) ? a.drop.scale : 0.0f;
        const float ds = p * (dp * f - Dq);
#pragma unroll
        for (int i = 0; i < D; ++i) dq[i] += ds * to_f(K[(size_t)j * D + i]);
    }
    const float sc = 1.0f / sqrtf((float)D);
    T* out = (T*)a.dqkv + (size_t)(b * S + q) * (3 * H) + h * D;
#pragma unroll
    for (int i = 0; i < D; ++i) out[i] = from_f<T>(dq[i] * sc);
}

template <typename T, int D>
__global__ __launch_bounds__(128) void attn_bwd_dkdv_simt(AttnArgs a) {
    const int idx = blockIdx.x * blockDim.x + threadIdx.x;
    const int S = a.S, NH = a.NH, B = a.B, H = NH * D;
    if (idx >= B * NH * S) return;
    const int j = idx % S, bh = idx / S, b = bh / NH, h = bh % NH;
    const int L = a.len ? a.len[b] : S;
    const size_t head = (size_t)S * D;
    const T* Q = (const T*)a.qkvh + ((size_t)(0 * B + b) * NH + h) * head;
    const T* K = (const T*)a.qkvh + ((size_t)(1 * B + b) * NH + h) * head;
    const T* V = (const T*)a.qkvh + ((size_t)(2 * B + b) * NH + h) * head;
    const T* dO = (const T*)a.dout + (size_t)bh * head;
    const float* lse = a.lse + (size_t)bh * S;
    const float* Dv = a.dvec + (size_t)bh * S;
    const float c = kLog2e / sqrtf((float)D);
    float kv[D], vv[D], dk[D], dv[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        kv[i] = to_f(K[(size_t)j * D + i]);
        vv[i] = to_f(V[(size_t)j * D + i]);
        dk[i] = 0.0f;
        dv[i] = 0.0f;
    }
    if (j < L) {
        for (int q = 0; q < S; ++q) {
            float s = 0.0f, dp = 0.0f;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                s += to_f(Q[(size_t)q * D + i]) * kv[i];
                dp += to_f(dO[(size_t)q * D + i]) * vv[i];
            }
            const float p = exp2f(s * c - lse[q]);
            float f = 1.0f;
            if (a.drop.thr) f = keep1(a.drop.rng, ((uint64_t)bh * S + q) * S + j, a.drop.thr) ? a.drop.scale : 0.0f;
            const float ds = p * (dp * f - Dv[q]);
#pragma unroll
            for (int i = 0; i < D; ++i) {
                dv[i] += p * f * to_f(dO[(size_t)q * D + i]);
                dk[i] += ds * to_f(Q[(size_t)q * D + i]);
            }
        }
    }
    const float sc = 1.0f / sqrtf((float)D);
    T* outk = (T*)a.dqkv + (size_t)(b * S + j) * (3 * H) + H + h * D;
    T* outv = outk + H;
#pragma unroll
    for (int i = 0; i < D; ++i) {
        outk[i] = from_f<T>(dk[i] * sc);
        outv[i] = from_f<T>(dv[i]);
    }
}

// ------------------------------------------------------------------ dispatch
static bool mfma_attn_ok(const AttnArgs& a) { return a.dtype != 0 && a.d == 64 && a.S % 64 == 0; }

template <typename T, int D>
static hipError_t simt_fwd(const AttnArgs& a0, hipStream_t st) {
    AttnArgs a = a0;
    a.bits = nullptr;  // the generic kernels regenerate the bits
    const int n = a.B * a.NH * a.S;
    hipLaunchKernelGGL((attn_fwd_simt<T, D>), dim3((n + 127) / 128), dim3(128), 0, st, a);
    return hipGetLastError();
}
template <typename T, int D>
static hipError_t simt_bwd(const AttnArgs& a0, hipStream_t st) {
    AttnArgs a = a0;
    a.bits = nullptr;
    const int n = a.B * a.NH * a.S;
    hipLaunchKernelGGL((attn_bwd_dq_simt<T, D>), dim3((n + 127) / 128), dim3(128), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dkdv_simt<T, D>), dim3((n + 127) / 128), dim3(128), 0, st, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t fwd_t(const AttnArgs& a, hipStream_t st, bool force_simt) {
    if constexpr (!std::is_same<T, float>::value) {
        if (!force_simt && mfma_attn_ok(a) && a.S <= 128) {
            hipLaunchKernelGGL(attn_fwd_short_mfma<T>, dim3(1, a.NH, a.B), dim3(256), 0, st, a);
            return hipGetLastError();
        }
        if (!force_simt && mfma_attn_ok(a)) {
            dim3 grid((a.S + 127) / 128, a.NH, a.B);
            hipLaunchKernelGGL(attn_fwd_mfma<T>, grid, dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
    if (a.packed) return hipErrorInvalidValue;  // packed rows: MFMA kernels only
    switch (a.d) {
        case 16: return simt_fwd<T, 16>(a, st);
        case 32: return simt_fwd<T, 32>(a, st);
        case 64: return simt_fwd<T, 64>(a, st);
        case 128: return simt_fwd<T, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t bwd_t(const AttnArgs& a, hipStream_t st, bool force_simt) {
    if constexpr (!std::is_same<T, float>::value) {
        if (!force_simt && mfma_attn_ok(a) && a.S <= 128) {
            hipLaunchKernelGGL(attn_bwd_short_mfma<T>, dim3(1, a.NH, a.B), dim3(256), 0, st, a);
            return hipGetLastError();
        }
        if (!force_simt && mfma_attn_ok(a)) {
            dim3 grid((a.S + 127) / 128, a.NH, a.B);
            hipLaunchKernelGGL(attn_bwd_dq_mfma<T>, grid, dim3(256), 0, st, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(attn_bwd_dkdv_mfma<T>, grid, dim3(256), 0, st, a);
            return hipGetLastError();
        }
    }
    if (a.packed) return hipErrorInvalidValue;  // packed rows: MFMA kernels only
    switch (a.d) {
        case 16: return simt_bwd<T, 16>(a, st);
        case 32: return simt_bwd<T, 32>(a, st);
        case 64: return simt_bwd<T, 64>(a, st);
        case 128: return simt_bwd<T, 128>(a, st);
    }
    return hipErrorInvalidValue;
}

hipError_t attn_forward(const AttnArgs& a, hipStream_t st, bool force_simt) {
    switch (a.dtype) {
        case 0: return fwd_t<float>(a, st, true);
        case 1: return fwd_t<f16>(a, st, force_simt);
        case 2: return fwd_t<bf16>(a, st, force_simt);
    }
    return hipErrorInvalidValue;
}

hipError_t attn_backward(const AttnArgs& a, hipStream_t st, bool force_simt) {
    switch (a.dtype) {
        case 0: return bwd_t<float>(a, st, true);
        case 1: return bwd_t<f16>(a, st, force_simt);
        case 2: return bwd_t<bf16>(a, st, force_simt);
    }
    return hipErrorInvalidValue;
}

}  // namespace tel
