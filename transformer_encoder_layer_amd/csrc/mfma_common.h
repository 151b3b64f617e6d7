// mfma_common.h -- gfx950 MFMA operand helpers shared by the GEMM and the
// attention kernels.
//
// v_mfma_f32_32x32x16_{f16,bf16} lane layout (checked on the device):
//   operand A: lane l holds A[i = l & 31][k = 8*(l >> 5) .. +7]
//   operand B: lane l holds B[k = 8*(l >> 5) .. +7][j = l & 31]
//   result:    register r holds D[i = 8*(r >> 2) + 4*(l >> 5) + (r & 3)][j = l & 31]
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i reads
// 8 bytes at its own address; afterwards lane i holds element (i & 3) of
// the reads of lanes 4r + (i >> 2), r = 0..3.  When lane i addresses row
// kb + (i >> 2), column c0 + 4*(i & 3) of a row-major tile, lane i receives
// the column c0 + i of rows kb .. kb+3: a transposed fragment.
#pragma once
#include "tel_common.h"

namespace tel {

template <typename T> struct MfmaOp;
template <> struct MfmaOp<f16> {
    typedef f16x8 v8;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};
template <> struct MfmaOp<bf16> {
    typedef bf16x8 v8;
    static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};

// Element offset of (row, k) in a k-major LDS tile with 64 elements
// (128 bytes) per row whose 16-byte chunks are XOR-swizzled by row.  The
// gfx950 LDS serves 16 lanes x 16 bytes per cycle from 64 4-byte banks, so
// a 128-bit fragment read (16 consecutive rows, one chunk each) is
// conflict-free only if those 16 rows cover all 16 bank groups: even and odd
// rows already sit in different 128-byte halves, and the chunk is XORed with
// (row >> 1) & 7 to spread each half over its 8 groups.
__device__ __forceinline__ int kmaj_off(int row, int k) {
    return row * 64 + ((((k >> 3) ^ ((row >> 1) & 7))) << 3) + (k & 7);
}

// Operand fragment from a swizzled k-major tile [rows][64]: lane l gets
// row rb + (l & 31), k = 16*ks + 8*(l >> 5) .. +7 (one 128-bit LDS read).
template <typename T>
__device__ __forceinline__ typename MfmaOp<T>::v8 frag_kmaj(const T* lds, int rb, int ks, int lane) {
    typedef typename MfmaOp<T>::v8 v8;
    const int row = rb + (lane & 31);
    return *reinterpret_cast<const v8*>(lds + kmaj_off(row, ks * 16 + (lane >> 5) * 8));
}

__device__ __forceinline__ i16x4 ds_read_tr16(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 __attribute__((address_space(3)))*)(p));
}

template <typename T>
__device__ __forceinline__ typename MfmaOp<T>::v8 join8(i16x4 lo, i16x4 hi) {
    typedef short s8 __attribute__((ext_vector_type(8)));
    s8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return *reinterpret_cast<typename MfmaOp<T>::v8*>(&r);
}

// Operand fragment whose rows are the columns of a row-major LDS tile
// [k][ld] (padded rows): lane l gets column cb + (l & 31) at k rows
// k0 .. k0+3 (first half) and k1 .. k1+3 (second half), where k0/k1 are
// chosen per lane half by the caller.
template <typename T>
__device__ __forceinline__ typename MfmaOp<T>::v8 frag_tr(const T* lds, int ld, int cb, int k0, int k1, int lane) {
    const int i = lane & 15, G = lane >> 4;
    const int col = cb + (G & 1) * 16 + (i & 3) * 4;
    const i16x4 lo = ds_read_tr16(lds + (k0 + (i >> 2)) * ld + col);
    const i16x4 hi = ds_read_tr16(lds + (k1 + (i >> 2)) * ld + col);
    return join8<T>(lo, hi);
}

// Same, from a swizzled k-major tile [rows][64] read "sideways": rows of the
// tile are the k index, columns (the 64 k-major elements) are the fragment
// rows.
template <typename T>
__device__ __forceinline__ typename MfmaOp<T>::v8 frag_tr_kmaj(const T* lds, int cb, int r0, int r1, int lane) {
    const int i = lane & 15, G = lane >> 4;
    const int col = cb + (G & 1) * 16 + (i & 3) * 4;
    const i16x4 lo = ds_read_tr16(lds + kmaj_off(r0 + (i >> 2), col));
    const i16x4 hi = ds_read_tr16(lds + kmaj_off(r1 + (i >> 2), col));
    return join8<T>(lo, hi);
}

}  // namespace tel
