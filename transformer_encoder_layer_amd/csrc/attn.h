// attn.h -- tiled attention forward/backward (online softmax; the S x S
// score matrix is never written to memory).
#pragma once
#include <hip/hip_runtime.h>
#include "tel_common.h"

namespace tel {

struct AttnArgs {
    int dtype;          // tel_dtype
    int B, S, NH, d;    // H = NH * d
    const void* qkvh;   // [3][B][NH][S][d]
    const int32_t* len; // [B] valid key counts, or nullptr
    Drop drop;          // site 0; thr == 0: no dropout
    uint32_t* bits;     // optional keep bits [B][NH][S][S/32] (bit j%32 of word j/32 = key j):
                        // written by the MFMA forwards (words of key blocks at or beyond
                        // len[b] are not visited, so not written); read by the S <= 128
                        // backward; nullptr there: it regenerates them from the
                        // counter-based RNG, as the longer-S and generic kernels always do
    // forward
    void* ctx;          // [B*S][H] head-merged output
    float* lse;         // [B][NH][S] log2-sum-exp2 of the scaled scores
    // backward
    const void* dout;   // [B][NH][S][d] gradient of ctx, head-split
    float* dvec;        // [B][NH][S] rowsum(dO * O) (written by the dq kernel)
    void* dqkv;         // [B*S][3H] token-major gradient of the fused projection
    // Packed rows (optional): the rows of ctx and dqkv are packed[b*S + s]
    // instead of b*S + s, and tokens with packed < 0 (padding) are neither
    // written nor read.  MFMA kernels only.
    const int32_t* packed;
};

hipError_t attn_forward(const AttnArgs& a, hipStream_t st, bool force_simt = false);
hipError_t attn_backward(const AttnArgs& a, hipStream_t st, bool force_simt = false);

}  // namespace tel
