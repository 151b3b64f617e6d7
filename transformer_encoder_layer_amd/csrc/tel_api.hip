// tel_api.hip -- the C ABI of the fused encoder layer: argument validation,
// workspace planning and the launch sequence of one forward / backward.
//
// Launch sequence (per call, all on the caller's stream, no host sync):
//   Pre-LN forward : LN1 -> QKV GEMM (+bias, head split) -> attention ->
//                    out-proj GEMM (+bias, dropout 1, +x) -> LN2 ->
//                    FFN1 GEMM (+bias, GELU) -> FFN2 GEMM (+bias, dropout 2, +x1)
//   Post-LN forward: QKV GEMM -> attention -> out-proj GEMM (+x) -> LN1 ->
//                    FFN1 -> FFN2 (+x1) -> LN2
//   backward       : the chain rule in reverse; each GEMM is split into an
//                    input-gradient GEMM (with the GELU' / head-split / residual
//                    epilogue) and a weight-gradient GEMM; bias, gamma and beta
//                    gradients are deterministic two-stage column sums.
// The residual stream (x1, and z1/z2 for Post-LN) is kept in fp32 for bf16
// layers, so that their output carries a single rounding to bf16 (whose 8-bit
// significand would otherwise round twice); fp16 layers keep it in fp16.
#include <algorithm>
#include <math.h>
#include <stdarg.h>
#include <new>
#include <stdio.h>
#include <string.h>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tel.h"
#include "attn.h"
#include "gemm.h"
#include "rowops.h"

using namespace tel;

static thread_local std::string g_err;

static tel_status fail(tel_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static tel_status fail(tel_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

#define HIP_TRY(expr)                                                                         \
    do {                                                                                      \
        hipError_t e_ = (expr);                                                               \
        if (e_ != hipSuccess) return fail(TEL_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

namespace {

// ------------------------------------------------------------------ workspace plan
struct Buf {
    size_t off = 0, bytes = 0;
    bool in_saved = false;
    bool used = false;
};

struct Plan {
    // saved (forward -> backward)
    Buf ln1_out, mu1, rs1, qkvh, ctx, lse, mu2, rs2, ln2_out, u, g;
    Buf abits;    // attention keep bits, 1 per score (not kept under attention-dropout checkpointing)
    Buf res1;     // Pre-LN x1 | Post-LN z1 (fp32; the storage dtype for fp16 layers)
    Buf x1e;      // Post-LN LN1 output, dtype
    Buf x1f;      // Post-LN LN1 output, fp32 (residual of the FFN branch; bf16 and fp32 layers)
    Buf res2;     // Post-LN z2 (fp32; the storage dtype for fp16 layers)
    Buf ycopy;    // Post-LN output copy (invertible LN2 backward)
    // scratch (backward)
    Buf df, du, dgemm, dres, dz, dout, dvec, dqkv, dres2;
    Buf gck_g;    // GELU(u) recomputed in the backward under gelu checkpointing
    Buf part_ln, part_ln2, part_col, splitk;
    // token packing: row maps and x packed (saved); y, dy, dx packed (scratch)
    Buf rmap, rinv, xp, yp, dyp, dxp;
    size_t saved_bytes = 0, scratch_bytes = 0;
    size_t fwd_scratch_bytes = 0;  // the forward's own temporaries (a prefix of scratch)
};

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

}  // namespace

struct tel_layer {
    tel_config cfg;
    int B, S, H, NH, d, F, T;
    size_t esz;
    Plan plan;
    long pending_fwd;  // forwards with saved state not yet consumed by a backward
    long valid_tokens = 0;  // token packing: sum of the key lengths (0: not packed)
    // optional benchmark hook: events recorded around one kernel's launches
    int prof_kernel = -1;
    hipEvent_t* prof_start = nullptr;
    hipEvent_t* prof_stop = nullptr;
    int prof_count = 0;
    long prof_calls = 0;
    // optional test hook: the next training forward copies its attention keep bits here
    uint32_t* dbg_bits = nullptr;
};

// Run one launch; if it is the profiled kernel, bracket it with the next
// pair of the caller's events (same stream, so the pair spans exactly it).
#define TIMED(kid, expr)                                                                  \
    do {                                                                                  \
        const bool prof_ = L->prof_kernel == (kid) && L->prof_count > 0;                  \
        const int pi_ = prof_ ? (int)(L->prof_calls % L->prof_count) : 0;                 \
        if (prof_) HIP_TRY(hipEventRecord(L->prof_start[pi_], st));                       \
        HIP_TRY(expr);                                                                    \
        if (prof_) {                                                                      \
            HIP_TRY(hipEventRecord(L->prof_stop[pi_], st));                               \
            L->prof_calls++;                                                              \
        }                                                                                 \
    } while (0)

static void place(Buf& b, size_t bytes, bool saved, size_t& sv, size_t& sc) {
    b.bytes = bytes;
    b.used = true;
    b.in_saved = saved;
    size_t& top = saved ? sv : sc;
    b.off = top;
    top = align_up(top + bytes);
}

// Residual stream in fp32 (bf16 and fp32 layers) or in the storage dtype (fp16).
static bool residual_f32(const tel_layer* L) { return L->cfg.dtype != TEL_F16; }

static void make_plan(tel_layer* L) {
    Plan& p = L->plan;
    p = Plan();
    const size_t T = L->T, H = L->H, F = L->F, e = L->esz, f4 = 4;
    const size_t BNS = (size_t)L->B * L->NH * L->S;
    const bool inv = L->cfg.normalize_invertible != 0;
    const bool gck = L->cfg.gelu_checkpoint != 0;
    const size_t rs = residual_f32(L) ? f4 : e;  // residual stream element size
    // The 1-bit keep mask of the attention probabilities is kept only where
    // the whole-sequence kernels run (S <= 128: B*N*S*S/8 bytes, 2 MiB per
    // BERT-Large layer).  Longer sequences always regenerate it in the
    // backward, so nothing the layer keeps grows with S^2.
    const bool keep_bits = L->cfg.attn_dropout > 0.0f && !L->cfg.attn_dropout_checkpoint &&
                           L->d == 64 && L->S % 64 == 0 && L->S <= 128 && L->cfg.dtype != TEL_F32;
    size_t sv = 0, sc = 0;
    if (keep_bits) place(p.abits, BNS * (size_t)(L->S / 32) * 4, true, sv, sc);
    if (L->cfg.pack_tokens) {
        place(p.rmap, T * 4, true, sv, sc);
        place(p.rinv, T * 4, true, sv, sc);
        place(p.xp, T * H * e, true, sv, sc);
        place(p.yp, T * H * e, false, sv, sc);
    }
    if (L->cfg.pre_ln) {
        place(p.ln1_out, T * H * e, true, sv, sc);
        place(p.mu1, T * f4, true, sv, sc);
        place(p.rs1, T * f4, true, sv, sc);
        place(p.qkvh, 3 * T * H * e, true, sv, sc);
        place(p.ctx, T * H * e, true, sv, sc);
        place(p.lse, BNS * f4, true, sv, sc);
        place(p.res1, T * H * rs, !inv, sv, sc);
        place(p.mu2, T * f4, true, sv, sc);
        place(p.rs2, T * f4, true, sv, sc);
        place(p.ln2_out, T * H * e, true, sv, sc);
        place(p.u, T * F * e, true, sv, sc);  // GELU input u, or GELU'(u) unless GELU is checkpointed
        place(p.g, T * F * e, !gck, sv, sc);
    } else {
        place(p.qkvh, 3 * T * H * e, true, sv, sc);
        place(p.ctx, T * H * e, true, sv, sc);
        place(p.lse, BNS * f4, true, sv, sc);
        place(p.res1, T * H * rs, !inv, sv, sc);
        place(p.mu1, T * f4, true, sv, sc);
        place(p.rs1, T * f4, true, sv, sc);
        place(p.x1e, T * H * e, true, sv, sc);
        if (rs == f4) place(p.x1f, T * H * f4, inv, sv, sc);  // fp32 copy of x1 (FFN-branch residual)
        place(p.u, T * F * e, true, sv, sc);
        place(p.g, T * F * e, !gck, sv, sc);
        place(p.res2, T * H * rs, !inv, sv, sc);
        place(p.mu2, T * f4, true, sv, sc);
        place(p.rs2, T * f4, true, sv, sc);
        if (inv) place(p.ycopy, T * H * e, true, sv, sc);
    }
    const size_t fwd_scratch = sc;
    // backward scratch starts again at 0: forward temporaries are dead by then
    sc = 0;
    place(p.df, T * H * e, false, sv, sc);
    place(p.du, T * F * e, false, sv, sc);
    if (gck) place(p.gck_g, T * F * e, false, sv, sc);
    place(p.dgemm, T * H * e, false, sv, sc);
    // gradient of the residual stream between the two LayerNorm backwards:
    // Pre-LN keeps it in the residual's type (fp16 for fp16 layers)
    place(p.dres, T * H * (L->cfg.pre_ln ? rs : f4), false, sv, sc);
    place(p.dres2, T * H * f4, false, sv, sc);
    place(p.dz, T * H * e, false, sv, sc);
    place(p.dout, T * H * e, false, sv, sc);
    place(p.dvec, BNS * f4, false, sv, sc);
    place(p.dqkv, 3 * T * H * e, false, sv, sc);
    if (L->cfg.pack_tokens) {
        place(p.dyp, T * H * e, false, sv, sc);
        place(p.dxp, T * H * e, false, sv, sc);
    }
    const size_t maxN = 3 * H > F ? 3 * H : F;
    // gamma/beta partial rows of LN1 and LN2 (both are finalized at the end)
    place(p.part_ln, 2 * (size_t)ln_backward_parts(L->T) * H * f4, false, sv, sc);
    place(p.part_ln2, 2 * (size_t)ln_backward_parts(L->T) * H * f4, false, sv, sc);
    place(p.part_col, (size_t)colsum_parts(L->T) * maxN * f4, false, sv, sc);
    // split-K partials of the four weight-gradient GEMMs
    size_t sk = 0;
    const int wg[4][2] = {{3 * L->H, L->H}, {L->H, L->H}, {L->F, L->H}, {L->H, L->F}};
    GemmDesc wd[4];
    for (int i = 0; i < 4; ++i) {
        GemmDesc& gd = wd[i];
        gd.dtype = L->cfg.dtype;
        gd.M = wg[i][0]; gd.N = wg[i][1]; gd.K = L->T;
        gd.lda = wg[i][0]; gd.ldb = wg[i][1];
        gd.a_kmajor = false; gd.b_kmajor = false;
        gd.epi = EPI_STORE;
        sk = std::max(sk, gemm_splitk_elems(gd));
    }
    // the paired launches: W_o with W_qkv, W_2 with W_1
    sk = std::max(sk, gemm_splitk_group_elems(wd[1], wd[0]));
    sk = std::max(sk, gemm_splitk_group_elems(wd[3], wd[2]));
    if (sk) place(p.splitk, sk * f4, false, sv, sc);
    p.saved_bytes = sv;
    p.scratch_bytes = sc > fwd_scratch ? sc : fwd_scratch;
    p.fwd_scratch_bytes = fwd_scratch;
}

// smallest non-zero dropout probability a 16-bit draw realises
constexpr float kMinDropP = 1.0f / 65536.0f;

static tel_status validate_cfg(const tel_config* c) {
    if (!c) return fail(TEL_ERR_INVALID_ARG, "config is NULL");
    if (c->batch <= 0 || c->seq <= 0 || c->hidden <= 0 || c->heads <= 0)
        return fail(TEL_ERR_INVALID_ARG, "batch, seq, hidden and heads must be positive");
    const int F = c->ffn <= 0 ? 4 * c->hidden : c->ffn;
    if (c->hidden % c->heads) return fail(TEL_ERR_INVALID_ARG, "hidden %d not divisible by heads %d", c->hidden, c->heads);
    if (c->seq % 16 || c->hidden % 16 || F % 16)
        return fail(TEL_ERR_INVALID_ARG, "seq, hidden and ffn must be multiples of 16");
    const int d = c->hidden / c->heads;
    if (d != 16 && d != 32 && d != 64 && d != 128) return fail(TEL_ERR_UNSUPPORTED, "head width %d not in {16,32,64,128}", d);
    if (c->hidden > 2048) return fail(TEL_ERR_UNSUPPORTED, "hidden %d > 2048", c->hidden);
    if (!(c->attn_dropout >= 0.0f && c->attn_dropout < 1.0f) || !(c->hidden_dropout >= 0.0f && c->hidden_dropout < 1.0f))
        return fail(TEL_ERR_INVALID_ARG, "dropout probabilities must lie in [0,1)");
    // Each element draws a 16-bit value, so the drop probability is realised
    // as floor(p * 2^16) / 2^16: below 2^-16 that is zero, i.e. no dropout at
    // all, which would silently differ from the p asked for.
    if ((c->attn_dropout > 0.0f && c->attn_dropout < kMinDropP) ||
        (c->hidden_dropout > 0.0f && c->hidden_dropout < kMinDropP))
        return fail(TEL_ERR_UNSUPPORTED, "dropout probabilities in (0, 2^-16) cannot be realised by 16-bit draws");
    if (c->dtype != TEL_F32 && c->dtype != TEL_F16 && c->dtype != TEL_BF16)
        return fail(TEL_ERR_INVALID_ARG, "unknown dtype %d", c->dtype);
    if (!(c->ln_eps >= 0.0f)) return fail(TEL_ERR_INVALID_ARG, "ln_eps must be >= 0");
    if (c->pack_tokens && (c->dtype == TEL_F32 || d != 64 || c->seq % 64))
        return fail(TEL_ERR_UNSUPPORTED, "pack_tokens needs fp16/bf16, head width 64 and seq a multiple of 64");
    const double T = (double)c->batch * c->seq;
    if (T * (double)(3 * c->hidden > F ? 3 * c->hidden : F) >= 2147483647.0 ||
        (double)c->batch * c->heads * c->seq * (double)c->seq >= 9.0e18)
        return fail(TEL_ERR_UNSUPPORTED, "problem too large for 32-bit row indexing");
    return TEL_OK;
}

static bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ------------------------------------------------------------------ static workspace
// For callers that cannot allocate (code under graph capture, tight serving
// loops): tel_layer_forward_noalloc runs the inference forward in this
// file-scope device array.  Each device the library runs on holds its own
// copy until the process ends.  In host code `scratch` is only a stand-in
// for the symbol; its device address comes from hipGetSymbolAddress, taken
// once per device with that device current and kept in g_noalloc_ptr.
constexpr size_t kNoAllocBytes = (size_t)64 << 20;
namespace noalloc {
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];
}
constexpr int kMaxDevices = 64;
static std::mutex g_noalloc_mu;
static void* g_noalloc_ptr[kMaxDevices];

// Bytes the inference forward (saved = NULL) uses of its scratch: the
// forward's temporaries, then the region that holds the kept tensors.
static size_t noalloc_need(const tel_layer* L) {
    return align_up(L->plan.fwd_scratch_bytes) + L->plan.saved_bytes;
}

static tel_status noalloc_base(void** out) {
    int dev = 0;
    HIP_TRY(hipGetDevice(&dev));
    if (dev < 0 || dev >= kMaxDevices) return fail(TEL_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_noalloc_mu);
    if (!g_noalloc_ptr[dev]) {
        void* p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc::scratch)));
        if (!p) return fail(TEL_ERR_HIP, "hipGetSymbolAddress returned NULL for the static workspace");
        g_noalloc_ptr[dev] = p;
    }
    *out = g_noalloc_ptr[dev];
    return TEL_OK;
}

static tel_status check_lengths_host(const int32_t* len, int B, int S) {
    for (int b = 0; b < B; ++b)
        if (len[b] < 1 || len[b] > S)
            return fail(TEL_ERR_INVALID_ARG, "key_lengths[%d] = %d outside [1, %d]", b, (int)len[b], S);
    return TEL_OK;
}

#ifdef TEL_DEBUG_CHECKS
// Debug builds: copy the device key lengths to the host and check them
// before any kernel reads them (this synchronises the stream).
static tel_status debug_check_lengths(const tel_layer* L, const int32_t* key_lengths, hipStream_t st) {
    if (!key_lengths) return TEL_OK;
    std::vector<int32_t> h(L->B);
    HIP_TRY(hipMemcpyAsync(h.data(), key_lengths, sizeof(int32_t) * L->B, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    return check_lengths_host(h.data(), L->B, L->S);
}
#define DEBUG_CHECK_LENGTHS(L, kl, st)                      \
    do {                                                    \
        tel_status ds_ = debug_check_lengths((L), (kl), (st)); \
        if (ds_ != TEL_OK) return ds_;                      \
    } while (0)
#else
#define DEBUG_CHECK_LENGTHS(L, kl, st) \
    do {                               \
    } while (0)
#endif

static Drop make_drop(const tel_layer* L, float p, uint32_t site, uint64_t step, int training) {
    Drop d;
    d.rng.key0 = (uint32_t)L->cfg.seed;
    d.rng.key1 = (uint32_t)L->cfg.layer_id;
    d.rng.site = site;
    d.rng.step = (uint32_t)step;
    d.thr = 0;
    d.scale = 1.0f;
    if (training && p > 0.0f) {
        // drop iff the element's 16-bit value < floor(p * 2^16) (>= 1 for every
        // p the config accepts); kept values are scaled by 1/(1-p)
        d.thr = (uint32_t)floor((double)p * 65536.0);
        if (d.thr) d.scale = (float)(1.0 / (1.0 - (double)p));
    }
    return d;
}

extern "C" {

const char* tel_last_error(void) { return g_err.c_str(); }

tel_status tel_layer_create(const tel_config* cfg, tel_layer** out) {
    if (!out) return fail(TEL_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    tel_status s = validate_cfg(cfg);
    if (s != TEL_OK) return s;
    tel_layer* L = new (std::nothrow) tel_layer();
    if (!L) return fail(TEL_ERR_INVALID_ARG, "out of host memory");
    L->cfg = *cfg;
    L->B = cfg->batch; L->S = cfg->seq; L->H = cfg->hidden; L->NH = cfg->heads;
    L->d = cfg->hidden / cfg->heads;
    L->F = cfg->ffn <= 0 ? 4 * cfg->hidden : cfg->ffn;
    L->cfg.ffn = L->F;
    L->T = L->B * L->S;
    L->esz = cfg->dtype == TEL_F32 ? 4 : 2;
    L->pending_fwd = 0;
    make_plan(L);
    *out = L;
    g_err.clear();
    return TEL_OK;
}

tel_status tel_layer_workspace_bytes(const tel_layer* L, size_t* saved_bytes, size_t* scratch_bytes) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    if (saved_bytes) *saved_bytes = L->plan.saved_bytes;
    if (scratch_bytes) *scratch_bytes = L->plan.scratch_bytes;
    return TEL_OK;
}

tel_status tel_layer_set_valid_tokens(tel_layer* L, int64_t valid_tokens) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    if (!L->cfg.pack_tokens) return fail(TEL_ERR_UNSUPPORTED, "layer was created without pack_tokens");
    if (valid_tokens < 0 || valid_tokens > (int64_t)L->T)
        return fail(TEL_ERR_INVALID_ARG, "valid_tokens %lld outside [0, %d]", (long long)valid_tokens, L->T);
    L->valid_tokens = (long)valid_tokens;
    g_err.clear();
    return TEL_OK;
}

tel_status tel_layer_destroy(tel_layer* L) {
    delete L;
    return TEL_OK;
}

static tel_status check_params(const tel_params* p) {
    if (!p) return fail(TEL_ERR_INVALID_ARG, "params is NULL");
    const void* ptrs[12] = {p->w_qkv, p->b_qkv, p->w_o, p->b_o, p->ln1_g, p->ln1_b,
                            p->w_1, p->b_1, p->w_2, p->b_2, p->ln2_g, p->ln2_b};
    for (int i = 0; i < 12; ++i) {
        if (!ptrs[i]) return fail(TEL_ERR_INVALID_ARG, "parameter %d is NULL", i);
        if (!aligned(ptrs[i])) return fail(TEL_ERR_INVALID_ARG, "parameter %d not 16-byte aligned", i);
    }
    return TEL_OK;
}

static tel_status check_grads(const tel_grads* g) {
    if (!g) return fail(TEL_ERR_INVALID_ARG, "grads is NULL");
    void* ptrs[12] = {g->w_qkv, g->b_qkv, g->w_o, g->b_o, g->ln1_g, g->ln1_b,
                      g->w_1, g->b_1, g->w_2, g->b_2, g->ln2_g, g->ln2_b};
    for (int i = 0; i < 12; ++i) {
        if (!ptrs[i]) return fail(TEL_ERR_INVALID_ARG, "gradient %d is NULL", i);
        if (!aligned(ptrs[i])) return fail(TEL_ERR_INVALID_ARG, "gradient %d not 16-byte aligned", i);
    }
    return TEL_OK;
}

// Rows the layer runs on: the valid tokens rounded up to the 256-row GEMM
// tile when packing pays (some padding, key lengths given), else all B*S.
static int packed_rows(const tel_layer* L, const int32_t* key_lengths) {
    if (!L->cfg.pack_tokens || !key_lengths || L->valid_tokens <= 0) return 0;
    const long P = (L->valid_tokens + 255) / 256 * 256;
    return P < L->T ? (int)P : 0;
}

struct Bases {
    void* saved;
    void* scratch;
    void* of(const Buf& b) const { return (char*)(b.in_saved ? saved : scratch) + b.off; }
};

tel_status tel_layer_forward(tel_layer* L, const tel_params* P, const void* x, const int32_t* key_lengths,
                             int training, uint64_t step, void* y, void* saved, void* scratch,
                             tel_stream_t stream) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    tel_status s = check_params(P);
    if (s != TEL_OK) return s;
    if (!x || !y || !scratch) return fail(TEL_ERR_INVALID_ARG, "x, y and scratch must be non-NULL");
    if (!aligned(x) || !aligned(y) || !aligned(scratch) || (saved && !aligned(saved)) ||
        (key_lengths && !aligned(key_lengths)))
        return fail(TEL_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    if (x == y) return fail(TEL_ERR_INVALID_ARG, "y must not alias x");
    hipStream_t st = (hipStream_t)stream;
    DEBUG_CHECK_LENGTHS(L, key_lengths, st);
    const tel_config& c = L->cfg;
    const Plan& p = L->plan;
    const int H = L->H, F = L->F, dt = c.dtype;
    // without a saved buffer every "saved" tensor lives in a private region of
    // scratch placed after the forward's own temporaries; callers that pass
    // saved = NULL size scratch as saved_bytes + scratch_bytes (at least that)
    void* sv = saved ? saved : (char*)scratch + align_up(p.fwd_scratch_bytes);
    Bases bs{sv, scratch};
    // token packing: the layer runs on PR packed rows (x gathered, y scattered back)
    const int PR = packed_rows(L, key_lengths);
    const int T = PR ? PR : L->T;
    const int32_t* rmap = PR ? (const int32_t*)bs.of(p.rmap) : nullptr;
    const int32_t* rinv = PR ? (const int32_t*)bs.of(p.rinv) : nullptr;
    const void* xin = x;
    void* yout = y;
    if (PR) {
        HIP_TRY(build_row_maps(key_lengths, L->B, L->S, PR, (int32_t*)bs.of(p.rmap), (int32_t*)bs.of(p.rinv), st));
        HIP_TRY(gather_rows(dt, x, bs.of(p.xp), rmap, PR, H, st));
        // the QKV epilogue writes valid tokens only; attention reads the rest as zeros
        HIP_TRY(zero_padded_heads(dt, bs.of(p.qkvh), 3, L->B, L->NH, L->S, L->d, key_lengths, st));
        xin = bs.of(p.xp);
        yout = bs.of(p.yp);
    }
    const Drop d0 = make_drop(L, c.attn_dropout, 0, step, training);
    const Drop d1 = make_drop(L, c.hidden_dropout, 1, step, training);
    const Drop d2 = make_drop(L, c.hidden_dropout, 2, step, training);
    const int r32 = residual_f32(L) ? 1 : 0;

    AttnArgs aa{};
    aa.dtype = dt; aa.B = L->B; aa.S = L->S; aa.NH = L->NH; aa.d = L->d;
    aa.qkvh = bs.of(p.qkvh); aa.len = key_lengths; aa.drop = d0;
    aa.ctx = bs.of(p.ctx); aa.lse = (float*)bs.of(p.lse);
    aa.bits = p.abits.used ? (uint32_t*)bs.of(p.abits) : nullptr;
    aa.packed = rinv;
    // test hook: the keep bits this forward applies go to the caller's buffer
    // too (written there directly when the layer keeps none of its own)
    uint32_t* dbg_bits = d0.thr ? L->dbg_bits : nullptr;
    L->dbg_bits = nullptr;
    if (dbg_bits && !aa.bits) aa.bits = dbg_bits;
    // attention writes the valid tokens' rows of ctx; filler rows must be finite
    auto attn = [&]() -> hipError_t {
        hipError_t e = attn_forward(aa, st);
        if (e == hipSuccess && dbg_bits && aa.bits != dbg_bits)
            e = hipMemcpyAsync(dbg_bits, aa.bits, p.abits.bytes, hipMemcpyDeviceToDevice, st);
        if (e != hipSuccess || !PR) return e;
        return zero_rows(dt, aa.ctx, (int)L->valid_tokens, PR, H, st);
    };

    auto proj = [&](const void* A, const void* W, int N, int K, int epi) {
        GemmDesc g;
        g.dtype = dt; g.M = T; g.N = N; g.K = K;
        g.A = A; g.lda = K; g.a_kmajor = true;
        g.B = W; g.ldb = K; g.b_kmajor = true;
        g.epi = epi;
        g.ea.row_map = rmap;
        return g;
    };

    if (c.pre_ln) {
        LnFwdArgs l1{dt, T, H, c.ln_eps, xin, 0, P->ln1_g, P->ln1_b, bs.of(p.ln1_out), nullptr, nullptr,
                     (float*)bs.of(p.mu1), (float*)bs.of(p.rs1)};
        TIMED(TEL_K_LN1_FWD, ln_forward(l1, st));
        GemmDesc g = proj(bs.of(p.ln1_out), P->w_qkv, 3 * H, H, EPI_QKV);
        g.ea.out = bs.of(p.qkvh); g.ea.bias = P->b_qkv;
        g.ea.B = L->B; g.ea.S = L->S; g.ea.H = H; g.ea.NH = L->NH; g.ea.d = L->d;
        TIMED(TEL_K_QKV_FWD, gemm_launch(g, st));
        TIMED(TEL_K_ATTN_FWD, attn());
        g = proj(bs.of(p.ctx), P->w_o, H, H, EPI_BIAS_DROP_RES);
        g.ea.out = bs.of(p.res1); g.ea.ldo = H; g.ea.out_f32 = r32; g.ea.bias = P->b_o;
        g.ea.res = xin; g.ea.res_f32 = 0; g.ea.drop = d1;
        TIMED(TEL_K_OUT_FWD, gemm_launch(g, st));
        LnFwdArgs l2{dt, T, H, c.ln_eps, bs.of(p.res1), r32, P->ln2_g, P->ln2_b, bs.of(p.ln2_out), nullptr, nullptr,
                     (float*)bs.of(p.mu2), (float*)bs.of(p.rs2)};
        TIMED(TEL_K_LN2_FWD, ln_forward(l2, st));
        g = proj(bs.of(p.ln2_out), P->w_1, F, H, EPI_BIAS_GELU);
        g.ea.out = bs.of(p.u); g.ea.ldo = F; g.ea.bias = P->b_1; g.ea.out2 = bs.of(p.g);
        g.ea.gelu_grad_out = !c.gelu_checkpoint;
        TIMED(TEL_K_FFN1_FWD, gemm_launch(g, st));
        g = proj(bs.of(p.g), P->w_2, H, F, EPI_BIAS_DROP_RES);
        g.ea.out = yout; g.ea.ldo = H; g.ea.out_f32 = 0; g.ea.bias = P->b_2;
        g.ea.res = bs.of(p.res1); g.ea.res_f32 = r32; g.ea.drop = d2;
        TIMED(TEL_K_FFN2_FWD, gemm_launch(g, st));
    } else {
        GemmDesc g = proj(xin, P->w_qkv, 3 * H, H, EPI_QKV);
        g.ea.out = bs.of(p.qkvh); g.ea.bias = P->b_qkv;
        g.ea.B = L->B; g.ea.S = L->S; g.ea.H = H; g.ea.NH = L->NH; g.ea.d = L->d;
        TIMED(TEL_K_QKV_FWD, gemm_launch(g, st));
        TIMED(TEL_K_ATTN_FWD, attn());
        g = proj(bs.of(p.ctx), P->w_o, H, H, EPI_BIAS_DROP_RES);
        g.ea.out = bs.of(p.res1); g.ea.ldo = H; g.ea.out_f32 = r32; g.ea.bias = P->b_o;
        g.ea.res = xin; g.ea.res_f32 = 0; g.ea.drop = d1;
        TIMED(TEL_K_OUT_FWD, gemm_launch(g, st));
        LnFwdArgs l1{dt, T, H, c.ln_eps, bs.of(p.res1), r32, P->ln1_g, P->ln1_b, bs.of(p.x1e),
                     p.x1f.used ? (float*)bs.of(p.x1f) : nullptr, nullptr, (float*)bs.of(p.mu1), (float*)bs.of(p.rs1)};
        TIMED(TEL_K_LN1_FWD, ln_forward(l1, st));
        g = proj(bs.of(p.x1e), P->w_1, F, H, EPI_BIAS_GELU);
        g.ea.out = bs.of(p.u); g.ea.ldo = F; g.ea.bias = P->b_1; g.ea.out2 = bs.of(p.g);
        g.ea.gelu_grad_out = !c.gelu_checkpoint;
        TIMED(TEL_K_FFN1_FWD, gemm_launch(g, st));
        g = proj(bs.of(p.g), P->w_2, H, F, EPI_BIAS_DROP_RES);
        g.ea.out = bs.of(p.res2); g.ea.ldo = H; g.ea.out_f32 = r32; g.ea.bias = P->b_2;
        g.ea.res = r32 ? bs.of(p.x1f) : bs.of(p.x1e); g.ea.res_f32 = r32; g.ea.drop = d2;
        TIMED(TEL_K_FFN2_FWD, gemm_launch(g, st));
        LnFwdArgs l2{dt, T, H, c.ln_eps, bs.of(p.res2), r32, P->ln2_g, P->ln2_b, yout, nullptr,
                     p.ycopy.used ? bs.of(p.ycopy) : nullptr, (float*)bs.of(p.mu2), (float*)bs.of(p.rs2)};
        TIMED(TEL_K_LN2_FWD, ln_forward(l2, st));
    }
    if (PR) HIP_TRY(scatter_rows(dt, yout, y, rinv, L->T, H, st));
    if (saved) L->pending_fwd++;
    g_err.clear();
    return TEL_OK;
}

// The backward, optionally chained through a Pre-LN stack: dy_dropped (if
// set) is this layer's site-2 masked dy, computed by the layer above; below
// (if set) is the next layer down, whose site-2 mask the LN1 backward applies
// to dx into dx_dropped.
static tel_status backward_impl(tel_layer* L, const tel_params* P, const void* x, const int32_t* key_lengths,
                                int training, uint64_t step, const void* dy, const void* dy_dropped,
                                const void* saved, void* scratch, void* dx, const tel_layer* below,
                                void* dx_dropped, const tel_grads* G, tel_stream_t stream) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    tel_status s = check_params(P);
    if (s != TEL_OK) return s;
    s = check_grads(G);
    if (s != TEL_OK) return s;
    const tel_config& c = L->cfg;
    const bool need_x = !(c.pre_ln && c.normalize_invertible);
    if (!dy || !saved || !scratch || !dx || (need_x && !x))
        return fail(TEL_ERR_INVALID_ARG, "dy, saved, scratch, dx (and x unless Pre-LN invertible) must be non-NULL");
    if (!aligned(dy) || !aligned(saved) || !aligned(scratch) || !aligned(dx) || (x && !aligned(x)) ||
        (key_lengths && !aligned(key_lengths)))
        return fail(TEL_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
    const bool chained = dy_dropped || below || dx_dropped;
    if (chained) {
        if (!c.pre_ln)
            return fail(TEL_ERR_INVALID_ARG, "chained backward is for Pre-LN layers (Post-LN applies site 2 "
                                             "after its own LayerNorm backward)");
        if (!below != !dx_dropped) return fail(TEL_ERR_INVALID_ARG, "below and dx_dropped go together");
        if (dx_dropped && (dx_dropped == dx || dx_dropped == dy || dx_dropped == dy_dropped))
            return fail(TEL_ERR_INVALID_ARG, "dx_dropped may not alias dy, dy_dropped or dx");
        if ((dy_dropped && !aligned(dy_dropped)) || (dx_dropped && !aligned(dx_dropped)))
            return fail(TEL_ERR_INVALID_ARG, "buffers must be 16-byte aligned");
        if (below) {
            const tel_config& b = below->cfg;
            if (b.batch != c.batch || b.seq != c.seq || b.hidden != c.hidden || b.dtype != c.dtype || !b.pre_ln ||
                b.hidden_dropout != c.hidden_dropout)
                return fail(TEL_ERR_INVALID_ARG, "below must be a Pre-LN layer of the same batch, sequence, hidden "
                                                 "size, dtype and hidden dropout");
        }
        if (packed_rows(L, key_lengths))
            return fail(TEL_ERR_UNSUPPORTED, "chained backward does not run on packed tokens");
    }
    if (L->pending_fwd <= 0) return fail(TEL_ERR_STATE, "backward called without a preceding forward with saved state");
    hipStream_t st = (hipStream_t)stream;
    DEBUG_CHECK_LENGTHS(L, key_lengths, st);
    const Plan& p = L->plan;
    const int H = L->H, F = L->F, dt = c.dtype;
    Bases bs{const_cast<void*>(saved), scratch};
    // token packing: the forward's PR packed rows (dy gathered, dx scattered back)
    const int PR = packed_rows(L, key_lengths);
    const int T = PR ? PR : L->T;
    const int32_t* rmap = PR ? (const int32_t*)bs.of(p.rmap) : nullptr;
    const int32_t* rinv = PR ? (const int32_t*)bs.of(p.rinv) : nullptr;
    const void* xin = PR ? bs.of(p.xp) : x;
    const void* dyin = dy;
    void* dxout = dx;
    if (PR) {
        HIP_TRY(gather_rows(dt, dy, bs.of(p.dyp), rmap, PR, H, st));
        dyin = bs.of(p.dyp);
        dxout = bs.of(p.dxp);
    }
    const Drop d0 = make_drop(L, c.attn_dropout, 0, step, training);
    const Drop d1 = make_drop(L, c.hidden_dropout, 1, step, training);
    const Drop d2 = make_drop(L, c.hidden_dropout, 2, step, training);
    const bool inv = c.normalize_invertible != 0;
    const bool gck = c.gelu_checkpoint != 0;
    const int r32 = residual_f32(L) ? 1 : 0;
    // LN1's and LN2's gamma/beta partial rows (separate buffers: both are
    // finalized at the end, with the last weight-gradient pair when it runs)
    const int lnP = ln_backward_parts(T);
    float* part_ln1_g = (float*)bs.of(p.part_ln);
    float* part_ln1_b = part_ln1_g + (size_t)lnP * H;
    float* part_ln2_g = (float*)bs.of(p.part_ln2);
    float* part_ln2_b = part_ln2_g + (size_t)lnP * H;
    float* part_col = (float*)bs.of(p.part_col);
    const int colP = colsum_parts(T);
    float* skws = p.splitk.used ? (float*)bs.of(p.splitk) : nullptr;
    const size_t skn = p.splitk.used ? p.splitk.bytes / 4 : 0;

    // dX[T][in] = dY[T][out] . W[out][in]
    auto dgrad = [&](const void* dY, const void* W, int out, int in, int epi) {
        GemmDesc g;
        g.dtype = dt; g.M = T; g.N = in; g.K = out;
        g.A = dY; g.lda = out; g.a_kmajor = true;
        g.B = W; g.ldb = in; g.b_kmajor = false;
        g.epi = epi;
        g.ea.row_map = rmap;
        return g;
    };
    // dW[out][in] = dY^T . X, written to the caller's gradient (dtype)
    auto bias_grad = [&](const void* dY, int N, void* out) -> hipError_t {
        hipError_t e = colsum_partial(dt, dY, T, N, part_col, st);
        if (e != hipSuccess) return e;
        return colsum_finalize(dt, part_col, colP, N, out, st);
    };
    // dW = dY^T X and db = sum_t dY: fused into the GEMM when its kernel can
    struct Wg {
        const void *dY, *X;
        int out, in;
        void *dW, *db;
    };
    auto wdesc = [&](const Wg& w) {
        GemmDesc g;
        g.dtype = dt; g.M = w.out; g.N = w.in; g.K = T;
        g.A = w.dY; g.lda = w.out; g.a_kmajor = false;
        g.B = w.X; g.ldb = w.in; g.b_kmajor = false;
        g.epi = EPI_STORE;
        g.ea.out = w.dW; g.ea.ldo = w.in;
        g.splitk_ws = skws; g.splitk_ws_elems = skn;
        g.splitk_atomic = c.stochastic_mode != 0;  // honoured by grouped launches only
        if (gemm_rowsum_fused(g)) g.rowsum_out = w.db;
        return g;
    };
    auto wgrad1 = [&](const Wg& w) -> hipError_t {
        const GemmDesc g = wdesc(w);
        hipError_t e = gemm_launch(g, st);
        if (e != hipSuccess || g.rowsum_out) return e;
        return bias_grad(w.dY, w.out, w.db);
    };
    // Two weight gradients run as one grouped launch when both qualify (the
    // tiles of both fill the chip with fewer k-splits), else one after the
    // other.  A profiled kernel id always runs alone, so its events cover
    // only it.
    auto grouped = [&](int ka, const Wg& a, int kb, const Wg& b) {
        const GemmDesc ga = wdesc(a), gb = wdesc(b);
        const bool alone = L->prof_kernel == ka || L->prof_kernel == kb;
        return !alone && ga.rowsum_out && gb.rowsum_out && gemm_group_ok(ga, gb);
    };
    // The LayerNorm gamma/beta finalizes (fixed-order column sums of the
    // partial rows): when the last pair (W_o with W_qkv, the end of the
    // backward) runs grouped, they wait for it and ride with its reduction
    // launch; otherwise each runs right after its LayerNorm backward.
    const bool fold_ln = grouped(TEL_K_OUT_WGRAD, Wg{nullptr, nullptr, H, H, G->w_o, G->b_o},
                                 TEL_K_QKV_WGRAD, Wg{nullptr, nullptr, 3 * H, H, G->w_qkv, G->b_qkv});
    ColsumJob ln_fin[kMaxColsumJobs];
    int n_ln_fin = 0;
    auto ln_grads = [&](const float* pg, const float* pb, void* gg, void* gb) -> hipError_t {
        if (!fold_ln) return colsum_finalize2(dt, pg, pb, lnP, H, gg, gb, st);
        ln_fin[n_ln_fin++] = ColsumJob{pg, lnP, H, gg};
        ln_fin[n_ln_fin++] = ColsumJob{pb, lnP, H, gb};
        return hipSuccess;
    };
    // with_ln: the last pair, which takes the pending LayerNorm finalizes
    auto wgrad_pair = [&](int ka, const Wg& a, int kb, const Wg& b, bool with_ln) -> tel_status {
        const GemmDesc ga = wdesc(a), gb = wdesc(b);
        if (grouped(ka, a, kb, b)) {
            const bool ffn = ka == TEL_K_FFN2_WGRAD;
            const int pair = ffn ? TEL_K_FFN_WGRAD_PAIR : TEL_K_ATTN_WGRAD_PAIR;
            const int red = ffn ? TEL_K_FFN_WGRAD_REDUCE : TEL_K_ATTN_WGRAD_REDUCE;
            // profiled: events around the GEMM kernel, or around the launch after it
            GroupEvents ev{};
            if (L->prof_count > 0 && (L->prof_kernel == pair || L->prof_kernel == red)) {
                const int pi = (int)(L->prof_calls++ % L->prof_count);
                if (L->prof_kernel == pair) {
                    ev.gemm_start = L->prof_start[pi];
                    ev.gemm_stop = L->prof_stop[pi];
                } else {
                    ev.red_start = L->prof_start[pi];
                    ev.red_stop = L->prof_stop[pi];
                }
            }
            HIP_TRY(gemm_launch_group(ga, gb, st, with_ln ? ln_fin : nullptr, with_ln ? n_ln_fin : 0, &ev));
            if (with_ln) n_ln_fin = 0;
        } else {
            TIMED(ka, wgrad1(a));
            TIMED(kb, wgrad1(b));
        }
        if (with_ln) {
            for (int i = 0; i < n_ln_fin; i += 2)
                HIP_TRY(colsum_finalize2(dt, ln_fin[i].part, ln_fin[i + 1].part, lnP, H, ln_fin[i].out,
                                         ln_fin[i + 1].out, st));
            n_ln_fin = 0;
        }
        return TEL_OK;
    };

    AttnArgs aa{};
    aa.dtype = dt; aa.B = L->B; aa.S = L->S; aa.NH = L->NH; aa.d = L->d;
    aa.qkvh = bs.of(p.qkvh); aa.len = key_lengths; aa.drop = d0;
    aa.ctx = bs.of(p.ctx); aa.lse = (float*)bs.of(p.lse);
    aa.dout = bs.of(p.dout); aa.dvec = (float*)bs.of(p.dvec); aa.dqkv = bs.of(p.dqkv);
    aa.bits = p.abits.used ? (uint32_t*)bs.of(p.abits) : nullptr;
    aa.packed = rinv;
    // padding tokens: their dO is zero (the head-split scatter writes valid
    // tokens only), and the filler rows of dqkv must be finite for the GEMMs
    auto attn = [&]() -> hipError_t {
        hipError_t e = attn_backward(aa, st);
        if (e != hipSuccess || !PR) return e;
        return zero_rows(dt, aa.dqkv, (int)L->valid_tokens, PR, 3 * H, st);
    };
    auto zero_dout = [&]() -> hipError_t {
        return PR ? zero_padded_heads(dt, bs.of(p.dout), 1, L->B, L->NH, L->S, L->d, key_lengths, st) : hipSuccess;
    };

    // FFN2 input: kept by the forward, or (gelu checkpoint) recomputed from u
    // by the FFN2 input-gradient epilogue into scratch
    const void* g_src = gck ? bs.of(p.gck_g) : bs.of(p.g);

    if (c.pre_ln) {
        // y = x1 + drop2(g W2^T + b2); drop2(dy) handed down by the layer above, or made here
        const void* df = dy_dropped;
        if (!df) {
            HIP_TRY(dropout_apply(dt, dyin, bs.of(p.df), (size_t)T * H, d2, st, rmap, H));
            df = bs.of(p.df);
        }
        GemmDesc g = dgrad(df, P->w_2, H, F, gck ? EPI_GELU_BWD : EPI_MUL_AUX);
        g.ea.out = bs.of(p.du); g.ea.ldo = F; g.ea.aux = bs.of(p.u);
        if (gck) g.ea.out2 = bs.of(p.gck_g);
        TIMED(TEL_K_FFN2_DGRAD, gemm_launch(g, st));
        g = dgrad(bs.of(p.du), P->w_1, F, H, EPI_STORE);
        g.ea.out = bs.of(p.dgemm); g.ea.ldo = H;
        TIMED(TEL_K_FFN1_DGRAD, gemm_launch(g, st));
        s = wgrad_pair(TEL_K_FFN2_WGRAD, Wg{df, g_src, H, F, G->w_2, G->b_2},
                       TEL_K_FFN1_WGRAD, Wg{bs.of(p.du), bs.of(p.ln2_out), F, H, G->w_1, G->b_1}, false);
        if (s != TEL_OK) return s;
        // x1 -> LN2: dx1 = dy + LN2'(da2); dz = drop1(dx1)
        LnBwdArgs lb{};
        lb.dtype = dt; lb.T = T; lb.H = H;
        lb.dout = bs.of(p.dgemm);
        lb.src = inv ? bs.of(p.ln2_out) : bs.of(p.res1); lb.src_f32 = inv ? 0 : r32; lb.from_output = inv;
        lb.mu = (const float*)bs.of(p.mu2); lb.rstd = (const float*)bs.of(p.rs2);
        lb.gamma = P->ln2_g; lb.beta = P->ln2_b;
        lb.res = dyin; lb.res_f32 = 0;
        lb.out = bs.of(p.dres); lb.out_f32 = r32;
        lb.drop_out = bs.of(p.dz); lb.drop = d1;
        lb.part_g = part_ln2_g; lb.part_b = part_ln2_b; lb.row_map = rmap;
        TIMED(TEL_K_LN2_BWD, ln_backward(lb, st));
        HIP_TRY(ln_grads(part_ln2_g, part_ln2_b, G->ln2_g, G->ln2_b));
        // out-projection
        g = dgrad(bs.of(p.dz), P->w_o, H, H, EPI_HEADSPLIT);
        g.ea.out = bs.of(p.dout); g.ea.B = L->B; g.ea.S = L->S; g.ea.H = H; g.ea.NH = L->NH; g.ea.d = L->d;
        HIP_TRY(zero_dout());
        TIMED(TEL_K_OUT_DGRAD, gemm_launch(g, st));
        TIMED(TEL_K_ATTN_BWD, attn());
        // QKV projection; the out-projection weight gradient pairs with its
        g = dgrad(bs.of(p.dqkv), P->w_qkv, 3 * H, H, EPI_STORE);
        g.ea.out = bs.of(p.dgemm); g.ea.ldo = H;
        TIMED(TEL_K_QKV_DGRAD, gemm_launch(g, st));
        // x -> LN1: dx = dx1 + LN1'(da1) (ahead of the weight gradients, which
        // do not need it, so that its finalize can ride with their reduction)
        lb = LnBwdArgs{};
        lb.dtype = dt; lb.T = T; lb.H = H;
        lb.dout = bs.of(p.dgemm);
        lb.src = inv ? bs.of(p.ln1_out) : xin; lb.src_f32 = 0; lb.from_output = inv;
        lb.mu = (const float*)bs.of(p.mu1); lb.rstd = (const float*)bs.of(p.rs1);
        lb.gamma = P->ln1_g; lb.beta = P->ln1_b;
        lb.res = bs.of(p.dres); lb.res_f32 = r32;
        lb.out = dxout; lb.out_f32 = 0;
        if (below) {  // the layer below's drop2(dx), from dx as stored
            lb.drop_out = dx_dropped;
            lb.drop = make_drop(below, below->cfg.hidden_dropout, 2, step, training);
        }
        lb.part_g = part_ln1_g; lb.part_b = part_ln1_b; lb.row_map = rmap;
        TIMED(TEL_K_LN1_BWD, ln_backward(lb, st));
        HIP_TRY(ln_grads(part_ln1_g, part_ln1_b, G->ln1_g, G->ln1_b));
        s = wgrad_pair(TEL_K_OUT_WGRAD, Wg{bs.of(p.dz), bs.of(p.ctx), H, H, G->w_o, G->b_o},
                       TEL_K_QKV_WGRAD, Wg{bs.of(p.dqkv), bs.of(p.ln1_out), 3 * H, H, G->w_qkv, G->b_qkv},
                       true);
        if (s != TEL_OK) return s;
    } else {
        // y = LN2(z2): dz2 = LN2'(dy); df = drop2(dz2)
        LnBwdArgs lb{};
        lb.dtype = dt; lb.T = T; lb.H = H;
        lb.dout = dyin;
        lb.src = inv ? bs.of(p.ycopy) : bs.of(p.res2); lb.src_f32 = inv ? 0 : r32; lb.from_output = inv;
        lb.mu = (const float*)bs.of(p.mu2); lb.rstd = (const float*)bs.of(p.rs2);
        lb.gamma = P->ln2_g; lb.beta = P->ln2_b;
        lb.out = bs.of(p.dres2); lb.out_f32 = 1;
        lb.drop_out = bs.of(p.df); lb.drop = d2;
        lb.part_g = part_ln2_g; lb.part_b = part_ln2_b; lb.row_map = rmap;
        TIMED(TEL_K_LN2_BWD, ln_backward(lb, st));
        HIP_TRY(ln_grads(part_ln2_g, part_ln2_b, G->ln2_g, G->ln2_b));
        GemmDesc g = dgrad(bs.of(p.df), P->w_2, H, F, gck ? EPI_GELU_BWD : EPI_MUL_AUX);
        g.ea.out = bs.of(p.du); g.ea.ldo = F; g.ea.aux = bs.of(p.u);
        if (gck) g.ea.out2 = bs.of(p.gck_g);
        TIMED(TEL_K_FFN2_DGRAD, gemm_launch(g, st));
        g = dgrad(bs.of(p.du), P->w_1, F, H, EPI_STORE);
        g.ea.out = bs.of(p.dgemm); g.ea.ldo = H;
        TIMED(TEL_K_FFN1_DGRAD, gemm_launch(g, st));
        s = wgrad_pair(TEL_K_FFN2_WGRAD, Wg{bs.of(p.df), g_src, H, F, G->w_2, G->b_2},
                       TEL_K_FFN1_WGRAD, Wg{bs.of(p.du), bs.of(p.x1e), F, H, G->w_1, G->b_1}, false);
        if (s != TEL_OK) return s;
        // x1 = LN1(z1): dz1 = LN1'(dgemm + dz2); dz = drop1(dz1)
        lb = LnBwdArgs{};
        lb.dtype = dt; lb.T = T; lb.H = H;
        lb.dout = bs.of(p.dgemm); lb.dout_add = (const float*)bs.of(p.dres2);
        lb.src = inv ? (r32 ? bs.of(p.x1f) : bs.of(p.x1e)) : bs.of(p.res1); lb.src_f32 = r32; lb.from_output = inv;
        lb.mu = (const float*)bs.of(p.mu1); lb.rstd = (const float*)bs.of(p.rs1);
        lb.gamma = P->ln1_g; lb.beta = P->ln1_b;
        lb.out = bs.of(p.dres); lb.out_f32 = 1;
        lb.drop_out = bs.of(p.dz); lb.drop = d1;
        lb.part_g = part_ln1_g; lb.part_b = part_ln1_b; lb.row_map = rmap;
        TIMED(TEL_K_LN1_BWD, ln_backward(lb, st));
        HIP_TRY(ln_grads(part_ln1_g, part_ln1_b, G->ln1_g, G->ln1_b));
        g = dgrad(bs.of(p.dz), P->w_o, H, H, EPI_HEADSPLIT);
        g.ea.out = bs.of(p.dout); g.ea.B = L->B; g.ea.S = L->S; g.ea.H = H; g.ea.NH = L->NH; g.ea.d = L->d;
        HIP_TRY(zero_dout());
        TIMED(TEL_K_OUT_DGRAD, gemm_launch(g, st));
        TIMED(TEL_K_ATTN_BWD, attn());
        // dx = dz1 + dqkv W_qkv; the out-projection weight gradient pairs with its
        g = dgrad(bs.of(p.dqkv), P->w_qkv, 3 * H, H, EPI_ADD_RES);
        g.ea.out = dxout; g.ea.ldo = H; g.ea.res = bs.of(p.dres);
        TIMED(TEL_K_QKV_DGRAD, gemm_launch(g, st));
        s = wgrad_pair(TEL_K_OUT_WGRAD, Wg{bs.of(p.dz), bs.of(p.ctx), H, H, G->w_o, G->b_o},
                       TEL_K_QKV_WGRAD, Wg{bs.of(p.dqkv), xin, 3 * H, H, G->w_qkv, G->b_qkv}, true);
        if (s != TEL_OK) return s;
    }
    if (PR) HIP_TRY(scatter_rows(dt, dxout, dx, rinv, L->T, H, st));
    L->pending_fwd--;
    g_err.clear();
    return TEL_OK;
}


tel_status tel_layer_backward(tel_layer* L, const tel_params* P, const void* x, const int32_t* key_lengths,
                              int training, uint64_t step, const void* dy, const void* saved, void* scratch,
                              void* dx, const tel_grads* G, tel_stream_t stream) {
    return backward_impl(L, P, x, key_lengths, training, step, dy, nullptr, saved, scratch, dx, nullptr, nullptr, G,
                         stream);
}

tel_status tel_layer_backward_chain(tel_layer* L, const tel_params* P, const void* x, const int32_t* key_lengths,
                                    int training, uint64_t step, const void* dy, const void* dy_dropped,
                                    const void* saved, void* scratch, void* dx, const tel_layer* below,
                                    void* dx_dropped, const tel_grads* G, tel_stream_t stream) {
    return backward_impl(L, P, x, key_lengths, training, step, dy, dy_dropped, saved, scratch, dx, below,
                         dx_dropped, G, stream);
}

tel_status tel_debug_kernel_events(tel_layer* L, int kernel_id, void** start_events, void** stop_events,
                                   int count) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    if (kernel_id < 0 || count <= 0) {
        L->prof_kernel = -1;
        L->prof_count = 0;
        return TEL_OK;
    }
    if (!start_events || !stop_events) return fail(TEL_ERR_INVALID_ARG, "event arrays are NULL");
    L->prof_kernel = kernel_id;
    L->prof_start = reinterpret_cast<hipEvent_t*>(start_events);
    L->prof_stop = reinterpret_cast<hipEvent_t*>(stop_events);
    L->prof_count = count;
    L->prof_calls = 0;
    return TEL_OK;
}

tel_status tel_debug_dropout_mask(const tel_layer* L, int site, uint64_t step, uint8_t* out_dev, tel_stream_t stream) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    if (!out_dev) return fail(TEL_ERR_INVALID_ARG, "out is NULL");
    if (site < 0 || site > 2) return fail(TEL_ERR_INVALID_ARG, "site must be 0, 1 or 2");
    const float pr = site == 0 ? L->cfg.attn_dropout : L->cfg.hidden_dropout;
    const Drop d = make_drop(L, pr, (uint32_t)site, step, 1);
    const size_t n = site == 0 ? (size_t)L->B * L->NH * L->S * L->S : (size_t)L->T * L->H;
    HIP_TRY(dropout_mask_dump(d, out_dev, n, (hipStream_t)stream));
    return TEL_OK;
}

tel_status tel_layer_forward_noalloc(tel_layer* L, const tel_params* P, const void* x, const int32_t* key_lengths,
                                     void* y, tel_stream_t stream) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    const size_t need = noalloc_need(L);
    if (need > kNoAllocBytes)
        return fail(TEL_ERR_UNSUPPORTED,
                    "this layer's inference forward needs %zu bytes of workspace; the static buffer holds %zu "
                    "(use tel_layer_forward with a caller-owned scratch)",
                    need, kNoAllocBytes);
    void* base = nullptr;
    tel_status s = noalloc_base(&base);
    if (s != TEL_OK) return s;
    return tel_layer_forward(L, P, x, key_lengths, 0, 0, y, nullptr, base, stream);
}

tel_status tel_debug_attn_keep_bits(tel_layer* L, uint32_t* out_dev) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    if (!out_dev) {
        L->dbg_bits = nullptr;
        return TEL_OK;
    }
    if (!aligned(out_dev)) return fail(TEL_ERR_INVALID_ARG, "out_dev not 16-byte aligned");
    if (L->cfg.dtype == TEL_F32 || L->d != 64 || L->S % 64)
        return fail(TEL_ERR_UNSUPPORTED, "keep bits exist only for the MFMA attention (fp16/bf16, head width 64, "
                                         "seq a multiple of 64)");
    L->dbg_bits = out_dev;
    g_err.clear();
    return TEL_OK;
}

tel_status tel_debug_buffer(const tel_layer* L, int which, size_t* offset, size_t* bytes, int* in_saved) {
    if (!L) return fail(TEL_ERR_INVALID_ARG, "layer is NULL");
    if (!offset || !bytes || !in_saved) return fail(TEL_ERR_INVALID_ARG, "output pointers must be non-NULL");
    const Plan& p = L->plan;
    const Buf* b = nullptr;
    switch (which) {
        case TEL_BUF_DROP1_IN: b = &p.dres; break;
        case TEL_BUF_DROP1_OUT: b = &p.dz; break;
        case TEL_BUF_DROP2_IN:
            if (L->cfg.pre_ln) return fail(TEL_ERR_UNSUPPORTED, "Pre-LN: dropout site 2's backward input is dy itself");
            b = &p.dres2;
            break;
        case TEL_BUF_DROP2_OUT: b = &p.df; break;
        case TEL_BUF_ATTN_KEEP_BITS:
            if (!p.abits.used) return fail(TEL_ERR_UNSUPPORTED, "this layer keeps no attention keep bits");
            b = &p.abits;
            break;
        default: return fail(TEL_ERR_INVALID_ARG, "unknown buffer id %d", which);
    }
    *offset = b->off;
    *bytes = b->bytes;
    *in_saved = b->in_saved ? 1 : 0;
    return TEL_OK;
}

tel_status tel_check_key_lengths(const int32_t* host_lengths, int32_t batch, int32_t seq) {
    if (!host_lengths || batch <= 0 || seq <= 0) return fail(TEL_ERR_INVALID_ARG, "bad arguments");
    return check_lengths_host(host_lengths, batch, seq);
}

int32_t tel_debug_checks_enabled(void) {
#ifdef TEL_DEBUG_CHECKS
    return 1;
#else
    return 0;
#endif
}

double tel_pld_theta(double t, double theta_bar, double gamma) {
    return (1.0 - theta_bar) * exp(-gamma * t) + theta_bar;
}

int32_t tel_pld_keep(uint64_t seed, int32_t layer_id, uint64_t step, double theta) {
    // Philox4x32-10 on the host, site 3, element 0
    uint32_t c0 = 0, c1 = 0, c2 = 3u, c3 = (uint32_t)step;
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)layer_id;
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p2 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p2 >> 32) ^ c1 ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        c1 = (uint32_t)p2;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    const double thr = floor(theta * 4294967296.0);
    return (double)c0 < thr ? 1 : 0;
}

}  // extern "C"
