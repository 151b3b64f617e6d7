/*
 * tel.h -- C ABI of the fused Transformer encoder layer for AMD MI355X
 * (gfx950).  One layer, forward and backward, Pre-LN and Post-LN.
 *
 * What the layer computes (per sequence b of length S, hidden H, N heads of
 * width d = H/N, FFN width F):
 *   Pre-LN   x1 = x + Drop1(Attn(LN1(x)) W_o^T + b_o)
 *            y  = x1 + Drop2(GELU(LN2(x1) W_1^T + b_1) W_2^T + b_2)
 *   Post-LN  x1 = LN1(x + Drop1(Attn(x) W_o^T + b_o))
 *            y  = LN2(x1 + Drop2(GELU(x1 W_1^T + b_1) W_2^T + b_2))
 *   Attn(a): [Q|K|V] = a W_qkv^T + b_qkv (fused projection, rows of W_qkv
 *            stacked Q,K,V; head h = columns h*d..h*d+d-1 of each),
 *            P = softmax(Q K^T / sqrt(d)) over the valid keys j < len[b]
 *            (padded keys weigh exactly 0), context = Drop0(P) V, heads
 *            merged back to [token, H].
 * Sources: the op order of an encoder layer and the fusion of linear+bias+
 * activation are from "Forward computation-graph optimisation in the
 * Transformer" (sections 2 and 4); the config fields, Pre-/Post-LN switch,
 * LayerNorm epsilon, FFN default width and the three memory-saving switches
 * are from the DeepSpeed Transformer Kernel guide ("Step 2: configuration
 * parameters", "Step 3: memory-saving switches"); the fused QKV projection,
 * head split, 1/sqrt(d) scale, exact GELU and inverted dropout are from the
 * AI-infra blog (sections 2.1, 2.3 and 5.1); attention itself from the
 * deployment article's pseudo-code ("1. matrix-operation restructuring").
 *
 * Dropout (inverted: kept value * 1/(1-p)) draws its bits from
 * Philox4x32-10 (Salmon et al., SC'11): key = (seed mod 2^32, layer_id),
 * counter = (floor(e/8) low, floor(e/8) high, site, step mod 2^32); one
 * call serves the 8 elements 8g .. 8g+7, element e taking the 16-bit half
 * (e mod 2) of output word (e/2 mod 4), and it is dropped iff that value
 * < floor(p * 2^16) with p the fp32 value in tel_config.  The realised drop
 * probability is therefore q = floor(p * 2^16) / 2^16 (q <= p < q + 2^-16;
 * p = 0.1f gives q = 6553/65536 = 0.0999908), and a kept value times 1/(1-p)
 * has mean (1-q)/(1-p) = 1 + (p-q)/(1-p) times the input (1.00001 at
 * p = 0.1f).  Probabilities in (0, 2^-16), which would realise q = 0, are
 * rejected with TEL_ERR_UNSUPPORTED.  Sites: 0 attention
 * probabilities, element e = ((b*N + h)*S + i)*S + j; 1 attention-branch
 * output, 2 FFN-branch output, element e = t*H + c with token t = b*S + s;
 * 3 the progressive layer-drop gate (output word 0 of block 0, compared as
 * a 32-bit value with floor(theta * 2^32)).  Masks are a pure function of
 * (seed, layer_id, site, step, e).  For seq <= 128 the forward keeps the
 * attention keep bits (1 bit per score, in saved) unless
 * attn_dropout_checkpoint is set; longer sequences, and that switch, make
 * the backward regenerate them, so nothing kept grows with seq^2.
 * Hidden-dropout bits are always regenerated.  Every switch setting
 * therefore sees identical masks.
 *
 * Data layout: row-major, token-major activations [B*S, H] with t = b*S+s;
 * weights in nn.Linear layout W[out, in].  Params, activations and grads
 * all have dtype cfg.dtype; accumulation, softmax and LayerNorm statistics
 * are fp32.  Every pointer must be 16-byte aligned.
 *
 * Ownership: the caller owns every device buffer (x, y, params, grads,
 * saved, scratch, key_lengths); the library owns only the opaque host handle
 * and never allocates device memory.  No device pointer is retained across
 * calls.  All work is enqueued on the caller's stream; no call blocks the
 * host or synchronises the device.
 *
 * Errors: every argument is validated on the host before any HIP call, so
 * invalid input returns TEL_ERR_INVALID_ARG / TEL_ERR_UNSUPPORTED without
 * touching the GPU.  A failed kernel launch returns TEL_ERR_HIP.  The message
 * for the last non-OK status of the calling thread is tel_last_error().
 * Nothing aborts or throws across this interface.  The device key_lengths
 * are not read on the host: values outside [1, seq] give wrong results (but
 * no out-of-bounds access) in the release library; the debug library
 * (built with TEL_DEBUG_CHECKS, libtel_debug.so) copies them to the host at
 * every forward and backward and returns TEL_ERR_INVALID_ARG instead.
 *
 * Differences from the interface first planned for this layer: the backward
 * takes x, key_lengths, training and step again (the forward keeps no
 * pointers, and dropout masks are regenerated from them); tel_pld_keep
 * returns int32_t; tel_config orders its fields as below and adds
 * pack_tokens; token packing, the chained Pre-LN backward, the kernel-event
 * hook, the debug buffer hooks and tel_check_key_lengths are additions.
 */
#ifndef TEL_H
#define TEL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* tel_stream_t; /* hipStream_t; NULL = default stream */

typedef enum { TEL_F32 = 0, TEL_F16 = 1, TEL_BF16 = 2 } tel_dtype;

typedef enum {
    TEL_OK = 0,
    TEL_ERR_INVALID_ARG = -1, /* bad shape, probability, pointer or alignment */
    TEL_ERR_UNSUPPORTED = -2, /* valid but not implemented (e.g. head width) */
    TEL_ERR_STATE = -3,       /* backward without a forward that saved state */
    TEL_ERR_HIP = -4          /* a HIP call or kernel launch failed */
} tel_status;

/* Layer configuration; shapes are fixed at creation (DeepSpeed Transformer
 * Kernel guide, "Step 2": batch_size is the per-GPU micro-batch,
 * max_seq_length the sequence length). */
typedef struct {
    int32_t batch, seq, hidden, heads;
    int32_t ffn;                   /* <= 0 selects 4*hidden */
    float attn_dropout;            /* site 0 probability, in [0,1) */
    float hidden_dropout;          /* sites 1 and 2 probability, in [0,1) */
    int32_t pre_ln;                /* 1 Pre-LN, 0 Post-LN */
    uint64_t seed;                 /* dropout key word 0 (low 32 bits used) */
    int32_t layer_id;              /* dropout key word 1 */
    int32_t dtype;                 /* tel_dtype */
    float ln_eps;                  /* LayerNorm epsilon (the guide's default 1e-12) */
    int32_t attn_dropout_checkpoint; /* do not keep the attention keep bits (1 bit per score);
                                        backward regenerates them from the RNG */
    int32_t normalize_invertible;  /* LN backward from the LN output; drops the LN inputs */
    int32_t gelu_checkpoint;       /* keep the GELU input only; recompute GELU in backward */
    int32_t pack_tokens;           /* run the layer on the valid tokens only (see
                                      tel_layer_set_valid_tokens) */
    int32_t stochastic_mode;       /* relaxed determinism for speed (the DeepSpeed guide's
                                      stochastic_mode switch): the grouped weight-gradient
                                      launches add their k-splits into the zeroed gradients
                                      with packed fp16/bf16 atomics instead of reducing fp32
                                      partials in fixed order.  Those weight and bias
                                      gradients then carry one dtype rounding per split, and
                                      with more than two splits their last bits may differ
                                      from run to run; every other output keeps its bits.
                                      0 (default): every output is bitwise reproducible. */
} tel_config;

/* The twelve parameters, nn.Linear layout, dtype cfg.dtype, device memory:
 * w_qkv [3H,H], b_qkv [3H], w_o [H,H], b_o [H], ln1_g/ln1_b [H],
 * w_1 [F,H], b_1 [F], w_2 [H,F], b_2 [H], ln2_g/ln2_b [H]. */
typedef struct {
    const void *w_qkv, *b_qkv, *w_o, *b_o, *ln1_g, *ln1_b;
    const void *w_1, *b_1, *w_2, *b_2, *ln2_g, *ln2_b;
} tel_params;

/* Gradients, same shapes and dtype; OVERWRITTEN (not accumulated). */
typedef struct {
    void *w_qkv, *b_qkv, *w_o, *b_o, *ln1_g, *ln1_b;
    void *w_1, *b_1, *w_2, *b_2, *ln2_g, *ln2_b;
} tel_grads;

typedef struct tel_layer tel_layer;

/* Validate cfg and create a handle (host memory only).  Supported: dims
 * multiples of 16, hidden <= 2048, head width d in {16,32,64,128}, H % N == 0, dtype f32,
 * f16 or bf16.  *out is set to NULL on failure. */
tel_status tel_layer_create(const tel_config* cfg, tel_layer** out);

/* Bytes of the two caller-provided device workspaces:
 *   saved   -- activations written by forward and read by the matching
 *              backward; must stay unmodified in between;
 *   scratch -- temporaries of one call; may be reused by any later call on
 *              the same stream (shared by all layers of a stack). */
tel_status tel_layer_workspace_bytes(const tel_layer* layer, size_t* saved_bytes, size_t* scratch_bytes);

/* Forward.  x [B*S,H] in, y [B*S,H] out (may not alias x).  key_lengths:
 * device int32 [B], valid length of each sequence in [1,S] (NULL: all S).
 * training = 0 disables dropout.  step is the dropout counter word.
 * saved may be NULL (inference): the activations then live in scratch,
 * which must hold saved_bytes + scratch_bytes (rounded up to 256), and no
 * backward may follow.  scratch is always required. */
tel_status tel_layer_forward(tel_layer* layer, const tel_params* params, const void* x,
                             const int32_t* key_lengths, int training, uint64_t step, void* y,
                             void* saved, void* scratch, tel_stream_t stream);

/* Backward of the most recent forward that had a saved buffer.  x,
 * key_lengths, training and step must equal the forward's (x may be NULL
 * for Pre-LN with normalize_invertible, where it is not read).  dy [B*S,H]
 * in; dx [B*S,H] and all twelve grads out.  Returns TEL_ERR_STATE if no
 * forward with saved state preceded it. */
tel_status tel_layer_backward(tel_layer* layer, const tel_params* params, const void* x,
                              const int32_t* key_lengths, int training, uint64_t step, const void* dy,
                              const void* saved, void* scratch, void* dx, const tel_grads* grads,
                              tel_stream_t stream);

/* Backward through a stack of Pre-LN layers, with the hidden dropout of each
 * layer's FFN branch (DS guide: the layer's hidden_dropout_ratio; AI-infra
 * blog section 5.1: mask / (1-p)) applied where the gradient is made.  In a
 * Pre-LN layer y = x1 + drop2(FFN(LN2(x1))), so the backward needs both dy
 * and drop2(dy); the layer above produces dy = its dx in its LayerNorm-1
 * backward, and can apply this layer's mask in the same pass instead of a
 * separate pass over dy here.  As tel_layer_backward, plus:
 *   dy_dropped -- drop2(dy) with this layer's site-2 mask and 1/(1-p), as
 *                 the layer above's call wrote it into its dx_dropped, or
 *                 NULL (then computed here from dy);
 *   below      -- the next layer down the stack (the one whose input
 *                 gradient dx is), or NULL;
 *   dx_dropped -- [B*S,H] out, required iff below is set: below's site-2
 *                 mask and 1/(1-p) applied to dx as stored (dx rounded to
 *                 the dtype), i.e. the dy_dropped of below's backward.  The
 *                 mask is below's (its seed and layer id) at this call's step
 *                 and training flag, so below's forward and backward must use
 *                 the same step and training.
 * Every output equals tel_layer_backward's bit for bit.  TEL_ERR_INVALID_ARG
 * for a Post-LN layer (site 2 there follows its own LayerNorm backward and is
 * fused already), below without dx_dropped or vice versa, or a below that is
 * not a Pre-LN layer of the same batch, sequence, hidden size, dtype and
 * hidden dropout, or a dx_dropped equal to dy, dy_dropped or dx;
 * TEL_ERR_UNSUPPORTED under token packing. */
tel_status tel_layer_backward_chain(tel_layer* layer, const tel_params* params, const void* x,
                                    const int32_t* key_lengths, int training, uint64_t step, const void* dy,
                                    const void* dy_dropped, const void* saved, void* scratch, void* dx,
                                    const tel_layer* below, void* dx_dropped, const tel_grads* grads,
                                    tel_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * inference forward (training = 0, nothing kept for a backward) of
 * tel_layer_forward, with its workspace in a static device array of the
 * library instead of a caller-owned scratch.  The array holds
 * TEL_NOALLOC_MAX_BYTES (64 MiB) per device, reserved by the library on each
 * device it runs on until the process ends; a layer whose inference forward
 * needs more (its forward temporaries plus saved_bytes, e.g. BERT-Large
 * shapes beyond about 1900 tokens) gets TEL_ERR_UNSUPPORTED before any GPU
 * work.  Calls no hipMalloc / hipFree.  No kernel of that forward needs the
 * workspace zeroed; it keeps the last call's contents.  Every call on one
 * device shares its array: calls that overlap on one device (other streams,
 * other threads) race and must be serialised by the caller.  x, key_lengths
 * and y as in tel_layer_forward; y is identical to tel_layer_forward's with
 * training = 0. */
#define TEL_NOALLOC_MAX_BYTES (64ull << 20)
tel_status tel_layer_forward_noalloc(tel_layer* layer, const tel_params* params, const void* x,
                                     const int32_t* key_lengths, void* y, tel_stream_t stream);

/* Token packing (pack_tokens = 1): work on padding tokens is skipped, the
 * cost the AI-infra blog describes for padded batches (sections 2.1 and 4.2,
 * dynamic padding and length bucketing).  Declares that the next forward
 * and its backward see key_lengths summing to valid_tokens (0 or B*S: no
 * packing).  The layer then gathers the valid tokens b*S + s (s < len[b])
 * into consecutive rows, rounded up to a multiple of 256 with zero filler
 * rows, and runs LayerNorm, the projections and the FFN on those rows only;
 * attention keeps its per-sequence layout.  Results at valid tokens are the
 * unpacked layer's (dropout masks keep their padded element index); y and dx
 * are zero at padding tokens, and dy there is ignored (the gradient of a
 * loss that does not read padding outputs).  Requires the MFMA attention
 * (fp16/bf16, head width 64, S a multiple of 64).  valid_tokens must equal
 * the sum of the device key_lengths of those calls; it is not checked on the
 * device (a mismatch gives wrong values, never an out-of-bounds access).
 * Returns TEL_ERR_INVALID_ARG if valid_tokens is outside [0, B*S], and
 * TEL_ERR_UNSUPPORTED if the layer was not created with pack_tokens or its
 * attention cannot run packed. */
tel_status tel_layer_set_valid_tokens(tel_layer* layer, int64_t valid_tokens);

/* Free the handle.  NULL is accepted. */
tel_status tel_layer_destroy(tel_layer* layer);

/* Thread-local message describing the last non-OK status ("" if none). */
const char* tel_last_error(void);

/* Test hook: write the keep bits (1 keep, 0 drop) of dropout site 0, 1 or 2
 * for the whole layer at this step into out_dev (device uint8; B*N*S*S
 * bytes for site 0, B*S*H bytes for sites 1 and 2), computed by the same
 * device generator the kernels use. */
tel_status tel_debug_dropout_mask(const tel_layer* layer, int site, uint64_t step, uint8_t* out_dev,
                                  tel_stream_t stream);

/* Kernel ids of one layer's launches, for tel_debug_kernel_events. */
enum {
    TEL_K_LN1_FWD = 0, TEL_K_QKV_FWD = 1, TEL_K_ATTN_FWD = 2, TEL_K_OUT_FWD = 3, TEL_K_LN2_FWD = 4,
    TEL_K_FFN1_FWD = 5, TEL_K_FFN2_FWD = 6,
    TEL_K_FFN2_DGRAD = 10, TEL_K_FFN2_WGRAD = 11, TEL_K_FFN1_DGRAD = 12, TEL_K_FFN1_WGRAD = 13,
    TEL_K_LN2_BWD = 14, TEL_K_OUT_DGRAD = 15, TEL_K_OUT_WGRAD = 16, TEL_K_ATTN_BWD = 17,
    TEL_K_QKV_DGRAD = 18, TEL_K_QKV_WGRAD = 19, TEL_K_LN1_BWD = 20,
    /* the grouped weight-gradient kernel launches (W_2 with W_1, W_o with
       W_qkv), and the launch after each: its split-K reduction and, for the
       last, the LayerNorm gamma/beta sums (events back to back where the
       pair needs no such launch); only where the pair runs grouped */
    TEL_K_FFN_WGRAD_PAIR = 21, TEL_K_ATTN_WGRAD_PAIR = 22,
    TEL_K_FFN_WGRAD_REDUCE = 23, TEL_K_ATTN_WGRAD_REDUCE = 24
};

/* Benchmark hook: from now on, every launch of kernel kernel_id (a TEL_K_*
 * id) by this layer is bracketed on its stream by hipEventRecord of
 * start_events[i % count] and stop_events[i % count] (hipEvent_t handles the
 * caller created), i counting the launches since this call.  The arrays are
 * borrowed until the hook is disabled with kernel_id < 0.  Results are
 * unchanged, except that a weight-gradient pair that otherwise runs as one
 * grouped launch runs as two launches while one of its single ids
 * (TEL_K_*_WGRAD) is profiled: those two weight gradients and their bias
 * gradients may then take another k-split and round differently (every other
 * output keeps its bits).  The pair ids time the grouped GEMM kernel alone,
 * the reduce ids the launch that follows it. */
tel_status tel_debug_kernel_events(tel_layer* layer, int kernel_id, void** start_events, void** stop_events,
                                   int count);

/* Test hook: the next training forward of this layer (with attention
 * dropout on) also writes the attention keep bits it applies to out_dev:
 * device uint32 [B][N][S][S/32], bit j%32 of word j/32 of query row
 * (b, h, i) set iff key j is kept; words of 32-key groups at or beyond
 * len[b] are not written.  One-shot; out_dev NULL disarms it.  The bits are
 * written by the attention kernel itself (copied from saved where the layer
 * keeps them), so they are the mask the forward applied.
 * TEL_ERR_UNSUPPORTED unless the MFMA attention runs (fp16/bf16, head width
 * 64, seq a multiple of 64). */
tel_status tel_debug_attn_keep_bits(tel_layer* layer, uint32_t* out_dev);

/* Internal buffers a test may read after a call (their contents last until
 * the next call that uses the same saved / scratch buffer).  Rows are the
 * layer's rows: tokens, or packed rows under token packing. */
enum {
    TEL_BUF_DROP1_IN = 0,   /* scratch, fp32 [T,H] (the storage dtype for Pre-LN fp16 layers):
                               gradient reaching dropout site 1 in the backward (Pre-LN dx1,
                               Post-LN dz1) */
    TEL_BUF_DROP1_OUT = 1,  /* scratch, dtype [T,H]: the same after site 1's mask and 1/(1-p) */
    TEL_BUF_DROP2_IN = 2,   /* scratch, fp32 [T,H]: Post-LN dz2 reaching site 2 (Pre-LN: it is dy,
                               TEL_ERR_UNSUPPORTED) */
    TEL_BUF_DROP2_OUT = 3,  /* scratch, dtype [T,H]: gradient after site 2's mask and 1/(1-p) */
    TEL_BUF_ATTN_KEEP_BITS = 4 /* saved: the forward's attention keep bits (layout as in
                               tel_debug_attn_keep_bits), where the layer keeps them */
};
/* Offset (bytes) and size of buffer `which` within saved (*in_saved = 1) or
 * scratch (*in_saved = 0).  TEL_ERR_UNSUPPORTED if this layer has no such
 * buffer. */
tel_status tel_debug_buffer(const tel_layer* layer, int which, size_t* offset, size_t* bytes, int* in_saved);

/* Host-side check that host_lengths[0..batch-1] all lie in [1, seq]:
 * TEL_OK or TEL_ERR_INVALID_ARG naming the first bad entry.  The debug
 * library runs it on a host copy of the device key_lengths. */
tel_status tel_check_key_lengths(const int32_t* host_lengths, int32_t batch, int32_t seq);

/* 1 in the debug library (TEL_DEBUG_CHECKS), else 0. */
int32_t tel_debug_checks_enabled(void);

/* Progressive layer dropping (PLD page, "core mechanism": theta(t) =
 * (1 - theta_bar) exp(-gamma t) + theta_bar).  Host-only, pure functions.
 * tel_pld_keep returns 1 iff layer layer_id runs at this step: the site-3
 * Philox word for element 0 is < floor(theta * 2^32). */
double tel_pld_theta(double t, double theta_bar, double gamma);
int32_t tel_pld_keep(uint64_t seed, int32_t layer_id, uint64_t step, double theta);

#ifdef __cplusplus
}
#endif
#endif /* TEL_H */
