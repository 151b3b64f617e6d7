/*
 * oracle.c -- plain fp64 reference of one Transformer encoder layer,
 * forward and backward, Pre-LN and Post-LN.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this file's library.  The GPU
 * product path never calls it, and this file includes nothing from the GPU
 * path (no shared headers, helpers, tables or constants).
 *
 * Everything is written from the definitions, in the order the pages state
 * them, with no tiling, no online softmax and no fusion:
 *
 *  - Layer op order (QKV projection, scaled dot-product attention, output
 *    projection, residual + LayerNorm, FFN, residual + LayerNorm): the
 *    computation-graph page ("Forward computation-graph optimisation in the
 *    Transformer", section 2, main computation modules).  That order is the
 *    Post-LN layer.  Pre-LN (LayerNorm before each sublayer, residual added
 *    after, no final LayerNorm inside the layer) is the variant the DeepSpeed
 *    Transformer Kernel guide selects with pre_layer_norm (section "Step 2:
 *    configuration parameters") and the one the PLD page builds on.
 *  - Attention softmax(Q K^T / sqrt(d_k)) V per head: the deployment article
 *    ("Transformer deployment: from model design to GPU utilisation",
 *    section "1. matrix-operation restructuring", attention pseudo-code) and
 *    the AI-infra blog, section 5.1 (scale as a range guard).
 *  - Fused QKV projection Linear(D, 3D), rows stacked Q,K,V; head h uses
 *    columns h*d..h*d+d-1 of each: AI-infra blog, section 2.1, steps 2 and 3.
 *  - Inverted dropout, kept value * 1/(1-p): AI-infra blog, section 5.1
 *    (dropout_p).  Attention dropout on the probabilities; hidden dropout on
 *    each sublayer output before the residual add.
 *  - LayerNorm epsilon 1e-12 and FFN width 4H default: DeepSpeed Transformer
 *    Kernel guide, "Step 2", extra constructor parameters.
 *  - GELU in its exact erf form: AI-infra blog, section 2.3 (exact GELU).
 *  - PLD schedule theta(t) = (1-theta_bar) exp(-gamma t) + theta_bar: PLD
 *    page, section "core mechanism: theta, gamma and the schedule formula".
 *  - Dropout random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 *    "Parallel random numbers: as easy as 1, 2, 3", SC'11), written here from
 *    the paper's description of the round function and key schedule.
 *
 * Readings where the pages are silent (mask convention, dropout sites, RNG
 * counter layout, rounding) are listed in the project's design notes; the
 * functions below state the reading they implement.
 *
 * Build: gcc -O3 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 * (no fast-math: every sum keeps its written order)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#else
static int omp_get_num_threads(void) { return 1; }
#endif

#define ORC_OK 0
#define ORC_ERR (-1)

typedef struct {
    int32_t batch, seq, hidden, heads, ffn;
    int32_t pre_ln;        /* 1 Pre-LN, 0 Post-LN */
    int32_t training;      /* 0: dropout off */
    int32_t batch_offset;  /* global index of local sequence 0 (RNG element index) */
    double attn_p, hidden_p, ln_eps;
    uint64_t seed;
    uint64_t step;
    int32_t layer_id;
    int32_t pad_;
} orc_cfg;

typedef struct {
    const double *w_qkv, *b_qkv, *w_o, *b_o, *ln1_g, *ln1_b;
    const double *w_1, *b_1, *w_2, *b_2, *ln2_g, *ln2_b;
} orc_params;

typedef struct {
    double *w_qkv, *b_qkv, *w_o, *b_o, *ln1_g, *ln1_b;
    double *w_1, *b_1, *w_2, *b_2, *ln2_g, *ln2_b;
} orc_grads;

/* Intermediate activations.  Pre-LN: ln1_in = x, ln1_out = LN1(x),
 * ln2_in = x1, ln2_out = LN2(x1), y = x1 + drop(ffn).  Post-LN: ln1_in = z1,
 * ln1_out = x1, ln2_in = z2, ln2_out = y.  Any pointer may be NULL. */
typedef struct {
    double *qkv;       /* [T,3H] token-major projection output */
    double *ctx;       /* [T,H] head-merged attention output */
    double *lse;       /* [B,N,S] log-sum-exp of scaled scores (valid keys) */
    double *attn_proj; /* [T,H] ctx W_o^T + b_o, before dropout */
    double *ln1_in, *ln1_out, *mu1, *rstd1;
    double *u;         /* [T,F] FFN1 output (GELU input) */
    double *g;         /* [T,F] GELU(u) */
    double *ffn_out;   /* [T,H] g W_2^T + b_2, before dropout */
    double *ln2_in, *ln2_out, *mu2, *rstd2;
} orc_acts;

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (SC'11).  Round: two 32x32->64 multiplies of counter words
 * 0 and 2 by the round multipliers; the new counter is
 * (hi(c2*M1) ^ c1 ^ k0, lo(c2*M1), hi(c0*M0) ^ c3 ^ k1, lo(c0*M0)); the key
 * is bumped by the Weyl constants between rounds. */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)c0 * PHILOX_M0;
        uint64_t p1 = (uint64_t)c2 * PHILOX_M1;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        if (r != 9) { k0 += PHILOX_W0; k1 += PHILOX_W1; }
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Philox output word w of counter block g of one site:
 * key = (seed mod 2^32, layer_id); counter = (g low, g high, site,
 * step mod 2^32). */
static uint32_t rng_block_word(uint64_t seed, int32_t layer, uint32_t site, uint64_t step, uint64_t g, int w)
{
    uint32_t ctr[4] = { (uint32_t)g, (uint32_t)(g >> 32), site, (uint32_t)step };
    uint32_t key[2] = { (uint32_t)seed, (uint32_t)layer };
    uint32_t out[4];
    orc_philox4x32_10(ctr, key, out);
    return out[w];
}

/* 16-bit random value of logical element e of a dropout site: one Philox
 * call (128 bits) serves 8 consecutive elements; element e takes word
 * (e/2) mod 4 of block floor(e/8), low half for even e, high half for odd. */
static uint32_t rng_half(uint64_t seed, int32_t layer, uint32_t site, uint64_t step, uint64_t e)
{
    const uint32_t w = rng_block_word(seed, layer, site, step, e >> 3, (int)((e >> 1) & 3));
    return (e & 1) ? (w >> 16) : (w & 0xFFFFu);
}

/* An element is dropped iff its 16-bit value < floor(p * 2^16), so the
 * realised drop probability is floor(p * 2^16) / 2^16; a p in (0, 2^-16)
 * would realise none and is rejected by check_cfg. */
static uint64_t drop_threshold(double p)
{
    if (!(p > 0.0)) return 0;
    return (uint64_t)floor(p * 65536.0);
}

uint64_t orc_drop_threshold(double p) { return drop_threshold(p); }

/* Threads an OpenMP parallel region of this library runs with. */
int orc_omp_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

static int keep_elem(uint64_t seed, int32_t layer, uint32_t site, uint64_t step, uint64_t e, uint64_t thr)
{
    if (thr == 0) return 1;
    return (uint64_t)rng_half(seed, layer, site, step, e) >= thr;
}

/* Dump keep bits (1 keep, 0 drop) for elements e0 .. e0+n-1 of one site. */
void orc_dropout_mask(uint64_t seed, int32_t layer, uint32_t site, uint64_t step, double p,
                      uint64_t e0, uint64_t n, uint8_t *out)
{
    uint64_t thr = drop_threshold(p);
    #pragma omp parallel for schedule(static)
    for (long long i = 0; i < (long long)n; ++i)
        out[i] = (uint8_t)keep_elem(seed, layer, site, step, e0 + (uint64_t)i, thr);
}

/* PLD (site 3, element 0).  theta(t) from the PLD page's schedule formula;
 * the layer is kept iff its word < floor(theta * 2^32) (theta = 1 keeps all). */
double orc_pld_theta(double t, double theta_bar, double gamma)
{
    return (1.0 - theta_bar) * exp(-gamma * t) + theta_bar;
}

int orc_pld_keep(uint64_t seed, int32_t layer, uint64_t step, double theta)
{
    uint64_t thr = (uint64_t)floor(theta * 4294967296.0);
    return (uint64_t)rng_block_word(seed, layer, 3u, step, 0, 0) < thr;
}

/* ------------------------------------------------------------------ */
/* GELU, exact form: u * Phi(u); derivative Phi(u) + u * phi(u). */
double orc_gelu(double u) { return 0.5 * u * (1.0 + erf(u / sqrt(2.0))); }
double orc_gelu_grad(double u)
{
    const double inv_sqrt_2pi = 0.39894228040143267794;
    return 0.5 * (1.0 + erf(u / sqrt(2.0))) + u * inv_sqrt_2pi * exp(-0.5 * u * u);
}

/* ------------------------------------------------------------------ */
/* LayerNorm over the last dimension: biased variance, rstd = 1/sqrt(var+eps),
 * affine after normalising. */
void orc_ln_forward(int T, int H, const double *x, const double *gam, const double *bet,
                    double eps, double *y, double *mu, double *rstd)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *xr = x + (size_t)t * H;
        double m = 0.0;
        for (int c = 0; c < H; ++c) m += xr[c];
        m /= H;
        double v = 0.0;
        for (int c = 0; c < H; ++c) v += (xr[c] - m) * (xr[c] - m);
        v /= H;
        double r = 1.0 / sqrt(v + eps);
        for (int c = 0; c < H; ++c) y[(size_t)t * H + c] = (xr[c] - m) * r * gam[c] + bet[c];
        if (mu) mu[t] = m;
        if (rstd) rstd[t] = r;
    }
}

/* LayerNorm backward.  dy: gradient w.r.t. the LN output.  The normalised
 * value xhat comes from the LN input (from_output = 0: xhat = (x-mu)*rstd)
 * or, for the invertible mode, from the LN output (from_output = 1:
 * xhat = (y-beta)/gamma).  dx is OVERWRITTEN; dgam/dbet are OVERWRITTEN. */
void orc_ln_backward(int T, int H, const double *dy, const double *src, int from_output,
                     const double *mu, const double *rstd, const double *gam, const double *bet,
                     double *dx, double *dgam, double *dbet)
{
    double *xhat = (double *)malloc(sizeof(double) * (size_t)T * H);
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int c = 0; c < H; ++c) {
            double s = src[(size_t)t * H + c];
            xhat[(size_t)t * H + c] = from_output ? (s - bet[c]) / gam[c] : (s - mu[t]) * rstd[t];
        }
    }
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        double mg = 0.0, mgx = 0.0;
        for (int c = 0; c < H; ++c) {
            double gh = dy[(size_t)t * H + c] * gam[c];
            mg += gh;
            mgx += gh * xhat[(size_t)t * H + c];
        }
        mg /= H; mgx /= H;
        for (int c = 0; c < H; ++c) {
            double gh = dy[(size_t)t * H + c] * gam[c];
            dx[(size_t)t * H + c] = rstd[t] * (gh - mg - xhat[(size_t)t * H + c] * mgx);
        }
    }
    if (dgam || dbet) {
        #pragma omp parallel for schedule(static)
        for (int c = 0; c < H; ++c) {
            double sg = 0.0, sb = 0.0;
            for (int t = 0; t < T; ++t) {
                sg += dy[(size_t)t * H + c] * xhat[(size_t)t * H + c];
                sb += dy[(size_t)t * H + c];
            }
            if (dgam) dgam[c] = sg;
            if (dbet) dbet[c] = sb;
        }
    }
    free(xhat);
}

/* ------------------------------------------------------------------ */
/* nn.Linear: Y[t][o] = b[o] + sum_i X[t][i] W[o][i]. */
static void linear_fwd(int T, int in, int out, const double *X, const double *W, const double *b, double *Y)
{
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int o = 0; o < out; ++o) {
            double s = b ? b[o] : 0.0;
            const double *xr = X + (size_t)t * in, *wr = W + (size_t)o * in;
            for (int i = 0; i < in; ++i) s += xr[i] * wr[i];
            Y[(size_t)t * out + o] = s;
        }
}

/* Linear backward: dX = dY W (overwrite, if dX), dW = dY^T X, db = sum_t dY.
 * Each output element is accumulated over its reduction index in ascending
 * order; the loops are nested so that the innermost one walks rows. */
static void linear_bwd(int T, int in, int out, const double *dY, const double *X, const double *W,
                       double *dX, double *dW, double *db)
{
    if (dX) {
        #pragma omp parallel for schedule(static)
        for (int t = 0; t < T; ++t) {
            double *dx = dX + (size_t)t * in;
            for (int i = 0; i < in; ++i) dx[i] = 0.0;
            for (int o = 0; o < out; ++o) {
                const double a = dY[(size_t)t * out + o];
                const double *w = W + (size_t)o * in;
                for (int i = 0; i < in; ++i) dx[i] += a * w[i];
            }
        }
    }
    if (dW) {
        #pragma omp parallel for schedule(static)
        for (int o = 0; o < out; ++o) {
            double *dw = dW + (size_t)o * in;
            for (int i = 0; i < in; ++i) dw[i] = 0.0;
            for (int t = 0; t < T; ++t) {
                const double a = dY[(size_t)t * out + o];
                const double *x = X + (size_t)t * in;
                for (int i = 0; i < in; ++i) dw[i] += a * x[i];
            }
        }
    }
    if (db) {
        #pragma omp parallel for schedule(static)
        for (int o = 0; o < out; ++o) {
            double s = 0.0;
            for (int t = 0; t < T; ++t) s += dY[(size_t)t * out + o];
            db[o] = s;
        }
    }
}

/* ------------------------------------------------------------------ */
/* Attention.  Key j of sequence b is valid iff j < len[b]; an invalid key
 * has weight exactly 0.  Query rows at padded positions are computed like
 * any other row.  Attention dropout (site 0) multiplies the normalised
 * probability P[i][j] by keep/(1-p); its element index is
 * ((b_global*N + h)*S + i)*S + j. */
typedef struct {
    int B, S, H, N, d;
    const int *len;
    int training, boff;
    double pa;
    uint64_t seed, step;
    int32_t layer;
} attn_ctx;

static void attn_row_probs(const attn_ctx *a, const double *qkv, int b, int h, int i, double *P, double *lse)
{
    const int S = a->S, H = a->H, d = a->d, L = a->len[b];
    const double scale = 1.0 / sqrt((double)d);
    const double *q = qkv + ((size_t)(b * S + i)) * 3 * H + (size_t)h * d;
    double m = -INFINITY;
    for (int j = 0; j < S; ++j) {
        if (j < L) {
            const double *k = qkv + ((size_t)(b * S + j)) * 3 * H + H + (size_t)h * d;
            double s = 0.0;
            for (int c = 0; c < d; ++c) s += q[c] * k[c];
            P[j] = s * scale;
            if (P[j] > m) m = P[j];
        } else {
            P[j] = -INFINITY;
        }
    }
    double z = 0.0;
    for (int j = 0; j < S; ++j) {
        P[j] = (j < L) ? exp(P[j] - m) : 0.0;
        z += P[j];
    }
    for (int j = 0; j < S; ++j) P[j] /= z;
    if (lse) *lse = m + log(z);
}

static double attn_drop_factor(const attn_ctx *a, uint64_t thr, double sd, int b, int h, int i, int j)
{
    if (!a->training || thr == 0) return 1.0;
    uint64_t e = (((uint64_t)(a->boff + b) * a->N + h) * a->S + i) * (uint64_t)a->S + j;
    return keep_elem(a->seed, a->layer, 0u, a->step, e, thr) ? sd : 0.0;
}

/* Forward: ctx [T,H] head-merged; lse [B,N,S]; P_out [B,N,S,S] (pre-dropout
 * probabilities) if non-NULL. */
static void attn_fwd(const attn_ctx *a, const double *qkv, double *ctx, double *lse, double *P_out)
{
    const int B = a->B, S = a->S, H = a->H, N = a->N, d = a->d;
    const uint64_t thr = drop_threshold(a->pa);
    const double sd = 1.0 / (1.0 - a->pa);
    #pragma omp parallel
    {
        double *P = (double *)malloc(sizeof(double) * S);
        #pragma omp for schedule(static) collapse(3)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < N; ++h)
                for (int i = 0; i < S; ++i) {
                    double l;
                    attn_row_probs(a, qkv, b, h, i, P, &l);
                    if (lse) lse[((size_t)b * N + h) * S + i] = l;
                    if (P_out) memcpy(P_out + (((size_t)b * N + h) * S + i) * S, P, sizeof(double) * S);
                    double *o = ctx + ((size_t)(b * S + i)) * H + (size_t)h * d;
                    for (int c = 0; c < d; ++c) o[c] = 0.0;
                    for (int j = 0; j < S; ++j) {
                        double w = P[j] * attn_drop_factor(a, thr, sd, b, h, i, j);
                        if (w == 0.0) continue;
                        const double *v = qkv + ((size_t)(b * S + j)) * 3 * H + 2 * H + (size_t)h * d;
                        for (int c = 0; c < d; ++c) o[c] += w * v[c];
                    }
                }
        free(P);
    }
}

/* Backward: dctx [T,H] -> dqkv [T,3H] (overwritten). */
static void attn_bwd(const attn_ctx *a, const double *qkv, const double *dctx, double *dqkv)
{
    const int B = a->B, S = a->S, H = a->H, N = a->N, d = a->d;
    const uint64_t thr = drop_threshold(a->pa);
    const double sd = 1.0 / (1.0 - a->pa);
    const double scale = 1.0 / sqrt((double)d);
    memset(dqkv, 0, sizeof(double) * (size_t)B * S * 3 * H);
    #pragma omp parallel
    {
        double *P = (double *)malloc(sizeof(double) * S);
        double *dP = (double *)malloc(sizeof(double) * S);
        #pragma omp for schedule(static) collapse(2)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < N; ++h) {
                /* each (b,h) owns its own columns of dqkv: no sharing */
                for (int i = 0; i < S; ++i) {
                    attn_row_probs(a, qkv, b, h, i, P, NULL);
                    const double *dO = dctx + ((size_t)(b * S + i)) * H + (size_t)h * d;
                    const double *q = qkv + ((size_t)(b * S + i)) * 3 * H + (size_t)h * d;
                    double D = 0.0;
                    for (int j = 0; j < S; ++j) {
                        const double *v = qkv + ((size_t)(b * S + j)) * 3 * H + 2 * H + (size_t)h * d;
                        double dPt = 0.0; /* gradient w.r.t. the dropped probability */
                        for (int c = 0; c < d; ++c) dPt += dO[c] * v[c];
                        double f = attn_drop_factor(a, thr, sd, b, h, i, j);
                        /* dV[j] += Ptilde[i][j] dO[i] */
                        double w = P[j] * f;
                        if (w != 0.0) {
                            double *dv = dqkv + ((size_t)(b * S + j)) * 3 * H + 2 * H + (size_t)h * d;
                            for (int c = 0; c < d; ++c) dv[c] += w * dO[c];
                        }
                        dP[j] = dPt * f;
                        D += P[j] * dP[j];
                    }
                    double *dq = dqkv + ((size_t)(b * S + i)) * 3 * H + (size_t)h * d;
                    for (int j = 0; j < S; ++j) {
                        double dS = P[j] * (dP[j] - D);
                        if (dS == 0.0) continue;
                        const double *k = qkv + ((size_t)(b * S + j)) * 3 * H + H + (size_t)h * d;
                        double *dk = dqkv + ((size_t)(b * S + j)) * 3 * H + H + (size_t)h * d;
                        for (int c = 0; c < d; ++c) {
                            dq[c] += dS * k[c] * scale;
                            dk[c] += dS * q[c] * scale;
                        }
                    }
                }
            }
        free(P); free(dP);
    }
}

/* Softmax probabilities and context of a standalone attention call (used by
 * the invariant tests).  qkv [T,3H]; P_out [B,N,S,S] may be NULL. */
int orc_attention_forward(const orc_cfg *cfg, const double *qkv, const int32_t *len,
                          double *ctx, double *lse, double *P_out)
{
    attn_ctx a = { cfg->batch, cfg->seq, cfg->hidden, cfg->heads, cfg->hidden / cfg->heads,
                   len, cfg->training, cfg->batch_offset, cfg->attn_p, cfg->seed, cfg->step, cfg->layer_id };
    attn_fwd(&a, qkv, ctx, lse, P_out);
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Hidden dropout (sites 1 and 2) on a [T,H] tensor, element t_global*H + c. */
static void hidden_dropout(const orc_cfg *cfg, uint32_t site, int T, int H, const double *in, double *out)
{
    const uint64_t thr = cfg->training ? drop_threshold(cfg->hidden_p) : 0;
    const double sd = 1.0 / (1.0 - cfg->hidden_p);
    const uint64_t t0 = (uint64_t)cfg->batch_offset * cfg->seq;
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            size_t i = (size_t)t * H + c;
            if (thr == 0) { out[i] = in[i]; continue; }
            uint64_t e = (t0 + t) * (uint64_t)H + c;
            out[i] = keep_elem(cfg->seed, cfg->layer_id, site, cfg->step, e, thr) ? in[i] * sd : 0.0;
        }
}

static int check_cfg(const orc_cfg *c)
{
    if (c->batch <= 0 || c->seq <= 0 || c->hidden <= 0 || c->heads <= 0 || c->ffn <= 0) return ORC_ERR;
    if (c->hidden % c->heads) return ORC_ERR;
    if (c->attn_p < 0 || c->attn_p >= 1 || c->hidden_p < 0 || c->hidden_p >= 1) return ORC_ERR;
    if ((c->attn_p > 0 && drop_threshold(c->attn_p) == 0) || (c->hidden_p > 0 && drop_threshold(c->hidden_p) == 0))
        return ORC_ERR;
    return ORC_OK;
}

#define ALLOC(n) ((double *)calloc((size_t)(n), sizeof(double)))

typedef struct {
    double *qkv, *ctx, *lse, *attn_proj, *ln1_in, *ln1_out, *mu1, *rstd1;
    double *u, *g, *ffn_out, *ln2_in, *ln2_out, *mu2, *rstd2, *y;
} fwd_state;

static void free_state(fwd_state *s)
{
    free(s->qkv); free(s->ctx); free(s->lse); free(s->attn_proj); free(s->ln1_in); free(s->ln1_out);
    free(s->mu1); free(s->rstd1); free(s->u); free(s->g); free(s->ffn_out); free(s->ln2_in);
    free(s->ln2_out); free(s->mu2); free(s->rstd2); free(s->y);
}

/* Full forward; every intermediate kept in st. */
static void layer_fwd(const orc_cfg *cfg, const orc_params *p, const double *x, const int32_t *len, fwd_state *st)
{
    const int B = cfg->batch, S = cfg->seq, H = cfg->hidden, N = cfg->heads, F = cfg->ffn;
    const int T = B * S;
    st->qkv = ALLOC((size_t)T * 3 * H); st->ctx = ALLOC((size_t)T * H); st->lse = ALLOC((size_t)B * N * S);
    st->attn_proj = ALLOC((size_t)T * H); st->ln1_in = ALLOC((size_t)T * H); st->ln1_out = ALLOC((size_t)T * H);
    st->mu1 = ALLOC(T); st->rstd1 = ALLOC(T); st->u = ALLOC((size_t)T * F); st->g = ALLOC((size_t)T * F);
    st->ffn_out = ALLOC((size_t)T * H); st->ln2_in = ALLOC((size_t)T * H); st->ln2_out = ALLOC((size_t)T * H);
    st->mu2 = ALLOC(T); st->rstd2 = ALLOC(T); st->y = ALLOC((size_t)T * H);
    attn_ctx a = { B, S, H, N, H / N, len, cfg->training, cfg->batch_offset, cfg->attn_p,
                   cfg->seed, cfg->step, cfg->layer_id };
    double *tmp = ALLOC((size_t)T * H);

    if (cfg->pre_ln) {
        /* x1 = x + drop1(attn(LN1(x)) W_o^T + b_o); y = x1 + drop2(FFN(LN2(x1))) */
        memcpy(st->ln1_in, x, sizeof(double) * (size_t)T * H);
        orc_ln_forward(T, H, x, p->ln1_g, p->ln1_b, cfg->ln_eps, st->ln1_out, st->mu1, st->rstd1);
        linear_fwd(T, H, 3 * H, st->ln1_out, p->w_qkv, p->b_qkv, st->qkv);
        attn_fwd(&a, st->qkv, st->ctx, st->lse, NULL);
        linear_fwd(T, H, H, st->ctx, p->w_o, p->b_o, st->attn_proj);
        hidden_dropout(cfg, 1u, T, H, st->attn_proj, tmp);
        for (size_t i = 0; i < (size_t)T * H; ++i) st->ln2_in[i] = x[i] + tmp[i];
        orc_ln_forward(T, H, st->ln2_in, p->ln2_g, p->ln2_b, cfg->ln_eps, st->ln2_out, st->mu2, st->rstd2);
        linear_fwd(T, H, F, st->ln2_out, p->w_1, p->b_1, st->u);
        for (size_t i = 0; i < (size_t)T * F; ++i) st->g[i] = orc_gelu(st->u[i]);
        linear_fwd(T, F, H, st->g, p->w_2, p->b_2, st->ffn_out);
        hidden_dropout(cfg, 2u, T, H, st->ffn_out, tmp);
        for (size_t i = 0; i < (size_t)T * H; ++i) st->y[i] = st->ln2_in[i] + tmp[i];
    } else {
        /* x1 = LN1(x + drop1(attn(x) W_o^T + b_o)); y = LN2(x1 + drop2(FFN(x1))) */
        linear_fwd(T, H, 3 * H, x, p->w_qkv, p->b_qkv, st->qkv);
        attn_fwd(&a, st->qkv, st->ctx, st->lse, NULL);
        linear_fwd(T, H, H, st->ctx, p->w_o, p->b_o, st->attn_proj);
        hidden_dropout(cfg, 1u, T, H, st->attn_proj, tmp);
        for (size_t i = 0; i < (size_t)T * H; ++i) st->ln1_in[i] = x[i] + tmp[i];
        orc_ln_forward(T, H, st->ln1_in, p->ln1_g, p->ln1_b, cfg->ln_eps, st->ln1_out, st->mu1, st->rstd1);
        linear_fwd(T, H, F, st->ln1_out, p->w_1, p->b_1, st->u);
        for (size_t i = 0; i < (size_t)T * F; ++i) st->g[i] = orc_gelu(st->u[i]);
        linear_fwd(T, F, H, st->g, p->w_2, p->b_2, st->ffn_out);
        hidden_dropout(cfg, 2u, T, H, st->ffn_out, tmp);
        for (size_t i = 0; i < (size_t)T * H; ++i) st->ln2_in[i] = st->ln1_out[i] + tmp[i];
        orc_ln_forward(T, H, st->ln2_in, p->ln2_g, p->ln2_b, cfg->ln_eps, st->ln2_out, st->mu2, st->rstd2);
        memcpy(st->y, st->ln2_out, sizeof(double) * (size_t)T * H);
    }
    free(tmp);
}

static void copy_out(double *dst, const double *src, size_t n) { if (dst) memcpy(dst, src, sizeof(double) * n); }

/* Forward.  y [T,H]; acts optional. */
int orc_layer_forward(const orc_cfg *cfg, const orc_params *p, const double *x, const int32_t *len,
                      double *y, orc_acts *acts)
{
    if (check_cfg(cfg)) return ORC_ERR;
    const int B = cfg->batch, S = cfg->seq, H = cfg->hidden, N = cfg->heads, F = cfg->ffn;
    const size_t T = (size_t)B * S;
    fwd_state st;
    memset(&st, 0, sizeof(st));
    layer_fwd(cfg, p, x, len, &st);
    copy_out(y, st.y, T * H);
    if (acts) {
        copy_out(acts->qkv, st.qkv, T * 3 * H);
        copy_out(acts->ctx, st.ctx, T * H);
        copy_out(acts->lse, st.lse, (size_t)B * N * S);
        copy_out(acts->attn_proj, st.attn_proj, T * H);
        copy_out(acts->ln1_in, st.ln1_in, T * H);
        copy_out(acts->ln1_out, st.ln1_out, T * H);
        copy_out(acts->mu1, st.mu1, T);
        copy_out(acts->rstd1, st.rstd1, T);
        copy_out(acts->u, st.u, T * F);
        copy_out(acts->g, st.g, T * F);
        copy_out(acts->ffn_out, st.ffn_out, T * H);
        copy_out(acts->ln2_in, st.ln2_in, T * H);
        copy_out(acts->ln2_out, st.ln2_out, T * H);
        copy_out(acts->mu2, st.mu2, T);
        copy_out(acts->rstd2, st.rstd2, T);
    }
    free_state(&st);
    return ORC_OK;
}

/* Backward by the chain rule through the forward above (recomputed here).
 * dy [T,H] upstream gradient; dx [T,H] and all 12 grads OVERWRITTEN.
 * ln_invertible selects the LayerNorm backward from the LN output.  y_out
 * (may be NULL) receives the recomputed forward output. */
int orc_layer_backward(const orc_cfg *cfg, const orc_params *p, const double *x, const int32_t *len,
                       const double *dy, int ln_invertible, double *dx, orc_grads *gr, double *y_out)
{
    if (check_cfg(cfg)) return ORC_ERR;
    const int B = cfg->batch, S = cfg->seq, H = cfg->hidden, N = cfg->heads, F = cfg->ffn;
    const int T = B * S;
    const size_t TH = (size_t)T * H, TF = (size_t)T * F;
    fwd_state st;
    memset(&st, 0, sizeof(st));
    layer_fwd(cfg, p, x, len, &st);
    copy_out(y_out, st.y, TH);
    attn_ctx a = { B, S, H, N, H / N, len, cfg->training, cfg->batch_offset, cfg->attn_p,
                   cfg->seed, cfg->step, cfg->layer_id };

    double *df = ALLOC(TH), *dg = ALLOC(TF), *dsub = ALLOC(TH), *dres = ALLOC(TH), *tmp = ALLOC(TH);
    double *dctx = ALLOC(TH), *dqkv = ALLOC(TH * 3), *dz = ALLOC(TH);
    const int inv = ln_invertible ? 1 : 0;

    if (cfg->pre_ln) {
        /* FFN branch: y = x1 + drop2(f) */
        hidden_dropout(cfg, 2u, T, H, dy, df);
        linear_bwd(T, F, H, df, st.g, p->w_2, dg, gr->w_2, gr->b_2);
        for (size_t i = 0; i < TF; ++i) dg[i] *= orc_gelu_grad(st.u[i]);      /* dg -> du */
        linear_bwd(T, H, F, dg, st.ln2_out, p->w_1, dsub, gr->w_1, gr->b_1);  /* dsub = da2 */
        orc_ln_backward(T, H, dsub, inv ? st.ln2_out : st.ln2_in, inv, st.mu2, st.rstd2,
                        p->ln2_g, p->ln2_b, tmp, gr->ln2_g, gr->ln2_b);
        for (size_t i = 0; i < TH; ++i) dres[i] = dy[i] + tmp[i];               /* dres = dx1 */
        /* attention branch: x1 = x + drop1(o) */
        hidden_dropout(cfg, 1u, T, H, dres, dz);
        linear_bwd(T, H, H, dz, st.ctx, p->w_o, dctx, gr->w_o, gr->b_o);
        attn_bwd(&a, st.qkv, dctx, dqkv);
        linear_bwd(T, H, 3 * H, dqkv, st.ln1_out, p->w_qkv, dsub, gr->w_qkv, gr->b_qkv); /* da1 */
        orc_ln_backward(T, H, dsub, inv ? st.ln1_out : st.ln1_in, inv, st.mu1, st.rstd1,
                        p->ln1_g, p->ln1_b, tmp, gr->ln1_g, gr->ln1_b);
        for (size_t i = 0; i < TH; ++i) dx[i] = dres[i] + tmp[i];
    } else {
        /* y = LN2(z2), z2 = x1 + drop2(f) */
        orc_ln_backward(T, H, dy, inv ? st.ln2_out : st.ln2_in, inv, st.mu2, st.rstd2,
                        p->ln2_g, p->ln2_b, dres, gr->ln2_g, gr->ln2_b);       /* dres = dz2 */
        hidden_dropout(cfg, 2u, T, H, dres, df);
        linear_bwd(T, F, H, df, st.g, p->w_2, dg, gr->w_2, gr->b_2);
        for (size_t i = 0; i < TF; ++i) dg[i] *= orc_gelu_grad(st.u[i]);
        linear_bwd(T, H, F, dg, st.ln1_out, p->w_1, dsub, gr->w_1, gr->b_1);
        for (size_t i = 0; i < TH; ++i) dsub[i] += dres[i];                      /* dsub = dx1 */
        /* x1 = LN1(z1), z1 = x + drop1(o) */
        orc_ln_backward(T, H, dsub, inv ? st.ln1_out : st.ln1_in, inv, st.mu1, st.rstd1,
                        p->ln1_g, p->ln1_b, dres, gr->ln1_g, gr->ln1_b);       /* dres = dz1 */
        hidden_dropout(cfg, 1u, T, H, dres, dz);
        linear_bwd(T, H, H, dz, st.ctx, p->w_o, dctx, gr->w_o, gr->b_o);
        attn_bwd(&a, st.qkv, dctx, dqkv);
        linear_bwd(T, H, 3 * H, dqkv, x, p->w_qkv, tmp, gr->w_qkv, gr->b_qkv);
        for (size_t i = 0; i < TH; ++i) dx[i] = dres[i] + tmp[i];
    }
    free(df); free(dg); free(dsub); free(dres); free(tmp); free(dctx); free(dqkv); free(dz);
    free_state(&st);
    return ORC_OK;
}
