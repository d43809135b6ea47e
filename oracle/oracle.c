/*
 * oracle.c -- plain CPU reference of the uniform byte encoder's forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library includes, links or
 * calls this file; only the test-suite, the package's smoke check and the
 * benchmark's CPU-baseline leg load it. It shares no code, header, table or
 * helper with the HIP path.
 *
 * Arithmetic: IEEE double throughout (libm sqrt, exp, cos, sin), plain loops,
 * no blocking, fusion or reordering beyond what each definition states. Weight
 * matrices arrive as float32 arrays holding bfloat16-exact values (the model's
 * stored precision); gains are float32. Matrices use y = x W with W row-major
 * [in x out].
 *
 * Sources (UForm documentation pages):
 *   - "UForm" page, section "Architecture & Goals": bytes in, N same-width
 *     blocks of RMSNorm, QKV attention and a SwiGLU MLP, multi-axis M-RoPE,
 *     attention-pooled embedding out.
 *   - "UForm" page, section "One Omni Model": byte-gather, 16x16 patch and
 *     tube frontends with 1-D, 2-D and 3-D rotary coordinates.
 *   - "UForm" page, section "Precision by Design": fp32 block input,
 *     accumulation and normalisation in fp32; E4M3 inference mode.
 *   - "UForm" page, FAQ "Why attention pooling instead of mean pooling?": one
 *     learned query of encoder width, per-byte outputs as keys and values.
 *   - "Arenas" page, section "Rows and Tapes": Arrow tapes, count+1 offsets.
 *   - "Python" page, section "Encoding": stats report truncated items and
 *     encoded tokens.
 * Readings where the pages are silent are listed with each function.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_INVALID_ARGUMENT 1
#define ORACLE_SHAPE_MISMATCH 2

/* ------------------------------------------------------------------ tapes */

/* Tape ingest ("Arenas" page, "Rows and Tapes"; "Python" page, "Encoding"
 * stats). Item i spans data[offsets[i] .. offsets[i+1]); offsets must not
 * decrease (offsets[0] may be non-zero, as in an Arrow slice). Reading: an item
 * longer than `context` keeps its first `context` bytes and counts once in
 * `truncated`; `tokens` is the number of bytes encoded.
 * lengths[i] = kept length, cu[0] = 0, cu[i+1] = cu[i] + lengths[i]. */
int oracle_tape_plan(const uint64_t *offsets, size_t count, size_t context, uint64_t *lengths, uint64_t *cu,
                     uint64_t *stats) {
    uint64_t truncated = 0, tokens = 0;
    cu[0] = 0;
    for (size_t i = 0; i < count; ++i) {
        if (offsets[i + 1] < offsets[i]) return ORACLE_INVALID_ARGUMENT;
        uint64_t len = offsets[i + 1] - offsets[i];
        uint64_t kept = len;
        if (kept > context) {
            kept = context;
            truncated += 1;
        }
        lengths[i] = kept;
        cu[i + 1] = cu[i] + kept;
        tokens += kept;
    }
    stats[0] = truncated;
    stats[1] = tokens;
    return ORACLE_OK;
}

/* -------------------------------------------------------------- frontends */

/* Byte-gather frontend ("UForm" page, "One Omni Model": raw bytes embedded
 * directly, a byte per token). Reading: token id = byte value, no added
 * special tokens; positions restart at 0 in every item. x is [T x D], pos is
 * [T x 3] (axes beyond the first are 0). */
void oracle_embed_text(const uint8_t *data, const uint64_t *offsets, const uint64_t *lengths, const uint64_t *cu,
                       size_t count, const float *embed, size_t D, double *x, int32_t *pos) {
    for (size_t i = 0; i < count; ++i) {
        for (uint64_t t = 0; t < lengths[i]; ++t) {
            uint8_t byte = data[offsets[i] + t];
            uint64_t row = cu[i] + t;
            for (size_t f = 0; f < D; ++f) x[row * D + f] = (double)embed[(size_t)byte * D + f];
            pos[row * 3 + 0] = (int32_t)t;
            pos[row * 3 + 1] = 0;
            pos[row * 3 + 2] = 0;
        }
    }
}

/* Patch frontend for images and per-frame video patches ("UForm" page, "One
 * Omni Model"). Readings: an item is `frames` frames of height x width
 * interleaved 8-bit pixels with `channels` channels; patch (r, c) of frame f
 * is token f*gh*gw + r*gw + c; element k = (py*p + px)*channels + ch of the
 * patch vector holds pixel (p*r + py, p*c + px, ch) / 255; x = vector W_patch
 * with no bias. Positions: (r, c) for one frame (axes = 2), (f, r, c) for a
 * clip (axes = 3). The caller has checked side % p == 0. */
void oracle_embed_patches(const uint8_t *pixels, uint64_t frames, uint64_t height, uint64_t width, size_t channels,
                          size_t p, const float *patch_proj, size_t D, int axes, double *x, int32_t *pos) {
    uint64_t gh = height / p, gw = width / p;
    size_t K = p * p * channels;
    double *vec = (double *)malloc(K * sizeof(double));
    for (uint64_t f = 0; f < frames; ++f) {
        const uint8_t *frame = pixels + f * height * width * channels;
        for (uint64_t r = 0; r < gh; ++r) {
            for (uint64_t c = 0; c < gw; ++c) {
                uint64_t token = f * gh * gw + r * gw + c;
                for (size_t py = 0; py < p; ++py)
                    for (size_t px = 0; px < p; ++px)
                        for (size_t ch = 0; ch < channels; ++ch) {
                            uint64_t yy = p * r + py, xx = p * c + px;
                            vec[(py * p + px) * channels + ch] =
                                (double)frame[(yy * width + xx) * channels + ch] / 255.0;
                        }
                double *out = x + token * D;
                for (size_t n = 0; n < D; ++n) out[n] = 0.0;
                for (size_t k = 0; k < K; ++k) {
                    double a = vec[k];
                    const float *w = patch_proj + k * D;
                    for (size_t n = 0; n < D; ++n) out[n] += a * (double)w[n];
                }
                if (axes == 3) {
                    pos[token * 3 + 0] = (int32_t)f;
                    pos[token * 3 + 1] = (int32_t)r;
                    pos[token * 3 + 2] = (int32_t)c;
                } else {
                    pos[token * 3 + 0] = (int32_t)r;
                    pos[token * 3 + 1] = (int32_t)c;
                    pos[token * 3 + 2] = 0;
                }
            }
        }
    }
    free(vec);
}

/* ------------------------------------------------------------ E4M3 (FP8) */

/* Nearest OCP E4M3FN value (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, no infinities; largest finite 448 = 1.75 * 2^8; smallest normal 2^-6,
 * subnormals k * 2^-9), ties to even, magnitudes past 448 saturate to 448.
 * Used by the E4M3 inference mode ("UForm" page, "Precision by Design"). */
double oracle_e4m3_round(double v) {
    if (isnan(v)) return v;
    double a = fabs(v);
    double q;
    if (a < 0x1p-6) {
        q = nearbyint(a / 0x1p-9) * 0x1p-9;
    } else {
        int e;
        frexp(a, &e); /* a = m * 2^e with m in [0.5, 1): binade exponent is e-1 */
        int be = e - 1;
        if (be > 8) be = 8;
        double quantum = ldexp(1.0, be - 3);
        q = nearbyint(a / quantum) * quantum;
    }
    if (q > 448.0) q = 448.0;
    return v < 0 ? -q : q;
}

/* Quantise-dequantise with one scale s = amax / 448 over `n` values (a whole
 * weight tensor, or one activation row). Reading: the scale multiplies the
 * E4M3 code back; an all-zero input stays zero. */
static void e4m3_qdq(const double *in, double *out, size_t n) {
    double amax = 0.0;
    for (size_t i = 0; i < n; ++i) amax = fmax(amax, fabs(in[i]));
    if (amax == 0.0) {
        for (size_t i = 0; i < n; ++i) out[i] = 0.0;
        return;
    }
    double s = amax / 448.0;
    for (size_t i = 0; i < n; ++i) out[i] = oracle_e4m3_round(in[i] / s) * s;
}

void oracle_e4m3_qdq(const double *in, double *out, size_t n) { e4m3_qdq(in, out, n); }

/* Nearest bfloat16 value of v, as stored by a GPU that holds activations in
 * bf16 ("UForm" page, "Precision by Design": store and compute in BF16,
 * accumulate in Float32): v is first rounded to float32, then to bf16 with ties
 * to even (the fp32 accumulator -> bf16 storage path). */
double oracle_bf16_round(double v) {
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7f800000u) == 0x7f800000u) return v; /* inf / nan unchanged */
    u += 0x7fffu + ((u >> 16) & 1u);
    u &= 0xffff0000u;
    memcpy(&f, &u, 4);
    return (double)f;
}

static void bf16_round_all(double *a, size_t n) {
    for (size_t i = 0; i < n; ++i) a[i] = oracle_bf16_round(a[i]);
}

/* ------------------------------------------------------------- the blocks */

/* Observation points for the pins: when a tap is installed, the blocks hand it
 * every GEMM input exactly as the product reads it (after its per-row E4M3
 * quantise-dequantise in E4M3 mode), every weight matrix as the products use it,
 * and the activations stored between steps (q and k as attention reads them, v,
 * the attention output o and the SwiGLU output a). A tap only reads; it changes
 * no value. Not thread-safe: one forward at a time while a tap is installed. */
typedef void (*oracle_tap_t)(const char *name, const double *data, size_t rows, size_t cols);
static oracle_tap_t g_tap = NULL;

void oracle_set_tap(oracle_tap_t fn) { g_tap = fn; }

static void tap(const char *name, const double *data, size_t rows, size_t cols) {
    if (g_tap && name) g_tap(name, data, rows, cols);
}

/* y[T x N] = x[T x K] W[K x N]. With `e4m3`, every row of x is first
 * replaced by its per-row quantise-dequantise (W is already quantised).
 * `name` labels the product's input for the tap (NULL: not observed). */
static void matmul_named(const char *name, const double *x, size_t T, size_t K, const double *W, size_t N, double *y,
                         int e4m3) {
    double *xq = NULL;
    if (e4m3) {
        xq = (double *)malloc((T ? T : 1) * K * sizeof(double));
#pragma omp parallel for schedule(static)
        for (size_t t = 0; t < T; ++t) e4m3_qdq(x + t * K, xq + t * K, K);
        x = xq;
    }
    tap(name, x, T, K);
#pragma omp parallel for schedule(static)
    for (size_t t = 0; t < T; ++t) {
        const double *xr = x + t * K;
        double *yr = y + t * N;
        for (size_t n = 0; n < N; ++n) yr[n] = 0.0;
        for (size_t k = 0; k < K; ++k) {
            double a = xr[k];
            const double *w = W + k * N;
            for (size_t n = 0; n < N; ++n) yr[n] += a * w[n];
        }
    }
    free(xq);
}

static void matmul(const double *x, size_t T, size_t K, const double *W, size_t N, double *y, int e4m3) {
    matmul_named(NULL, x, T, K, W, N, y, e4m3);
}

/* One block product on its own (exposed for pins): y = x W, W [K x N] used as
 * given; with `e4m3` the rows of x are quantised per row as in the blocks. */
void oracle_matmul(const double *x, size_t T, size_t K, const double *W, size_t N, double *y, int e4m3) {
    matmul(x, T, K, W, N, y, e4m3);
}

/* RMSNorm ("UForm" page, "Architecture & Goals"; inverse RMS in at least
 * fp32 per "Precision by Design"): out = x * g / sqrt(mean(x^2) + eps).
 * Reading: eps inside the square root, a learned gain, no bias. */
void oracle_rmsnorm(const double *x, const float *g, size_t T, size_t D, double eps, double *out) {
#pragma omp parallel for schedule(static)
    for (size_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (size_t f = 0; f < D; ++f) ss += x[t * D + f] * x[t * D + f];
        double inv = 1.0 / sqrt(ss / (double)D + eps);
        for (size_t f = 0; f < D; ++f) out[t * D + f] = x[t * D + f] * inv * (double)g[f];
    }
}

/* Multi-axis rotary positions ("UForm" page, "Architecture & Goals" and "One
 * Omni Model": one block serves 1-D text, 2-D image and 3-D video
 * coordinates). Readings: within each head of width d, pair j rotates
 * dimensions (2j, 2j+1) by angle pos[axis(j)] * base^(-2j/d) (RoFormer's
 * adjacent pairing and frequency ladder); the d/2 pairs are split into
 * `axes` contiguous sections as evenly as possible, leading sections taking
 * the remainder. v is [T x H*d]; applied to queries and keys only. */
int oracle_rope_axis_of(size_t pair, size_t d, int axes) {
    size_t pairs = d / 2, base_n = pairs / (size_t)axes, rem = pairs % (size_t)axes;
    size_t start = 0;
    for (int a = 0; a < axes; ++a) {
        size_t len = base_n + ((size_t)a < rem ? 1 : 0);
        if (pair < start + len) return a;
        start += len;
    }
    return axes - 1;
}

void oracle_rope(double *v, const int32_t *pos, size_t T, size_t H, size_t d, int axes, double base) {
#pragma omp parallel for schedule(static)
    for (size_t t = 0; t < T; ++t) {
        for (size_t h = 0; h < H; ++h) {
            double *head = v + t * H * d + h * d;
            for (size_t j = 0; j < d / 2; ++j) {
                int a = oracle_rope_axis_of(j, d, axes);
                double theta = pow(base, -2.0 * (double)j / (double)d);
                double phi = (double)pos[t * 3 + a] * theta;
                double c = cos(phi), s = sin(phi);
                double x0 = head[2 * j], x1 = head[2 * j + 1];
                head[2 * j] = x0 * c - x1 * s;
                head[2 * j + 1] = x0 * s + x1 * c;
            }
        }
    }
}

/* Bidirectional variable-length attention ("UForm" page, FAQ "Why no cuDNN,
 * FlashAttention...": ragged attention with every segment summed on its own).
 * Readings: each item's tokens attend to all tokens of that item and no
 * other; scores q.k / sqrt(d); exact softmax (max subtracted, then
 * normalised). q, k, v, out are [T x H*d]; head h owns columns [h*d, h*d+d). */
void oracle_attention(const double *q, const double *k, const double *v, const uint64_t *cu, size_t count,
                      size_t H, size_t d, double *out) {
    size_t W = H * d;
    double scale = 1.0 / sqrt((double)d);
    for (size_t i = 0; i < count; ++i) {
        uint64_t a = cu[i], b = cu[i + 1];
        if (b == a) continue;
        uint64_t L = b - a;
#pragma omp parallel
        {
            double *s = (double *)malloc(L * sizeof(double));
#pragma omp for collapse(2) schedule(static)
            for (size_t h = 0; h < H; ++h) {
                for (uint64_t t = a; t < b; ++t) {
                    const double *qt = q + t * W + h * d;
                    double m = -INFINITY;
                    for (uint64_t u = a; u < b; ++u) {
                        const double *ku = k + u * W + h * d;
                        double dot = 0.0;
                        for (size_t e = 0; e < d; ++e) dot += qt[e] * ku[e];
                        s[u - a] = dot * scale;
                        if (s[u - a] > m) m = s[u - a];
                    }
                    double sum = 0.0;
                    for (uint64_t u = 0; u < L; ++u) {
                        s[u] = exp(s[u] - m);
                        sum += s[u];
                    }
                    double *ot = out + t * W + h * d;
                    for (size_t e = 0; e < d; ++e) ot[e] = 0.0;
                    for (uint64_t u = a; u < b; ++u) {
                        double p = s[u - a] / sum;
                        const double *vu = v + u * W + h * d;
                        for (size_t e = 0; e < d; ++e) ot[e] += p * vu[e];
                    }
                }
            }
            free(s);
        }
    }
}

/* SiLU(z) = z / (1 + e^-z). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

typedef struct oracle_geometry_t {
    size_t depth, hidden, heads, ffn;
    int rope_axes;
    double rope_base, rms_epsilon;
    int e4m3; /* 1: blocks run with E4M3 weights and activations */
} oracle_geometry_t;

/* Per-block weights, float32 holding bf16 values; gains float32. */
typedef struct oracle_block_t {
    const float *attn_norm, *w_qkv, *w_o, *mlp_norm, *w_gate, *w_up, *w_down;
} oracle_block_t;

static double *widen(const float *w, size_t n, int e4m3) {
    double *out = (double *)malloc(n * sizeof(double));
    for (size_t i = 0; i < n; ++i) out[i] = (double)w[i];
    if (e4m3) e4m3_qdq(out, out, n);
    return out;
}

/* A block matrix as the E4M3 blocks use it (exposed for pins): one
 * quantise-dequantise over the whole tensor of n values. */
void oracle_e4m3_weights(const float *w, size_t n, double *out) {
    double *q = widen(w, n, 1);
    memcpy(out, q, n * sizeof(double));
    free(q);
}

/* One pre-norm block ("UForm" page, "Architecture & Goals"; the residual
 * stream is the block's fp32 input kept across the block, "Precision by
 * Design"). Readings: x += Attn(RMSNorm1(x)); x += MLP(RMSNorm2(x)); fused
 * W_qkv = [W_q | W_k | W_v] with no biases; MLP = (SiLU(h W_gate) * (h W_up))
 * W_down. In E4M3 mode every block matrix is quantised per tensor and every
 * GEMM input row per row, and the activations the pages store in bf16 are
 * rounded to bf16 where they are stored: q and k after the rotation, v, the
 * attention output o and the SwiGLU output a (the normalised rows h are
 * quantised straight from their fp32 values). x is [T x D], updated in place. */
void oracle_block(const oracle_geometry_t *g, const oracle_block_t *w, double *x, const int32_t *pos,
                  const uint64_t *cu, size_t count, size_t T) {
    size_t D = g->hidden, H = g->heads, F = g->ffn, d = D / H;
    double *h = (double *)malloc(T * D * sizeof(double));
    double *qkv = (double *)malloc(T * 3 * D * sizeof(double));
    double *q = (double *)malloc(T * D * sizeof(double));
    double *k = (double *)malloc(T * D * sizeof(double));
    double *v = (double *)malloc(T * D * sizeof(double));
    double *o = (double *)malloc(T * D * sizeof(double));
    double *y = (double *)malloc(T * D * sizeof(double));
    double *gt = (double *)malloc(T * F * sizeof(double));
    double *up = (double *)malloc(T * F * sizeof(double));
    double *Wqkv = widen(w->w_qkv, D * 3 * D, g->e4m3), *Wo = widen(w->w_o, D * D, g->e4m3);
    double *Wg = widen(w->w_gate, D * F, g->e4m3), *Wu = widen(w->w_up, D * F, g->e4m3);
    double *Wd = widen(w->w_down, F * D, g->e4m3);

    tap("w_qkv", Wqkv, D, 3 * D);
    tap("w_o", Wo, D, D);
    tap("w_gate", Wg, D, F);
    tap("w_up", Wu, D, F);
    tap("w_down", Wd, F, D);

    /* attention half */
    oracle_rmsnorm(x, w->attn_norm, T, D, g->rms_epsilon, h);
    matmul_named("qkv_in", h, T, D, Wqkv, 3 * D, qkv, g->e4m3);
    for (size_t t = 0; t < T; ++t)
        for (size_t f = 0; f < D; ++f) {
            q[t * D + f] = qkv[t * 3 * D + f];
            k[t * D + f] = qkv[t * 3 * D + D + f];
            v[t * D + f] = qkv[t * 3 * D + 2 * D + f];
        }
    oracle_rope(q, pos, T, H, d, g->rope_axes, g->rope_base);
    oracle_rope(k, pos, T, H, d, g->rope_axes, g->rope_base);
    if (g->e4m3) {
        bf16_round_all(q, T * D);
        bf16_round_all(k, T * D);
        bf16_round_all(v, T * D);
    }
    tap("q", q, T, D);
    tap("k", k, T, D);
    tap("v", v, T, D);
    oracle_attention(q, k, v, cu, count, H, d, o);
    if (g->e4m3) bf16_round_all(o, T * D);
    tap("o", o, T, D);
    matmul_named("out_in", o, T, D, Wo, D, y, g->e4m3);
    for (size_t i = 0; i < T * D; ++i) x[i] += y[i];

    /* MLP half */
    oracle_rmsnorm(x, w->mlp_norm, T, D, g->rms_epsilon, h);
    matmul_named("mlp_in", h, T, D, Wg, F, gt, g->e4m3);
    matmul_named("up_in", h, T, D, Wu, F, up, g->e4m3);
    for (size_t i = 0; i < T * F; ++i) gt[i] = silu(gt[i]) * up[i];
    if (g->e4m3) bf16_round_all(gt, T * F);
    tap("a", gt, T, F);
    matmul_named("down_in", gt, T, F, Wd, D, y, g->e4m3);
    for (size_t i = 0; i < T * D; ++i) x[i] += y[i];

    free(h); free(qkv); free(q); free(k); free(v); free(o); free(y); free(gt); free(up);
    free(Wqkv); free(Wo); free(Wg); free(Wu); free(Wd);
}

/* The MLP half alone on already-normalised rows (exposed for pins):
 * out = (SiLU(h W_gate) * (h W_up)) W_down. */
void oracle_swiglu(const double *h, size_t T, size_t D, size_t F, const float *w_gate, const float *w_up,
                   const float *w_down, double *out) {
    double *Wg = widen(w_gate, D * F, 0), *Wu = widen(w_up, D * F, 0), *Wd = widen(w_down, F * D, 0);
    double *gt = (double *)malloc(T * F * sizeof(double)), *up = (double *)malloc(T * F * sizeof(double));
    matmul(h, T, D, Wg, F, gt, 0);
    matmul(h, T, D, Wu, F, up, 0);
    for (size_t i = 0; i < T * F; ++i) gt[i] = silu(gt[i]) * up[i];
    matmul(gt, T, F, Wd, D, out, 0);
    free(Wg); free(Wu); free(Wd); free(gt); free(up);
}

/* Attention pooling ("UForm" page, FAQ "Why attention pooling instead of
 * mean pooling?"; the pool reads the final-norm states, "Training" page,
 * objective `joint`). Readings: learned query q in R^D split into H heads;
 * keys K = xf W_k and values V = xf W_v (D x D, no biases); per item and head
 * p = softmax_t(q_h . K_t,h / sqrt(d)), pooled_h = sum_t p_t V_t,h; heads
 * concatenated; no output projection and no normalisation; an item with no
 * tokens pools to the zero row. Computed in the dense form. xf is [T x D]. */
void oracle_pool(const double *xf, const uint64_t *cu, size_t count, size_t D, size_t H, const float *query,
                 const float *wk, const float *wv, double *pooled) {
    size_t T = cu[count], d = D / H;
    double *K = (double *)malloc((T ? T : 1) * D * sizeof(double));
    double *V = (double *)malloc((T ? T : 1) * D * sizeof(double));
    double *Wk = widen(wk, D * D, 0), *Wv = widen(wv, D * D, 0);
    matmul(xf, T, D, Wk, D, K, 0);
    matmul(xf, T, D, Wv, D, V, 0);
    double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for collapse(2) schedule(static)
    for (size_t i = 0; i < count; ++i) {
        for (size_t h = 0; h < H; ++h) {
            uint64_t a = cu[i], b = cu[i + 1];
            double *out = pooled + i * D + h * d;
            for (size_t e = 0; e < d; ++e) out[e] = 0.0;
            if (b == a) continue;
            double m = -INFINITY;
            for (uint64_t t = a; t < b; ++t) {
                double s = 0.0;
                for (size_t e = 0; e < d; ++e) s += (double)query[h * d + e] * K[t * D + h * d + e];
                s *= scale;
                if (s > m) m = s;
            }
            double sum = 0.0;
            for (uint64_t t = a; t < b; ++t) {
                double s = 0.0;
                for (size_t e = 0; e < d; ++e) s += (double)query[h * d + e] * K[t * D + h * d + e];
                sum += exp(s * scale - m);
            }
            for (uint64_t t = a; t < b; ++t) {
                double s = 0.0;
                for (size_t e = 0; e < d; ++e) s += (double)query[h * d + e] * K[t * D + h * d + e];
                double p = exp(s * scale - m) / sum;
                for (size_t e = 0; e < d; ++e) out[e] += p * V[t * D + h * d + e];
            }
        }
    }
    free(K); free(V); free(Wk); free(Wv);
}

/* The encoder after its frontend: N blocks, final RMSNorm, attention pool.
 * x0 is [T x D] (copied), pos [T x 3], cu [count+1]; pooled is [count x D].
 * `blocks` holds `depth` entries. */
void oracle_forward(const oracle_geometry_t *g, const oracle_block_t *blocks, const float *final_norm,
                    const float *pool_query, const float *pool_wk, const float *pool_wv, const double *x0,
                    const int32_t *pos, const uint64_t *cu, size_t count, double *pooled) {
    size_t T = cu[count], D = g->hidden;
    double *x = (double *)malloc((T ? T : 1) * D * sizeof(double));
    double *xf = (double *)malloc((T ? T : 1) * D * sizeof(double));
    memcpy(x, x0, T * D * sizeof(double));
    for (size_t l = 0; l < g->depth; ++l) oracle_block(g, &blocks[l], x, pos, cu, count, T);
    oracle_rmsnorm(x, final_norm, T, D, g->rms_epsilon, xf);
    oracle_pool(xf, cu, count, D, g->heads, pool_query, pool_wk, pool_wv, pooled);
    free(x); free(xf);
}

/* Same, but returns the final-norm states xf [T x D] too (for step checks). */
void oracle_forward_states(const oracle_geometry_t *g, const oracle_block_t *blocks, const float *final_norm,
                           const double *x0, const int32_t *pos, const uint64_t *cu, size_t count, double *x_out,
                           double *xf_out) {
    size_t T = cu[count], D = g->hidden;
    memcpy(x_out, x0, T * D * sizeof(double));
    for (size_t l = 0; l < g->depth; ++l) oracle_block(g, &blocks[l], x_out, pos, cu, count, T);
    oracle_rmsnorm(x_out, final_norm, T, D, g->rms_epsilon, xf_out);
}

/* ------------------------------------------------------- per-token outputs */

/* Token head ("UForm" page, the reranker paragraph of its losses: the per-byte
 * encoder output refined through a per-byte projection head into unit vectors;
 * "Rust" and "Python" pages, "Encoding": TOKEN_VECTORS are the head's unit
 * rows, one per state, token_width wide). Readings: a bias-free linear map of
 * the final-norm states, y = xf W with W [D x width] (bf16-exact), then every
 * row divided by its Euclidean norm; a zero row stays zero. out is [T x width]. */
void oracle_token_vectors(const double *xf, size_t T, size_t D, const float *w, size_t width, double *out) {
    double *W = widen(w, D * width, 0);
    matmul(xf, T, D, W, width, out, 0);
    for (size_t t = 0; t < T; ++t) {
        double ss = 0.0;
        for (size_t e = 0; e < width; ++e) ss += out[t * width + e] * out[t * width + e];
        if (ss > 0.0) {
            double norm = sqrt(ss);
            for (size_t e = 0; e < width; ++e) out[t * width + e] /= norm;
        }
    }
    free(W);
}

/* Hard MaxSim ("UForm" page, same paragraph): the score of query i against
 * document j is the mean, over the query's rows t, of the largest inner product
 * <q_t, d_s> over the document's rows s. q and d are row-major [rows x width];
 * query i owns rows qoff[i] .. qoff[i+1], document j rows doff[j] .. doff[j+1].
 * Readings: the query's rows start past its first `prefix` rows and at most
 * `span` of them count (the trainer's max_query_span, "Training" page,
 * uform_late_interaction_t); a query with no counted rows, or a document with
 * no rows, scores 0. scores is [nq x nd]. */
void oracle_maxsim(const double *q, const uint64_t *qoff, size_t nq, const double *d, const uint64_t *doff,
                   size_t nd, size_t width, size_t prefix, size_t span, double *scores) {
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (size_t i = 0; i < nq; ++i) {
        for (size_t j = 0; j < nd; ++j) {
            uint64_t qa = qoff[i] + prefix, qb = qoff[i + 1];
            if (qa > qb) qa = qb;
            if (qb - qa > span) qb = qa + span;
            uint64_t da = doff[j], db = doff[j + 1];
            double total = 0.0;
            if (qb > qa && db > da) {
                for (uint64_t t = qa; t < qb; ++t) {
                    double best = -INFINITY;
                    for (uint64_t s = da; s < db; ++s) {
                        double dot = 0.0;
                        for (size_t e = 0; e < width; ++e) dot += q[t * width + e] * d[s * width + e];
                        if (dot > best) best = dot;
                    }
                    total += best;
                }
                total /= (double)(qb - qa);
            }
            scores[i * nd + j] = total;
        }
    }
}
