/*
 * CPU oracle for the DFlash batched verify forward -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke entry and the benchmark's CPU-baseline leg load this library. The GPU
 * library never links or calls it, and it shares no code, header or table with the GPU path: it
 * receives the same seeded host arrays and computes, slowly and plainly, what the pages define.
 *
 * Sources (web pages; cited by title and section):
 *   [PR2303]  engine PR #2303 "npu forward: Gemma4 verifies a draft in one batched pass; KV row width
 *             per layer" -- sections "What changes", "Proof", the reviewer guide (kv_widths), reviews.
 *   [CARD]    "FastFlowLM build: Nemotron-3.5-Bolt-E4B-DFlash-NPU2" -- table rows Draft / Weights /
 *             Taps, "How it is used".
 *   [PR2236]  engine PR #2236 "npu: a Gemma4 pack stops re-reading its weights every token;
 *             tools/dflash_acceptance" -- section 2 and the acceptance tool's header comment.
 *
 * Precision contract: every operation is evaluated in double precision and rounded to the storage
 * precision at the points where the data is stored: the residual stream, every GEMM output, the
 * K/V planes and the logits are fp32; every GEMM input (normalised activations, attention output,
 * SwiGLU product, taps) is bf16, rounded to nearest even. Q4_1 weights are used exactly.
 *
 * Parity status: every function here is pinned by the CPU tests (closed forms, invariants, hand
 * cases, brute force on tiny shapes). No page prints values for the full-depth logits or the draft
 * block; those are pinned by hand cases with closed forms (the q/k path, the draft's fc, hidden
 * norm, context positions and head rows) and by an independent numpy float64 twin of the verify
 * and of the draft, which must agree with this file to 1e-12.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -lm. OpenMP only splits independent output
 * features; each output is summed by one thread in index order, so results do not depend on the
 * thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q4_1_BLOCK 32
#define Q4_1_BYTES 20

/* ------------------------------------------------------------------------------------------ */
/* number formats                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* IEEE 754 binary16 -> double, from the format's definition. */
static double half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)f, -24);                   /* subnormal: f * 2^-24 */
    else if (e == 31) v = f ? NAN : INFINITY;
    else v = ldexp((double)(1024 + f), e - 25);               /* (1 + f/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 (the top 16 bits of an fp32) -> double. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* double -> bfloat16, round to nearest, ties to even (8 significant bits). */
static uint16_t double_to_bf16(double v) {
    if (isnan(v)) return 0x7fc0;
    double a = fabs(v), r;
    if (a == 0.0) {
        r = 0.0;
    } else if (a < ldexp(1.0, -126)) {
        r = ldexp(nearbyint(ldexp(a, 133)), -133);            /* subnormal quantum 2^-133 */
    } else {
        int e;
        double m = frexp(a, &e);                              /* a = m 2^e, 0.5 <= m < 1 */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    }
    float f = (float)r;                                       /* exact: r has <= 8 bits */
    if (r > 3.3895313892515355e38) f = INFINITY;              /* beyond the largest bf16 */
    uint32_t u;
    memcpy(&u, &f, 4);
    uint16_t out = (uint16_t)(u >> 16);
    return v < 0 ? (uint16_t)(out | 0x8000) : out;
}

static double round_bf16(double v) { return bf16_to_double(double_to_bf16(v)); }
static double round_f32(double v) { return (double)(float)v; }

/* ------------------------------------------------------------------------------------------ */
/* Q4_1 [CARD, "Weights" row]: 32-weight blocks, 4-bit codes with an fp16 scale and an fp16     */
/* minimum, 5 bits per weight. Weight = scale * code + min (the minimum is the value of code 0). */
/* Block bytes: scale (LE), min (LE), 16 code bytes; code j<16 in the low nibble of byte j,      */
/* code j+16 in the high nibble.                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* Decode one block into 32 weights (the fp32 dequantised values, held as doubles). */
static void q4_1_block(const uint8_t* blk, double* w) {
    double s = half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    double m = half_to_double((uint16_t)(blk[2] | (blk[3] << 8)));
    for (int j = 0; j < Q4_1_BLOCK; j++) {
        int q = (j < 16) ? (blk[4 + j] & 15) : (blk[4 + j - 16] >> 4);
        w[j] = round_f32(s * q + m);
    }
}

void orc_q4_1_dequant(const uint8_t* img, int n_out, int n_in, float* out) {
    int nb = n_in / Q4_1_BLOCK;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < n_out; n++) {
        double w[Q4_1_BLOCK];
        for (int b = 0; b < nb; b++) {
            q4_1_block(img + ((size_t)n * nb + b) * Q4_1_BYTES, w);
            for (int j = 0; j < Q4_1_BLOCK; j++) out[(size_t)n * n_in + b * Q4_1_BLOCK + j] = (float)w[j];
        }
    }
}

/* y[r][n] = sum_k W[n][k] x[r][k] for r < m, W a Q4_1 image [n_out][n_in]; x holds bf16 values. */
static void q4_1_matmul(const uint8_t* img, int n_out, int n_in, const double* x, int m, double* y) {
    int nb = n_in / Q4_1_BLOCK;
#pragma omp parallel for schedule(static)
    for (int n = 0; n < n_out; n++) {
        double acc[64];   /* rows in groups of 64; each output still sums blocks and elements in order */
        double w[Q4_1_BLOCK];
        for (int r0 = 0; r0 < m; r0 += 64) {
            const int mr = m - r0 < 64 ? m - r0 : 64;
            for (int r = 0; r < mr; r++) acc[r] = 0.0;
            for (int b = 0; b < nb; b++) {
                q4_1_block(img + ((size_t)n * nb + b) * Q4_1_BYTES, w);
                for (int r = 0; r < mr; r++) {
                    const double* xr = x + (size_t)(r0 + r) * n_in + (size_t)b * Q4_1_BLOCK;
                    double a = acc[r];
                    for (int j = 0; j < Q4_1_BLOCK; j++) a += w[j] * xr[j];
                    acc[r] = a;
                }
            }
            for (int r = 0; r < mr; r++) y[(size_t)(r0 + r) * n_out + n] = acc[r];
        }
    }
}

/* y[r][n] = sum_k W[n][k] x[r][k], W bf16 [n_out][n_in]. */
static void bf16_matmul(const uint16_t* W, int n_out, int n_in, const double* x, int m, double* y) {
#pragma omp parallel for schedule(static)
    for (int n = 0; n < n_out; n++) {
        const uint16_t* row = W + (size_t)n * n_in;
        for (int r = 0; r < m; r++) {
            const double* xr = x + (size_t)r * n_in;
            double a = 0.0;
            for (int k = 0; k < n_in; k++) a += bf16_to_double(row[k]) * xr[k];
            y[(size_t)r * n_out + n] = a;
        }
    }
}

/* Exported forms for the tests: fp32 outputs of the GEMMs above, inputs given as bf16 bits. */
void orc_q4_1_matmul(const uint8_t* img, int n_out, int n_in, const uint16_t* x_bf16, int m, float* y) {
    double* x = malloc(sizeof(double) * (size_t)m * n_in);
    double* yy = malloc(sizeof(double) * (size_t)m * n_out);
    for (size_t i = 0; i < (size_t)m * n_in; i++) x[i] = bf16_to_double(x_bf16[i]);
    q4_1_matmul(img, n_out, n_in, x, m, yy);
    for (size_t i = 0; i < (size_t)m * n_out; i++) y[i] = (float)yy[i];
    free(x);
    free(yy);
}

void orc_bf16_matmul(const uint16_t* W, int n_out, int n_in, const uint16_t* x_bf16, int m, float* y) {
    double* x = malloc(sizeof(double) * (size_t)m * n_in);
    double* yy = malloc(sizeof(double) * (size_t)m * n_out);
    for (size_t i = 0; i < (size_t)m * n_in; i++) x[i] = bf16_to_double(x_bf16[i]);
    bf16_matmul(W, n_out, n_in, x, m, yy);
    for (size_t i = 0; i < (size_t)m * n_out; i++) y[i] = (float)yy[i];
    free(x);
    free(yy);
}

/* ------------------------------------------------------------------------------------------ */
/* Qwen3-style layer pieces ([CARD, "Draft" row]: "Qwen3-style layers"): RMSNorm with a         */
/* multiplicative gain, per-head RMSNorm on q and k, rotate-half RoPE, SwiGLU.                  */
/* ------------------------------------------------------------------------------------------ */

/* out[i] = x[i] / sqrt(mean(x^2) + eps) * g[i] */
static void rmsnorm(const double* x, const uint16_t* g, int n, double eps, double* out) {
    double ss = 0.0;
    for (int i = 0; i < n; i++) ss += x[i] * x[i];
    double r = 1.0 / sqrt(ss / n + eps);
    for (int i = 0; i < n; i++) out[i] = x[i] * r * bf16_to_double(g[i]);
}

/* Rotate-half RoPE at position p: pairs (i, i + hd/2), angle p * base^(-2i/hd). */
static void rope(double* v, int hd, long p, double base) {
    int h = hd / 2;
    for (int i = 0; i < h; i++) {
        double th = (double)p * pow(base, -2.0 * i / hd);
        double c = cos(th), s = sin(th);
        double a = v[i], b = v[i + h];
        v[i] = a * c - b * s;
        v[i + h] = a * s + b * c;
    }
}

static double silu(double g) { return g / (1.0 + exp(-g)); }

void orc_rmsnorm_bf16(const float* x, const uint16_t* g, int n, double eps, uint16_t* out) {
    double* xx = calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    double* o = calloc((size_t)(n > 0 ? n : 1), sizeof(double));
    for (int i = 0; i < n; i++) xx[i] = x[i];
    rmsnorm(xx, g, n, eps, o);
    for (int i = 0; i < n; i++) out[i] = double_to_bf16(o[i]);
    free(xx);
    free(o);
}

void orc_rope(const float* v_in, int hd, long p, double base, float* v_out) {
    double* v = malloc(sizeof(double) * hd);
    for (int i = 0; i < hd; i++) v[i] = v_in[i];
    rope(v, hd, p, base);
    for (int i = 0; i < hd; i++) v_out[i] = (float)v[i];
    free(v);
}

/* ------------------------------------------------------------------------------------------ */
/* model                                                                                        */
/* ------------------------------------------------------------------------------------------ */
typedef struct {
    int attn;        /* 0 sliding, 1 full */
    int n_kv_heads;
    int head_dim;
    int window;      /* sliding: keys j in [p - window + 1, p]; 0 = unlimited */
    int ffn;
    int kv_owner;    /* -1: own plane; else the layer whose plane this one reads */
} orc_layer_desc;

typedef struct {
    const uint8_t *wq, *wk, *wv, *wo, *wg, *wu, *wd;
    const uint16_t *attn_norm, *mlp_norm, *q_norm, *k_norm;
    const uint8_t *ple_gate, *ple_proj;   /* per-layer embedding gate [ple_dim][H], projection [H][ple_dim] */
    const uint16_t* layer_scalar;         /* one bf16 value */
} orc_layer_w;

typedef struct orc_model {
    int n_layers, hidden, n_q_heads, vocab, qk_norm, block_causal, draft_window, n_taps;
    long max_ctx;
    int* tap_layers;
    double rope_base, rms_eps;
    orc_layer_desc* L;
    orc_layer_w* W;
    const uint16_t *embed, *final_norm, *fc, *hidden_norm;
    float** plane;   /* own planes: [max_ctx][2][w] fp32 (K then V); NULL on a shared layer */
    long held;       /* positions held on every own plane */
    long pending;    /* rows appended by the last verify and not yet committed; -1 = none */
    int kv_bf16;     /* planes stored in bf16: every K/V value is rounded (from fp32, RNE) when stored */
    int kv_ring;     /* sliding layers of a verify model keep window + RING_SLACK position slots (ring) */
    int ple_dim;     /* per-layer embedding width (0: the model has none) */
    const uint16_t* ple_table;   /* [vocab][n_layers][ple_dim] bf16 per-layer inputs, indexed by token */
} orc_model;

static long kv_width(const orc_model* md, int l) {
    return (long)md->L[l].n_kv_heads * md->L[l].head_dim;
}

/* Ring planes (a memory variant [PR2303, "What changes" item 1 keeps the per-layer cut semantics]):
 * a sliding layer of a verify model needs at most the last `window` positions plus the rows of the
 * batch in flight, so its plane can hold window + RING_SLACK position slots with position p in slot
 * p mod capacity. RING_SLACK is the most rows one pass appends (16): a pass appending rows
 * P..P+k-1 overwrites positions older than P - window + 1, which no row of the pass and no row
 * after a rollback to P + n (n >= 0) can see. Other planes hold every position (capacity max_ctx). */
#define RING_SLACK 16
static long plane_cap(const orc_model* md, int l) {
    const orc_layer_desc* L = &md->L[l];
    if (md->kv_ring && md->block_causal && L->attn == 0 && L->window > 0 && (long)L->window + RING_SLACK < md->max_ctx)
        return (long)L->window + RING_SLACK;
    return md->max_ctx;
}
static float* plane_row(const orc_model* md, int l, long p) {
    return md->plane[l] + (size_t)(p % plane_cap(md, l)) * 2 * kv_width(md, l);
}
/* Positions a plane holds: every held position on a linear plane; on a ring plane the last
 * `window` of them (older slots may already carry rows of a pass that a commit cut back). */
static long plane_positions(const orc_model* md, int l, long held) {
    const long c = plane_cap(md, l) < md->max_ctx ? md->L[l].window : held;
    return held < c ? held : c;
}

orc_model* orc_model_new(int n_layers, int hidden, int n_q_heads, int vocab, long max_ctx, int qk_norm,
                         double rope_base, double rms_eps, int block_causal, int draft_window,
                         const int* layer_fields /* [n_layers][6] */, const int* tap_layers, int n_taps) {
    orc_model* md = calloc(1, sizeof(orc_model));
    md->n_layers = n_layers;
    md->hidden = hidden;
    md->n_q_heads = n_q_heads;
    md->vocab = vocab;
    md->max_ctx = max_ctx;
    md->qk_norm = qk_norm;
    md->rope_base = rope_base;
    md->rms_eps = rms_eps;
    md->block_causal = block_causal;
    md->draft_window = draft_window;
    md->n_taps = n_taps;
    md->tap_layers = calloc((size_t)(n_taps > 0 ? n_taps : 1), sizeof(int));
    for (int t = 0; t < n_taps; t++) md->tap_layers[t] = tap_layers[t];
    md->L = calloc((size_t)n_layers, sizeof(orc_layer_desc));
    md->W = calloc((size_t)n_layers, sizeof(orc_layer_w));
    md->plane = calloc((size_t)n_layers, sizeof(float*));
    for (int l = 0; l < n_layers; l++) {
        const int* f = layer_fields + 6 * l;
        md->L[l] = (orc_layer_desc){f[0], f[1], f[2], f[3], f[4], f[5]};
        if (md->L[l].kv_owner < 0)
            md->plane[l] = calloc((size_t)max_ctx * 2 * kv_width(md, l), sizeof(float));
    }
    md->pending = -1;
    return md;
}

void orc_model_free(orc_model* md) {
    if (!md) return;
    for (int l = 0; l < md->n_layers; l++) free(md->plane[l]);
    free(md->plane);
    free(md->L);
    free(md->W);
    free(md->tap_layers);
    free(md);
}

void orc_set_layer(orc_model* md, int l, const uint8_t* wq, const uint8_t* wk, const uint8_t* wv,
                   const uint8_t* wo, const uint8_t* wg, const uint8_t* wu, const uint8_t* wd,
                   const uint16_t* attn_norm, const uint16_t* mlp_norm, const uint16_t* q_norm,
                   const uint16_t* k_norm) {
    md->W[l] = (orc_layer_w){wq, wk, wv, wo, wg, wu, wd, attn_norm, mlp_norm, q_norm, k_norm, NULL, NULL, NULL};
}

/* Per-layer embeddings (PLE) [PR2303, "What changes": the batched body builds every row's per-layer
 * inputs and runs the PLE gate and projection as M-row GEMMs, then the layer scalar]. */
void orc_set_ple(orc_model* md, int ple_dim, const uint16_t* table) {
    md->ple_dim = ple_dim;
    md->ple_table = table;
}
void orc_set_layer_ple(orc_model* md, int l, const uint8_t* gate, const uint8_t* proj, const uint16_t* scalar) {
    md->W[l].ple_gate = gate;
    md->W[l].ple_proj = proj;
    md->W[l].layer_scalar = scalar;
}

void orc_set_globals(orc_model* md, const uint16_t* embed, const uint16_t* final_norm,
                     const uint16_t* fc, const uint16_t* hidden_norm) {
    md->embed = embed;
    md->final_norm = final_norm;
    md->fc = fc;
    md->hidden_norm = hidden_norm;
}

/* Cached context: every own plane gets `positions` rows [positions][2][w_l]. */
/* bf16 K/V planes (a memory variant of the planes the pages keep as floats, [PR2303] "What changes"
 * item 1): the stored value is the fp32 value rounded to bf16 (RNE); everything else is unchanged. */
void orc_set_kv_bf16(orc_model* md, int on) { md->kv_bf16 = on; }

/* Ring planes on (before any K/V is set): the sliding planes shrink to their ring capacity. */
void orc_set_kv_ring(orc_model* md, int on) {
    md->kv_ring = on;
    for (int l = 0; l < md->n_layers; l++) {
        if (!md->plane[l]) continue;
        free(md->plane[l]);
        md->plane[l] = calloc((size_t)plane_cap(md, l) * 2 * kv_width(md, l), sizeof(float));
    }
}
long orc_plane_capacity(const orc_model* md, int l) { return plane_cap(md, l); }

static float store_kv(const orc_model* md, double v) {
    const float f = (float)v;
    return md->kv_bf16 ? (float)round_bf16((double)f) : f;
}

int orc_set_kv(orc_model* md, int l, const float* kv, long positions) {
    if (l < 0 || l >= md->n_layers || !md->plane[l] || positions > md->max_ctx) return 1;
    const long w = kv_width(md, l);
    const long keep = positions < plane_cap(md, l) ? positions : plane_cap(md, l);
    for (long p = positions - keep; p < positions; p++) {
        float* row = plane_row(md, l, p);
        for (long i = 0; i < 2 * w; i++) row[i] = store_kv(md, kv[(size_t)p * 2 * w + i]);
    }
    return 0;
}

void orc_set_held(orc_model* md, long positions) {
    md->held = positions;
    md->pending = -1;
}

long orc_positions_held(const orc_model* md) { return md->held; }

const float* orc_plane(const orc_model* md, int l) { return md->plane[l]; }

/* [PR2303, "What changes" item 1 and the reviewer guide]: the KV row width is per layer. A shared
 * layer reads its owner's plane at the owner's width and holds no plane of its own. */
void orc_kv_widths(const orc_model* md, long* out) {
    for (int l = 0; l < md->n_layers; l++) {
        int src = md->L[l].kv_owner < 0 ? l : md->L[l].kv_owner;
        out[l] = kv_width(md, src);
    }
}

/* Floats held per plane: held positions x 2 x w_l on an own plane; 0 on a shared plane. */
void orc_plane_floats(const orc_model* md, long* out) {
    for (int l = 0; l < md->n_layers; l++)
        out[l] = md->L[l].kv_owner < 0 ? plane_positions(md, l, md->held) * 2 * kv_width(md, l) : 0;
}

/* Per-plane cut with the extrapolation rule of [PR2303, review "VERDICT at 4d10370: READY"]: plane i
 * is cut at per[i]; a plane past the end of the list is cut at the list's last entry. */
long orc_cut_floats(const long* per, int n_per, int plane, long positions) {
    long w = per[plane < n_per ? plane : n_per - 1];
    return positions * 2 * w;
}

/* ---- one layer over a set of rows (layer-major batched order) ------------------------------- */

/* Attention of one row at position p on layer l, all query heads: q [Hq][hd] (normalised, roped);
 * out [Hq][hd] before the bf16 rounding. Keys j in [lo, p] of the own plane or, on a KV-shared
 * layer, of the owner's plane [PR2303, "What changes": a KV-shared layer reads its owner layer's
 * cache and appends nothing]; lo = p - window + 1 on a sliding layer, else 0. Query head h reads
 * KV head h / (Hq / NKV). */
static void attend_row(const orc_model* md, int l, const double* q, long p, double* out) {
    const orc_layer_desc* Ld = &md->L[l];
    const int hd = Ld->head_dim, Hq = md->n_q_heads, nkv = Ld->n_kv_heads;
    const int src = Ld->kv_owner < 0 ? l : Ld->kv_owner;
    const long w = kv_width(md, src);
    const int group = Hq / nkv;
    long lo = 0;
    if (Ld->attn == 0 && Ld->window > 0 && p - Ld->window + 1 > 0) lo = p - Ld->window + 1;
    const long nk = p - lo + 1;
    double* sc = malloc(sizeof(double) * (size_t)nk);
    for (int h = 0; h < Hq; h++) {
        const int g = h / group;
        const double* qh = q + (size_t)h * hd;
        double mx = -INFINITY;
        for (long j = lo; j <= p; j++) {
            const float* kj = plane_row(md, src, j) + (size_t)g * hd;
            double s = 0.0;
            for (int i = 0; i < hd; i++) s += qh[i] * kj[i];
            s /= sqrt((double)hd);
            sc[j - lo] = s;
            if (s > mx) mx = s;
        }
        double z = 0.0;
        for (long j = 0; j < nk; j++) {
            sc[j] = exp(sc[j] - mx);
            z += sc[j];
        }
        for (int i = 0; i < hd; i++) {
            double acc = 0.0;
            for (long j = lo; j <= p; j++) acc += sc[j - lo] * plane_row(md, src, j)[w + (size_t)g * hd + i];
            out[(size_t)h * hd + i] = acc / z;
        }
    }
    free(sc);
}

/* Test hook: attention of one row (q given as fp32) against the current planes. */
void orc_attend(const orc_model* md, int l, const float* q_in, long p, double* out) {
    const int qd = md->n_q_heads * md->L[l].head_dim;
    double* q = malloc(sizeof(double) * qd);
    for (int i = 0; i < qd; i++) q[i] = q_in[i];
    attend_row(md, l, q, p, out);
    free(q);
}

/* x: [m][H] residual rows (fp32 values); pos[r]: position of row r. The rows run one after another
 * through the attention half (append at pos[r], then attend over j <= pos[r]), so a batch of rows
 * computes exactly what the same rows do as sequential single steps [PR2303, "Proof": k batched
 * rows bit-identical to k sequential steps]. */
static void target_layer(orc_model* md, int l, int m, double* x, const long* pos, const int* tokens) {
    const orc_layer_desc* Ld = &md->L[l];
    const orc_layer_w* W = &md->W[l];
    const int H = md->hidden, hd = Ld->head_dim, Hq = md->n_q_heads;
    const int qd = Hq * hd, nkv = Ld->n_kv_heads, kvd = nkv * hd;
    const int own = Ld->kv_owner < 0;
    const int src = own ? l : Ld->kv_owner;
    const long w = kv_width(md, src);
    double* a = malloc(sizeof(double) * (size_t)m * H);
    double* q = malloc(sizeof(double) * (size_t)m * qd);
    double* kx = malloc(sizeof(double) * (size_t)m * kvd);
    double* vx = malloc(sizeof(double) * (size_t)m * kvd);
    double* o = malloc(sizeof(double) * (size_t)m * qd);
    double* y = malloc(sizeof(double) * (size_t)m * (H > qd ? H : qd));
    double* t = malloc(sizeof(double) * (size_t)(H > hd ? H : hd));

    /* attention half */
    for (int r = 0; r < m; r++) {
        rmsnorm(x + (size_t)r * H, W->attn_norm, H, md->rms_eps, t);
        for (int i = 0; i < H; i++) a[(size_t)r * H + i] = round_bf16(t[i]);
    }
    q4_1_matmul(W->wq, qd, H, a, m, q);
    for (size_t i = 0; i < (size_t)m * qd; i++) q[i] = round_f32(q[i]);
    if (own) {
        q4_1_matmul(W->wk, kvd, H, a, m, kx);
        q4_1_matmul(W->wv, kvd, H, a, m, vx);
        for (size_t i = 0; i < (size_t)m * kvd; i++) {
            kx[i] = round_f32(kx[i]);
            vx[i] = round_f32(vx[i]);
        }
    }
    for (int r = 0; r < m; r++) {
        const long p = pos[r];
        for (int h = 0; h < Hq; h++) {
            double* qh = q + (size_t)r * qd + (size_t)h * hd;
            if (md->qk_norm) {
                rmsnorm(qh, W->q_norm, hd, md->rms_eps, t);
                memcpy(qh, t, sizeof(double) * hd);
            }
            rope(qh, hd, p, md->rope_base);
            for (int i = 0; i < hd; i++) qh[i] = round_f32(qh[i]);
        }
        if (own) {
            float* row = plane_row(md, l, p);
            for (int g = 0; g < nkv; g++) {
                double* kh = kx + (size_t)r * kvd + (size_t)g * hd;
                if (md->qk_norm) {
                    rmsnorm(kh, W->k_norm, hd, md->rms_eps, t);
                    memcpy(kh, t, sizeof(double) * hd);
                }
                rope(kh, hd, p, md->rope_base);
                for (int i = 0; i < hd; i++) {
                    row[g * hd + i] = store_kv(md, kh[i]);
                    row[w + g * hd + i] = store_kv(md, vx[(size_t)r * kvd + (size_t)g * hd + i]);
                }
            }
        }
        attend_row(md, l, q + (size_t)r * qd, p, o + (size_t)r * qd);
        for (int i = 0; i < qd; i++) o[(size_t)r * qd + i] = round_bf16(o[(size_t)r * qd + i]);
    }
    q4_1_matmul(W->wo, H, qd, o, m, y);
    for (size_t i = 0; i < (size_t)m * H; i++) x[i] = round_f32(x[i] + round_f32(y[i]));

    /* MLP half: x += Wd (silu(Wg b) * (Wu b)) */
    const int F = Ld->ffn;
    double* b = a;
    double* gg = malloc(sizeof(double) * (size_t)m * F);
    double* uu = malloc(sizeof(double) * (size_t)m * F);
    for (int r = 0; r < m; r++) {
        rmsnorm(x + (size_t)r * H, W->mlp_norm, H, md->rms_eps, t);
        for (int i = 0; i < H; i++) b[(size_t)r * H + i] = round_bf16(t[i]);
    }
    q4_1_matmul(W->wg, F, H, b, m, gg);
    q4_1_matmul(W->wu, F, H, b, m, uu);
    for (size_t i = 0; i < (size_t)m * F; i++) gg[i] = round_bf16(silu(round_f32(gg[i])) * round_f32(uu[i]));
    q4_1_matmul(W->wd, H, F, gg, m, y);
    for (size_t i = 0; i < (size_t)m * H; i++) x[i] = round_f32(x[i] + round_f32(y[i]));

    /* PLE tail: the gate reads the layer's output rows, u = Wg . bf16(x); the per-layer input p of the
     * row's token (row l of its table entry) multiplies silu(u); the projection adds Wp . bf16(silu(u) p)
     * to the residual stream, which the layer scalar then scales. */
    if (md->ple_dim > 0) {
        const int D = md->ple_dim;
        double* u = malloc(sizeof(double) * (size_t)m * D);
        for (size_t i = 0; i < (size_t)m * H; i++) a[i] = round_bf16(x[i]);
        q4_1_matmul(W->ple_gate, D, H, a, m, u);
        for (int r = 0; r < m; r++) {
            const uint16_t* p = md->ple_table + ((size_t)tokens[r] * md->n_layers + l) * D;
            for (int j = 0; j < D; j++)
                u[(size_t)r * D + j] = round_bf16(silu(round_f32(u[(size_t)r * D + j])) * bf16_to_double(p[j]));
        }
        q4_1_matmul(W->ple_proj, H, D, u, m, y);
        const double sc = bf16_to_double(W->layer_scalar[0]);
        for (size_t i = 0; i < (size_t)m * H; i++) x[i] = round_f32(round_f32(x[i] + round_f32(y[i])) * sc);
        free(u);
    }

    free(a); free(q); free(kx); free(vx); free(o); free(y); free(t); free(gg); free(uu);
}

/* Test hook: one layer over m rows at positions pos (appends on an own layer like a verify).
 * Refused (4) on a PLE model: injected rows carry no token ids for the per-layer inputs. */
int orc_layer_forward(orc_model* md, int l, int m, const float* x_in, const long* pos, float* x_out) {
    if (md->ple_dim > 0) return 4;
    double* x = malloc(sizeof(double) * (size_t)m * md->hidden);
    for (size_t i = 0; i < (size_t)m * md->hidden; i++) x[i] = x_in[i];
    target_layer(md, l, m, x, pos, NULL);
    for (size_t i = 0; i < (size_t)m * md->hidden; i++) x_out[i] = (float)x[i];
    free(x);
    return 0;
}

/* logits[r] = Head . bf16(rmsnorm(x[r]) * g_final); the head is the tied bf16 embedding table. */
static void head_logits(const orc_model* target, const uint16_t* final_norm, int m, const double* x,
                        float* logits) {
    const int H = target->hidden, V = target->vocab;
    double* a = malloc(sizeof(double) * (size_t)m * H);
    double* t = malloc(sizeof(double) * H);
    double* y = malloc(sizeof(double) * (size_t)m * V);
    for (int r = 0; r < m; r++) {
        rmsnorm(x + (size_t)r * H, final_norm, H, target->rms_eps, t);
        for (int i = 0; i < H; i++) a[(size_t)r * H + i] = round_bf16(t[i]);
    }
    bf16_matmul(target->embed, V, H, a, m, y);
    for (size_t i = 0; i < (size_t)m * V; i++) logits[i] = (float)y[i];
    free(a); free(t); free(y);
}

/* Run rows x0 [m][H] (fp32 residual rows) through every layer in layer-major order.
 * taps: [m][n_taps][H] bf16 or NULL ([CARD, "Taps" row]: zero-based layer outputs). */
static void forward_x(orc_model* md, const double* x0, int m, const long* pos, const int* tokens, float* logits,
                      uint16_t* taps) {
    const int H = md->hidden;
    double* x = malloc(sizeof(double) * (size_t)m * H);
    memcpy(x, x0, sizeof(double) * (size_t)m * H);
    for (int l = 0; l < md->n_layers; l++) {
        target_layer(md, l, m, x, pos, tokens);
        for (int ti = 0; ti < md->n_taps; ti++) {
            if (md->tap_layers[ti] != l || !taps) continue;
            for (int r = 0; r < m; r++)
                for (int i = 0; i < H; i++)
                    taps[((size_t)r * md->n_taps + ti) * H + i] = double_to_bf16(x[(size_t)r * H + i]);
        }
    }
    if (logits) head_logits(md, md->final_norm, m, x, logits);
    free(x);
}

/* The rows of the tied embedding table for the tokens. */
static void forward_rows(orc_model* md, const int* tokens, int m, const long* pos, float* logits,
                         uint16_t* taps) {
    const int H = md->hidden;
    double* x = malloc(sizeof(double) * (size_t)m * H);
    for (int r = 0; r < m; r++)
        for (int i = 0; i < H; i++) x[(size_t)r * H + i] = bf16_to_double(md->embed[(size_t)tokens[r] * H + i]);
    forward_x(md, x, m, pos, tokens, logits, taps);
    free(x);
}

/* A verify whose rows enter as given residual rows x0 [k][H] instead of token embeddings (the
 * injected-embedding form of a batch). Test hook: it lets a test perturb the entry rows. */
int orc_verify_embedded(orc_model* md, const float* x0, int k, float* logits_all, uint16_t* taps) {
    if (k < 1) return 1;
    if (md->ple_dim > 0) return 4;   /* injected rows carry no token ids for the per-layer inputs [PR2303] */
    if (md->held + k > md->max_ctx) return 3;
    long* pos = malloc(sizeof(long) * k);
    double* x = malloc(sizeof(double) * (size_t)k * md->hidden);
    for (int r = 0; r < k; r++) pos[r] = md->held + r;
    for (size_t i = 0; i < (size_t)k * md->hidden; i++) x[i] = x0[i];
    forward_x(md, x, k, pos, NULL, logits_all, taps);
    free(pos);
    free(x);
    md->held += k;
    md->pending = k;
    return 0;
}

/* One decode step: the token at position `held`; appends one position. */
int orc_step(orc_model* md, int token, float* logits, uint16_t* taps) {
    if (md->held + 1 > md->max_ctx) return 3;
    long p = md->held;
    forward_rows(md, &token, 1, &p, logits, taps);
    md->held += 1;
    md->pending = -1;
    return 0;
}

/* Batched verify [PR2303, "What changes"]: all k rows go through every layer in one pass; every
 * row's logits are returned ([PR2303] item 2: logits_all holds every row). The k rows stay appended
 * until commit_verify_rows cuts them back. */
int orc_verify_batch(orc_model* md, const int* tokens, int k, float* logits_all, uint16_t* taps) {
    if (k < 1) return 1;
    if (md->held + k > md->max_ctx) return 3;
    long* pos = malloc(sizeof(long) * k);
    for (int r = 0; r < k; r++) pos[r] = md->held + r;
    forward_rows(md, tokens, k, pos, logits_all, taps);
    free(pos);
    md->held += k;
    md->pending = k;
    return 0;
}

/* [PR2303, "What changes" item 1, "Proof"]: after a verify of k rows keep n of them on every plane:
 * positions held = (held before the verify) + n; shared planes stay empty. */
int orc_commit_verify_rows(orc_model* md, int n) {
    if (md->pending < 0) return 2;
    if (n < 0 || n > md->pending) return 2;
    md->held = md->held - md->pending + n;
    md->pending = -1;
    return 0;
}

/* extend_context [PR2303, "What changes" item 1: snapshot, restore, the verify rollback and
 * extend_context counted every layer at NKV * HD; the count is per layer]. Appends n positions of
 * given K/V rows to every own plane at the held count, each at that layer's own width: kv_all is
 * the own planes' new rows one after the other in layer order, [n][2][w_l] fp32 each (K already
 * normalised and rotated, as for a cached context). Shared planes stay empty. positions held += n.
 * Refused (2, no state change) while a verify is pending; (3) past max_ctx. */
int orc_extend_context(orc_model* md, const float* kv_all, long n) {
    if (md->pending >= 0) return 2;
    if (n < 0 || md->held + n > md->max_ctx) return 3;
    size_t off = 0;
    for (int l = 0; l < md->n_layers; l++) {
        if (!md->plane[l]) continue;
        const long w = kv_width(md, l);
        for (long r = 0; r < n; r++) {
            float* dst = plane_row(md, l, md->held + r);
            for (long i = 0; i < 2 * w; i++) dst[i] = store_kv(md, kv_all[off + (size_t)r * 2 * w + i]);
        }
        off += (size_t)n * 2 * w;
    }
    md->held += n;
    return 0;
}

/* Greedy longest-prefix accept [CARD, "How it is used"; PR2236, the acceptance tool]: row i's
 * greedy token is the first index of the row's maximum (NaN never wins); draft d_m = tokens[m] is
 * kept while it equals the greedy token of row m-1. Emits d_1..d_a and the target's own y_a. */
static int argmax_row(const float* v, int n) {
    int best = -1;
    for (int i = 0; i < n; i++) {
        if (isnan(v[i])) continue;
        if (best < 0 || v[i] > v[best]) best = i;
    }
    return best < 0 ? 0 : best;
}

int orc_argmax(const float* v, int n) { return argmax_row(v, n); }

int orc_accept_greedy(const float* logits_all, int k, int V, const int* tokens, int* out_tokens,
                      int* n_accepted) {
    int a = 0;
    while (a < k - 1 && tokens[a + 1] == argmax_row(logits_all + (size_t)a * V, V)) a++;
    for (int i = 0; i < a; i++) out_tokens[i] = tokens[i + 1];
    out_tokens[a] = argmax_row(logits_all + (size_t)a * V, V);
    *n_accepted = a;
    return 0;
}

/* ---- sampled verify (temperature T > 0) ---------------------------------------------------
 * [CARD, "How it is used"]: with a sampler every position is sampled and compared with the draft,
 * so the output distribution is the target's. Reading (the pages name no sampler): row i's token
 * y_i is a draw from softmax(z_i / T); draft d_m is kept while it equals y_{m-1}; the emitted
 * tokens are d_1..d_a and y_a -- the greedy accept with the argmax replaced by the draw.
 * The draw is the Gumbel-max method: the index of the largest z_ij / T + g_ij, with g = -log(-log u)
 * and u_ij uniform on (0, 1), is distributed as softmax(z_i / T).
 * The uniforms come from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3", SC 2011) under key (seed bits 0-31, 32-63) and
 * counter (j / 4, i, offset bits 0-31, 32-63): x = output word j % 4, u = (floor(x / 2^9) + 1/2) / 2^23,
 * every value of which is exact in fp32 and lies in [2^-24, 1 - 2^-24], so g is finite. The decision
 * is taken in fp32, the kernel's precision: inv_t = 1 / T rounded to fp32, score = fmaf(z, inv_t, g)
 * with g = -logf(-logf(u)); the first index of the maximum wins; NaN scores never win. */
static void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; r++) {
        if (r > 0) {   /* the key is bumped by the Weyl constants before every round after the first */
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

void orc_philox4x32_10(const uint32_t* ctr, const uint32_t* key, uint32_t* out) { philox4x32_10(ctr, key, out); }

/* the Gumbel noise of one generator word */
static float gumbel_of_word(uint32_t x) {
    const float u = ((float)(x >> 9) + 0.5f) * (1.0f / 8388608.0f);
    return -logf(-logf(u));
}

float orc_gumbel_of_word(uint32_t x) { return gumbel_of_word(x); }

/* fp32 scores z_ij / T + g_ij of row i (V entries) */
void orc_sample_scores(const float* z, int V, float temperature, uint64_t seed, uint64_t offset, int row,
                       float* scores) {
    const float inv_t = 1.0f / temperature;
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    for (int q = 0; q * 4 < V; q++) {
        const uint32_t ctr[4] = {(uint32_t)q, (uint32_t)row, (uint32_t)offset, (uint32_t)(offset >> 32)};
        uint32_t x[4];
        philox4x32_10(ctr, key, x);
        for (int w = 0; w < 4 && 4 * q + w < V; w++) {
            scores[4 * q + w] = fmaf(z[4 * q + w], inv_t, gumbel_of_word(x[w]));
        }
    }
}

/* the draws of k rows (row index i of the counter = row i) */
void orc_sample_rows(const float* z, int k, int V, float temperature, uint64_t seed, uint64_t offset, int* y) {
    float* sc = (float*)malloc(sizeof(float) * (size_t)V);
    for (int i = 0; i < k; i++) {
        orc_sample_scores(z + (size_t)i * V, V, temperature, seed, offset, i, sc);
        y[i] = argmax_row(sc, V);
    }
    free(sc);
}

int orc_accept_sampled(const float* logits_all, int k, int V, const int* tokens, float temperature, uint64_t seed,
                       uint64_t offset, int* out_tokens, int* n_accepted, int* draws) {
    int* y = (int*)malloc(sizeof(int) * (size_t)k);
    orc_sample_rows(logits_all, k, V, temperature, seed, offset, y);
    int a = 0;
    while (a < k - 1 && tokens[a + 1] == y[a]) a++;
    for (int i = 0; i < a; i++) out_tokens[i] = tokens[i + 1];
    out_tokens[a] = y[a];
    *n_accepted = a;
    if (draws) memcpy(draws, y, sizeof(int) * (size_t)k);
    free(y);
    return 0;
}

/* ---- snapshot / restore with per-layer widths [PR2303, "What changes" item 1] -------------- */
typedef struct orc_snapshot {
    int n_layers;
    long held;
    long* per;       /* width of each plane (shared: the owner's) */
    long* cap;       /* position capacity of each plane (ring planes: window + RING_SLACK) */
    long* kept;      /* positions kept of each plane: held, or on a ring plane the last min(held, window) */
    int* shared;
    float** data;    /* kept x 2 x per[l] floats of each own plane, in position order; NULL on a shared plane */
} orc_snapshot;

/* A snapshot is taken of committed state only: while a verify is pending (its rows not yet cut by
 * commit_verify_rows) it is refused (NULL) and nothing changes. */
orc_snapshot* orc_snapshot_take(const orc_model* md) {
    if (md->pending >= 0) return NULL;
    orc_snapshot* s = calloc(1, sizeof(orc_snapshot));
    s->n_layers = md->n_layers;
    s->held = md->held;
    s->per = calloc((size_t)md->n_layers, sizeof(long));
    s->cap = calloc((size_t)md->n_layers, sizeof(long));
    s->kept = calloc((size_t)md->n_layers, sizeof(long));
    s->shared = calloc((size_t)md->n_layers, sizeof(int));
    s->data = calloc((size_t)md->n_layers, sizeof(float*));
    orc_kv_widths(md, s->per);
    for (int l = 0; l < md->n_layers; l++) {
        s->shared[l] = md->L[l].kv_owner >= 0;
        s->cap[l] = plane_cap(md, s->shared[l] ? md->L[l].kv_owner : l);
        if (s->shared[l]) continue;
        s->kept[l] = plane_positions(md, l, md->held);
        const long nf = orc_cut_floats(s->per, md->n_layers, l, s->kept[l]);
        s->data[l] = malloc(sizeof(float) * (size_t)(nf > 0 ? nf : 1));
        const long row = 2 * s->per[l];
        for (long i = 0; i < s->kept[l]; i++)
            memcpy(s->data[l] + (size_t)i * row, plane_row(md, l, md->held - s->kept[l] + i), sizeof(float) * (size_t)row);
    }
    return s;
}

long orc_snapshot_floats(const orc_snapshot* s, int l) {
    return s->shared[l] ? 0 : orc_cut_floats(s->per, s->n_layers, l, s->kept[l]);
}

int orc_snapshot_restore(orc_model* md, const orc_snapshot* s) {
    if (s->n_layers != md->n_layers) return 1;
    long* w = calloc((size_t)md->n_layers, sizeof(long));
    orc_kv_widths(md, w);
    for (int l = 0; l < md->n_layers; l++)
        if (w[l] != s->per[l] || s->shared[l] != (md->L[l].kv_owner >= 0) ||
            s->cap[l] != plane_cap(md, s->shared[l] ? md->L[l].kv_owner : l)) { free(w); return 1; }
    for (int l = 0; l < md->n_layers; l++) {
        if (s->shared[l]) continue;
        const long row = 2 * w[l];
        for (long i = 0; i < s->kept[l]; i++)
            memcpy(plane_row(md, l, s->held - s->kept[l] + i), s->data[l] + (size_t)i * row, sizeof(float) * (size_t)row);
    }
    free(w);
    md->held = s->held;
    md->pending = -1;
    return 0;
}

void orc_snapshot_free(orc_snapshot* s) {
    if (!s) return;
    for (int l = 0; l < s->n_layers; l++) free(s->data[l]);
    free(s->data);
    free(s->per);
    free(s->cap);
    free(s->kept);
    free(s->shared);
    free(s);
}

/* ------------------------------------------------------------------------------------------ */
/* DFlash draft ([CARD, "Draft", "Taps", "How it is used"]; [PR2236, the acceptance tool's     */
/* header]). Context = the tapped target rows of positions < s, fused by fc and normalised; it   */
/* enters every draft layer as keys/values. Block = [token s, mask, ...] embeddings times the     */
/* embedding scale at positions s..s+B-1; block rows see each other (no causal mask) and the     */
/* context rows inside the window; rows 1..B-1 go through the target's head.                    */
/* ------------------------------------------------------------------------------------------ */

/* Append context rows for positions held..held+n-1 from their taps [n][T][H] bf16. */
int orc_draft_append(orc_model* dr, const uint16_t* taps, int n) {
    const int H = dr->hidden, T = dr->n_taps;
    if (dr->held + n > dr->max_ctx) return 3;
    double* in = malloc(sizeof(double) * (size_t)n * T * H);
    double* f = malloc(sizeof(double) * (size_t)n * H);
    double* c = malloc(sizeof(double) * (size_t)n * H);
    double* t = malloc(sizeof(double) * H);
    for (size_t i = 0; i < (size_t)n * T * H; i++) in[i] = bf16_to_double(taps[i]);
    bf16_matmul(dr->fc, H, T * H, in, n, f);
    for (int r = 0; r < n; r++) {
        for (int i = 0; i < H; i++) f[(size_t)r * H + i] = round_f32(f[(size_t)r * H + i]);
        rmsnorm(f + (size_t)r * H, dr->hidden_norm, H, dr->rms_eps, t);
        for (int i = 0; i < H; i++) c[(size_t)r * H + i] = round_bf16(t[i]);
    }
    for (int l = 0; l < dr->n_layers; l++) {
        const orc_layer_desc* Ld = &dr->L[l];
        const int hd = Ld->head_dim, nkv = Ld->n_kv_heads, kvd = nkv * hd;
        const long w = kv_width(dr, l);
        double* kx = malloc(sizeof(double) * (size_t)n * kvd);
        double* vx = malloc(sizeof(double) * (size_t)n * kvd);
        double* u = malloc(sizeof(double) * hd);
        q4_1_matmul(dr->W[l].wk, kvd, H, c, n, kx);
        q4_1_matmul(dr->W[l].wv, kvd, H, c, n, vx);
        for (int r = 0; r < n; r++) {
            const long p = dr->held + r;
            float* row = dr->plane[l] + (size_t)p * 2 * w;
            for (int g = 0; g < nkv; g++) {
                double* kh = kx + (size_t)r * kvd + (size_t)g * hd;
                for (int i = 0; i < hd; i++) kh[i] = round_f32(kh[i]);
                if (dr->qk_norm) {
                    rmsnorm(kh, dr->W[l].k_norm, hd, dr->rms_eps, u);
                    memcpy(kh, u, sizeof(double) * hd);
                }
                rope(kh, hd, p, dr->rope_base);
                for (int i = 0; i < hd; i++) {
                    row[g * hd + i] = store_kv(dr, kh[i]);
                    row[w + g * hd + i] = store_kv(dr, round_f32(vx[(size_t)r * kvd + (size_t)g * hd + i]));
                }
            }
        }
        free(kx); free(vx); free(u);
    }
    dr->held += n;
    free(in); free(f); free(c); free(t);
    return 0;
}

static int draft_block_x(orc_model* dr, const orc_model* target, int B, double* x, int* proposals, float* logits);

/* The block forward. Block size B (<= 16); proposals[B-1]; logits (optional) [B-1][V]. */
int orc_draft_block(orc_model* dr, const orc_model* target, int B, int last_token, double embedding_scale,
                    int mask_token, int* proposals, float* logits) {
    const int H = dr->hidden;
    if (B < 2 || B > 16) return 1;
    double* x = malloc(sizeof(double) * (size_t)B * H);
    for (int i = 0; i < B; i++) {
        const int tok = i == 0 ? last_token : mask_token;
        for (int j = 0; j < H; j++)
            x[(size_t)i * H + j] = round_f32(bf16_to_double(target->embed[(size_t)tok * H + j]) * embedding_scale);
    }
    return draft_block_x(dr, target, B, x, proposals, logits);
}

/* Test hook: the block forward from given block rows x0 [B][H] (fp32). */
int orc_draft_block_embedded(orc_model* dr, const orc_model* target, int B, const float* x0, int* proposals,
                             float* logits) {
    if (B < 2 || B > 16) return 1;
    double* x = malloc(sizeof(double) * (size_t)B * dr->hidden);
    for (size_t i = 0; i < (size_t)B * dr->hidden; i++) x[i] = x0[i];
    return draft_block_x(dr, target, B, x, proposals, logits);
}

/* The draft layers, final norm and target head over the block rows x [B][H] (consumed). */
static int draft_block_x(orc_model* dr, const orc_model* target, int B, double* x, int* proposals, float* logits) {
    const int H = dr->hidden, Hq = dr->n_q_heads;
    const long s = dr->held;
    long lo = 0;
    if (dr->draft_window > 0 && s - dr->draft_window > 0) lo = s - dr->draft_window;
    for (int l = 0; l < dr->n_layers; l++) {
        const orc_layer_desc* Ld = &dr->L[l];
        const orc_layer_w* W = &dr->W[l];
        const int hd = Ld->head_dim, nkv = Ld->n_kv_heads, kvd = nkv * hd, qd = Hq * hd;
        const int group = Hq / nkv;
        const long w = kv_width(dr, l);
        double* a = malloc(sizeof(double) * (size_t)B * H);
        double* q = malloc(sizeof(double) * (size_t)B * qd);
        double* kx = malloc(sizeof(double) * (size_t)B * kvd);
        double* vx = malloc(sizeof(double) * (size_t)B * kvd);
        double* o = malloc(sizeof(double) * (size_t)B * qd);
        double* y = malloc(sizeof(double) * (size_t)B * (H > qd ? H : qd));
        double* t = malloc(sizeof(double) * (size_t)(H > hd ? H : hd));
        for (int r = 0; r < B; r++) {
            rmsnorm(x + (size_t)r * H, W->attn_norm, H, dr->rms_eps, t);
            for (int i = 0; i < H; i++) a[(size_t)r * H + i] = round_bf16(t[i]);
        }
        q4_1_matmul(W->wq, qd, H, a, B, q);
        q4_1_matmul(W->wk, kvd, H, a, B, kx);
        q4_1_matmul(W->wv, kvd, H, a, B, vx);
        for (int r = 0; r < B; r++) {
            const long p = s + r;
            for (int h = 0; h < Hq; h++) {
                double* qh = q + (size_t)r * qd + (size_t)h * hd;
                for (int i = 0; i < hd; i++) qh[i] = round_f32(qh[i]);
                if (dr->qk_norm) {
                    rmsnorm(qh, W->q_norm, hd, dr->rms_eps, t);
                    memcpy(qh, t, sizeof(double) * hd);
                }
                rope(qh, hd, p, dr->rope_base);
                for (int i = 0; i < hd; i++) qh[i] = round_f32(qh[i]);
            }
            for (int g = 0; g < nkv; g++) {
                double* kh = kx + (size_t)r * kvd + (size_t)g * hd;
                for (int i = 0; i < hd; i++) kh[i] = round_f32(kh[i]);
                if (dr->qk_norm) {
                    rmsnorm(kh, W->k_norm, hd, dr->rms_eps, t);
                    memcpy(kh, t, sizeof(double) * hd);
                }
                rope(kh, hd, p, dr->rope_base);
                for (int i = 0; i < hd; i++) {   /* the block's rows are read as stored rows are */
                    kh[i] = store_kv(dr, kh[i]);
                    vx[(size_t)r * kvd + (size_t)g * hd + i] = store_kv(dr, round_f32(vx[(size_t)r * kvd + (size_t)g * hd + i]));
                }
            }
        }
        const float* P = dr->plane[l];
        const long nctx = s - lo;
        double* sc = malloc(sizeof(double) * (size_t)(nctx + B));
        for (int r = 0; r < B; r++) {
            for (int h = 0; h < Hq; h++) {
                const int g = h / group;
                const double* qh = q + (size_t)r * qd + (size_t)h * hd;
                double mx = -INFINITY;
                for (long j = 0; j < nctx + B; j++) {
                    double sdot = 0.0;
                    for (int i = 0; i < hd; i++) {
                        double kv = j < nctx ? (double)P[(size_t)(lo + j) * 2 * w + (size_t)g * hd + i]
                                             : kx[(size_t)(j - nctx) * kvd + (size_t)g * hd + i];
                        sdot += qh[i] * kv;
                    }
                    sc[j] = sdot / sqrt((double)hd);
                    if (sc[j] > mx) mx = sc[j];
                }
                double z = 0.0;
                for (long j = 0; j < nctx + B; j++) {
                    sc[j] = exp(sc[j] - mx);
                    z += sc[j];
                }
                for (int i = 0; i < hd; i++) {
                    double acc = 0.0;
                    for (long j = 0; j < nctx + B; j++) {
                        double vv = j < nctx ? (double)P[(size_t)(lo + j) * 2 * w + w + (size_t)g * hd + i]
                                             : vx[(size_t)(j - nctx) * kvd + (size_t)g * hd + i];
                        acc += sc[j] * vv;
                    }
                    o[(size_t)r * qd + (size_t)h * hd + i] = round_bf16(acc / z);
                }
            }
        }
        free(sc);
        q4_1_matmul(W->wo, H, qd, o, B, y);
        for (size_t i = 0; i < (size_t)B * H; i++) x[i] = round_f32(x[i] + round_f32(y[i]));
        const int F = Ld->ffn;
        double* gg = malloc(sizeof(double) * (size_t)B * F);
        double* uu = malloc(sizeof(double) * (size_t)B * F);
        for (int r = 0; r < B; r++) {
            rmsnorm(x + (size_t)r * H, W->mlp_norm, H, dr->rms_eps, t);
            for (int i = 0; i < H; i++) a[(size_t)r * H + i] = round_bf16(t[i]);
        }
        q4_1_matmul(W->wg, F, H, a, B, gg);
        q4_1_matmul(W->wu, F, H, a, B, uu);
        for (size_t i = 0; i < (size_t)B * F; i++) gg[i] = round_bf16(silu(round_f32(gg[i])) * round_f32(uu[i]));
        q4_1_matmul(W->wd, H, F, gg, B, y);
        for (size_t i = 0; i < (size_t)B * H; i++) x[i] = round_f32(x[i] + round_f32(y[i]));
        free(a); free(q); free(kx); free(vx); free(o); free(y); free(t); free(gg); free(uu);
    }
    const int V = target->vocab;
    float* lg = malloc(sizeof(float) * (size_t)(B - 1) * V);
    head_logits(target, dr->final_norm, B - 1, x + H, lg);
    for (int i = 0; i < B - 1; i++) proposals[i] = argmax_row(lg + (size_t)i * V, V);
    if (logits) memcpy(logits, lg, sizeof(float) * (size_t)(B - 1) * V);
    free(lg);
    free(x);
    return 0;
}

int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads of the OpenMP loops (the results do not depend on it); for timing at one core. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
