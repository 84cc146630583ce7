/*
 * mt_oracle.c -- plain CPU oracle for the MuScriptor INT4 decoder step.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; both sides are fed from the
 * seeded input generator and nothing else.
 *
 * What it computes (the quantised model, written out by definition):
 *   - weights: symmetric round-to-nearest INT4 with groups of 32 along the
 *     input axis, FP32 scale per group (medium ONNX README, "Model variant":
 *     backbone projections are symmetric RTN INT4 with group size 32);
 *   - everything else in FP32 (same table: activations, KV cache,
 *     embeddings and LM head stay FP32);
 *   - one decoder call appends P prefix rows and S token rows at position
 *     T_past of a fixed-capacity cache [L, B, T_cap, H, 64] and returns the
 *     logits of the last row (small ONNX conversion page, decoder inputs and
 *     outputs; medium ONNX README, "Model variant", for the fixed-capacity
 *     shared past/present buffer);
 *   - greedy argmax (small ONNX conversion page; model card, "Model
 *     description").
 *
 * Readings where the pages are silent (all listed in the design notes):
 * pre-norm residual blocks with LayerNorm (eps 1e-5, biased variance, gain and
 * bias), four bias-free projections per layer (fused QKV ordered Q|K|V,
 * O, FFN-up, FFN-down), exact-erf GELU, attention scale 1/8, attention causal
 * over the whole cache including the prefix, no positional term, a final
 * LayerNorm before an untied LM head, round-half-to-even in the quantiser,
 * low nibble = even input index, lowest index wins an argmax tie.
 *
 * W4A8 variant (one mode flag of the model): the medium ONNX README, "Model
 * variant", says the quantised MatMuls dynamically quantise their
 * activations to INT8 and accumulate in INT32.  Block, scale and rounding
 * are not on the pages; this oracle reads them as: per activation row and
 * group of 32 inputs (the weight group), s = max|x| / 127 (binary32
 * division), r = 1 / s (binary32 division), code = clamp(rint(x * r), -127,
 * 127) (binary32 multiply, ties to even), all-zero group -> codes 0; the
 * group product sum_k (u_k - 8) * code_k is an exact integer and the output
 * is sum_g s_w * s_a * I_g, accumulated in binary64 and rounded once.
 *
 * Dense variants (set_layer with quantize = 0): the Core AI conversion page
 * ships float32 models and a large model whose weights are cast to half
 * (its file table).  The oracle takes the projection weights unquantised;
 * for the half variant they are first rounded to IEEE binary16 by
 * oracle_round_half (ties to even, gradual underflow, overflow to infinity)
 * and everything downstream is unchanged.
 *
 * Classifier-free guidance over row pairs (oracle_cfg_combine): the model
 * card offers optional CFG, the paper's scaling table is quoted at CFG = 2,
 * the conditioner's instrument input has a class id for no condition, and
 * released models are run with the coefficient at 1; the combining rule itself is not
 * on the pages.  Reading: the usual guidance of logits, cond + (cfg - 1) *
 * (cond - uncond) (= uncond + cfg * (cond - uncond); cfg = 1 is the plain
 * conditional model), the next token being the argmax of the guided row.
 * Pinned by its special cases (cfg = 1, cfg = 0, equal rows) and by
 * affinity in cfg; the rule for other coefficients is a reading.
 *
 * Precision: every named tensor is stored as binary32; every dot product,
 * LayerNorm moment, softmax and GELU is evaluated in binary64 and rounded once.
 * Must be compiled without fast-math and with FP contraction off.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)
#define ORACLE_EFULL (-2)
#define ORACLE_ENOMEM (-4)

/* ------------------------------------------------------------------ */
/* Quantise one [N, K] FP32 matrix to INT4, groups of 32 along K.
 *   m = max |w| over the group; s = m / 7 (binary32 division);
 *   q = clamp(rint(w / s), -8, 7) (binary32 division, ties to even);
 *   an all-zero group (s == 0) gets q = 0;
 *   stored as u = q + 8; byte j of a row holds u[2j] in its low nibble and
 *   u[2j+1] in its high nibble.  q is [N, K/2] bytes, s is [N, K/32]. */
int oracle_quantize_int4(const float* W, int64_t N, int64_t K, uint8_t* q, float* s)
{
    if (!W || !q || !s || N < 0 || K <= 0 || K % 32 != 0) return ORACLE_EINVAL;
    const int64_t ng = K / 32;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < ng; ++g) {
            const float* w = W + n * K + g * 32;
            float m = 0.0f;
            for (int k = 0; k < 32; ++k) {
                float a = fabsf(w[k]);
                if (a > m) m = a;
            }
            float sc = m / 7.0f;
            s[n * ng + g] = sc;
            for (int k = 0; k < 32; ++k) {
                int code = 0;
                if (sc != 0.0f) {
                    float r = rintf(w[k] / sc);
                    if (r < -8.0f) r = -8.0f;
                    if (r > 7.0f) r = 7.0f;
                    code = (int)r;
                }
                uint8_t u = (uint8_t)(code + 8);
                int64_t byte = (n * K + g * 32 + k) / 2;
                if ((k & 1) == 0)
                    q[byte] = (uint8_t)((q[byte] & 0xF0u) | u);
                else
                    q[byte] = (uint8_t)((q[byte] & 0x0Fu) | (uint8_t)(u << 4));
            }
        }
    }
    return ORACLE_OK;
}

/* w'[n,k] = (float)(u - 8) * s[n, k/32]: one binary32 multiply. */
int oracle_dequantize_int4(const uint8_t* q, const float* s, int64_t N, int64_t K, float* Wd)
{
    if (!q || !s || !Wd || N < 0 || K <= 0 || K % 32 != 0) return ORACLE_EINVAL;
    const int64_t ng = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint8_t byte = q[(n * K + k) / 2];
            int u = (k & 1) ? (byte >> 4) : (byte & 0x0F);
            float qv = (float)(u - 8);
            Wd[n * K + k] = qv * s[n * ng + k / 32];
        }
    return ORACLE_OK;
}

/* Y[m, n] = sum_k A[m, k] * W[n, k], binary64 sum, rounded once. */
int oracle_matmul(const float* A, int64_t M, int64_t K, const float* W, int64_t N, float* Y)
{
    if (!A || !W || !Y || M < 0 || N < 0 || K < 0) return ORACLE_EINVAL;
    /* Loop over output features outermost so each weight row is read once. */
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const float* w = W + n * K;
        for (int64_t m = 0; m < M; ++m) {
            const float* a = A + m * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += (double)a[k] * (double)w[k];
            Y[m * N + n] = (float)acc;
        }
    }
    return ORACLE_OK;
}

/* IEEE binary16 rounding of binary32 values, ties to even: 11 significant
 * bits, quantum 2^(e - 10) for 2^e <= |x| < 2^(e + 1) and e >= -14, 2^-24
 * below 2^-14 (subnormals); |x| >= 65520 (halfway above the largest finite
 * half, 65504) becomes infinity.  Output as binary32 (exact). */
int oracle_round_half(const float* x, int64_t n, float* out)
{
    if (n < 0 || (n && (!x || !out))) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) {
        const double v = x[i];
        if (isnan(v)) {
            out[i] = x[i];
            continue;
        }
        const double a = fabs(v);
        if (a >= 65520.0) {
            out[i] = v > 0 ? INFINITY : -INFINITY;
            continue;
        }
        int e;
        frexp(a, &e); /* a = f 2^e, 0.5 <= f < 1, so 2^(e-1) <= a */
        const int q = (e - 1 < -14 ? -14 : e - 1) - 10;
        const double quantum = ldexp(1.0, q);
        out[i] = (float)(nearbyint(v / quantum) * quantum); /* scaling by 2^q is exact */
    }
    return ORACLE_OK;
}

/* W4A8: INT8 codes of activation rows, per row and group of 32.
 *   m = max |x| over the group; s = m / 127 (binary32 division);
 *   r = 1 / s (binary32 division); code = clamp(rint(x * r), -127, 127);
 *   an all-zero group (s == 0) gets codes 0.  q is [M, K], s is [M, K/32]. */
int oracle_quantize_act_int8(const float* X, int64_t M, int64_t K, int8_t* q, float* s)
{
    if (!X || !q || !s || M < 0 || K <= 0 || K % 32 != 0) return ORACLE_EINVAL;
    const int64_t ng = K / 32;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t g = 0; g < ng; ++g) {
            const float* x = X + m * K + g * 32;
            float mx = 0.0f;
            for (int k = 0; k < 32; ++k) {
                float a = fabsf(x[k]);
                if (a > mx) mx = a;
            }
            float sc = mx / 127.0f;
            s[m * ng + g] = sc;
            float r = sc != 0.0f ? 1.0f / sc : 0.0f;
            for (int k = 0; k < 32; ++k) {
                float v = rintf(x[k] * r);
                if (v < -127.0f) v = -127.0f;
                if (v > 127.0f) v = 127.0f;
                q[m * K + g * 32 + k] = (int8_t)v;
            }
        }
    return ORACLE_OK;
}

/* W4A8 product: Y[m, n] = sum_g ws[n, g] * sa[m, g] * I_g with
 * I_g = sum_{k in g} (u[n, k] - 8) * code[m, k] (exact integer), the codes
 * from oracle_quantize_act_int8 and the weights as packed INT4 (wq [N, K/2],
 * ws [N, K/32]).  Binary64 sum over groups, rounded once. */
int oracle_matmul_w4a8(const float* A, int64_t M, int64_t K, const uint8_t* wq, const float* ws,
                       int64_t N, float* Y)
{
    if (!A || !wq || !ws || !Y || M < 0 || N < 0 || K <= 0 || K % 32 != 0) return ORACLE_EINVAL;
    const int64_t ng = K / 32;
    int8_t* qa = (int8_t*)malloc((size_t)(M * K) + 1);
    float* sa = (float*)malloc(sizeof(float) * (size_t)(M * ng) + 1);
    if (!qa || !sa) { free(qa); free(sa); return ORACLE_ENOMEM; }
    oracle_quantize_act_int8(A, M, K, qa, sa);
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t g = 0; g < ng; ++g) {
                int64_t I = 0;
                for (int k = 0; k < 32; ++k) {
                    const int64_t kk = g * 32 + k;
                    const uint8_t byte = wq[(n * K + kk) / 2];
                    const int u = (kk & 1) ? (byte >> 4) : (byte & 0x0F);
                    I += (int64_t)(u - 8) * (int64_t)qa[m * K + kk];
                }
                acc += (double)ws[n * ng + g] * (double)sa[m * ng + g] * (double)I;
            }
            Y[m * N + n] = (float)acc;
        }
    free(qa);
    free(sa);
    return ORACLE_OK;
}

/* y = (x - mean) / sqrt(var + eps) * g + b, biased variance, per row. */
int oracle_layernorm(const float* X, int64_t M, int64_t d, const float* g, const float* b,
                     float eps, float* Y)
{
    if (!X || !g || !b || !Y || M < 0 || d <= 0) return ORACLE_EINVAL;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        const float* x = X + m * d;
        double mu = 0.0;
        for (int64_t j = 0; j < d; ++j) mu += (double)x[j];
        mu /= (double)d;
        double var = 0.0;
        for (int64_t j = 0; j < d; ++j) {
            double c = (double)x[j] - mu;
            var += c * c;
        }
        var /= (double)d;
        double rstd = 1.0 / sqrt(var + (double)eps);
        for (int64_t j = 0; j < d; ++j)
            Y[m * d + j] = (float)(((double)x[j] - mu) * rstd * (double)g[j] + (double)b[j]);
    }
    return ORACLE_OK;
}

/* GELU, exact erf form, evaluated in binary64. */
static float gelu1(float x)
{
    double v = (double)x;
    return (float)(0.5 * v * (1.0 + erf(v / sqrt(2.0))));
}

int oracle_gelu(const float* X, int64_t n, float* Y)
{
    if (!X || !Y || n < 0) return ORACLE_EINVAL;
    for (int64_t i = 0; i < n; ++i) Y[i] = gelu1(X[i]);
    return ORACLE_OK;
}

/* One query row against T cached keys of one head.
 *   score_t = (q . K_t) * 0.125 ; p = softmax(score) ; out = sum_t p_t V_t
 * k and v point at key/value 0 of this head; consecutive positions are
 * `stride` floats apart.  Computed in binary64, rounded once. */
static void attend_row(const float* qh, const float* k, const float* v, int64_t T,
                       int64_t stride, double* scratch, float* out)
{
    double mx = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
        const float* kt = k + t * stride;
        double acc = 0.0;
        for (int j = 0; j < 64; ++j) acc += (double)qh[j] * (double)kt[j];
        scratch[t] = acc * 0.125;
        if (scratch[t] > mx) mx = scratch[t];
    }
    double den = 0.0;
    for (int64_t t = 0; t < T; ++t) {
        scratch[t] = exp(scratch[t] - mx);
        den += scratch[t];
    }
    for (int j = 0; j < 64; ++j) {
        double acc = 0.0;
        for (int64_t t = 0; t < T; ++t) acc += scratch[t] * (double)v[t * stride + j];
        out[j] = (float)(acc / den);
    }
}

/* Attention for one row, all heads: q [H*64]; kc/vc [T, H, 64]; out [H*64]. */
int oracle_attention(const float* q, const float* kc, const float* vc, int64_t T, int64_t H,
                     float* out)
{
    if (!q || !kc || !vc || !out || T < 1 || H < 1) return ORACLE_EINVAL;
    double* scratch = (double*)malloc(sizeof(double) * (size_t)T);
    if (!scratch) return ORACLE_ENOMEM;
    for (int64_t h = 0; h < H; ++h)
        attend_row(q + h * 64, kc + h * 64, vc + h * 64, T, H * 64, scratch, out + h * 64);
    free(scratch);
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* The model: B sequences advancing in lockstep over a shared T_past.      */

typedef struct {
    int64_t L, d, H, F, V, B, Tcap;
    float eps;
    int64_t* tpos;  /* [B] positions already in the cache, per sequence */
    float* tok_emb; /* [V, d] */
    float* lm_head; /* [V, d] */
    float* lnf;     /* [2, d] gain, bias */
    float** wqkv;   /* dequantised [3d, d] */
    float** wo;     /* [d, d] */
    float** wup;    /* [F, d] */
    float** wdown;  /* [d, F] */
    float** ln;     /* [4, d]: g1, b1, g2, b2 */
    uint8_t** cq;   /* W4A8: packed codes of the 4 projections of layer l, or NULL */
    float** cs;     /*       their group scales */
    int w4a8;       /* 1: the projections run the W4A8 product */
    float* kc;      /* [L, B, Tcap, H, 64] */
    float* vc;
} oracle_model;

static void model_free(oracle_model* m)
{
    if (!m) return;
    if (m->wqkv)
        for (int64_t l = 0; l < m->L; ++l) {
            free(m->wqkv[l]); free(m->wo[l]); free(m->wup[l]); free(m->wdown[l]); free(m->ln[l]);
            free(m->cq[l]); free(m->cs[l]);
        }
    free(m->wqkv); free(m->wo); free(m->wup); free(m->wdown); free(m->ln); free(m->cq); free(m->cs);
    free(m->tok_emb); free(m->lm_head); free(m->lnf); free(m->kc); free(m->vc); free(m->tpos);
    free(m);
}

void oracle_model_free(oracle_model* m) { model_free(m); }

oracle_model* oracle_model_new(int64_t L, int64_t d, int64_t H, int64_t F, int64_t V,
                               int64_t B, int64_t Tcap, float eps)
{
    if (L < 1 || d < 32 || d % 32 || H < 1 || H * 64 != d || F < 32 || F % 32 || V < 1 ||
        B < 1 || Tcap < 1)
        return NULL;
    oracle_model* m = (oracle_model*)calloc(1, sizeof(oracle_model));
    if (!m) return NULL;
    m->L = L; m->d = d; m->H = H; m->F = F; m->V = V; m->B = B; m->Tcap = Tcap; m->eps = eps;
    m->wqkv = (float**)calloc((size_t)L, sizeof(float*));
    m->wo = (float**)calloc((size_t)L, sizeof(float*));
    m->wup = (float**)calloc((size_t)L, sizeof(float*));
    m->wdown = (float**)calloc((size_t)L, sizeof(float*));
    m->ln = (float**)calloc((size_t)L, sizeof(float*));
    m->cq = (uint8_t**)calloc((size_t)L, sizeof(uint8_t*));
    m->tpos = (int64_t*)calloc((size_t)B, sizeof(int64_t));
    m->cs = (float**)calloc((size_t)L, sizeof(float*));
    m->tok_emb = (float*)calloc((size_t)(V * d), sizeof(float));
    m->lm_head = (float*)calloc((size_t)(V * d), sizeof(float));
    m->lnf = (float*)calloc((size_t)(2 * d), sizeof(float));
    size_t kv = (size_t)(L * B * Tcap * d);
    m->kc = (float*)calloc(kv, sizeof(float));
    m->vc = (float*)calloc(kv, sizeof(float));
    if (!m->wqkv || !m->wo || !m->wup || !m->wdown || !m->ln || !m->cq || !m->cs || !m->tpos || !m->tok_emb || !m->lm_head ||
        !m->lnf || !m->kc || !m->vc) {
        model_free(m);
        return NULL;
    }
    return m;
}

int oracle_model_set_embed(oracle_model* m, const float* tok_emb, const float* lm_head,
                           const float* lnf_g, const float* lnf_b)
{
    if (!m || !tok_emb || !lm_head || !lnf_g || !lnf_b) return ORACLE_EINVAL;
    memcpy(m->tok_emb, tok_emb, sizeof(float) * (size_t)(m->V * m->d));
    memcpy(m->lm_head, lm_head, sizeof(float) * (size_t)(m->V * m->d));
    memcpy(m->lnf, lnf_g, sizeof(float) * (size_t)m->d);
    memcpy(m->lnf + m->d, lnf_b, sizeof(float) * (size_t)m->d);
    return ORACLE_OK;
}

/* Quantise then dequantise one FP32 projection into a fresh buffer. */
static float* quant_dequant(const float* W, int64_t N, int64_t K)
{
    uint8_t* q = (uint8_t*)calloc((size_t)(N * K / 2), 1);
    float* s = (float*)malloc(sizeof(float) * (size_t)(N * K / 32));
    float* wd = (float*)malloc(sizeof(float) * (size_t)(N * K));
    if (!q || !s || !wd) { free(q); free(s); free(wd); return NULL; }
    oracle_quantize_int4(W, N, K, q, s);
    oracle_dequantize_int4(q, s, N, K, wd);
    free(q); free(s);
    return wd;
}

/* Layer l from FP32 weights (quantised here).  If `quantize` is 0 the
 * matrices are taken as already dequantised values (used by closed-form
 * tests whose weights are exactly representable). */
int oracle_model_set_layer(oracle_model* m, int64_t l, const float* wqkv, const float* wo,
                           const float* wup, const float* wdown, const float* g1,
                           const float* b1, const float* g2, const float* b2, int quantize)
{
    if (!m || l < 0 || l >= m->L || !wqkv || !wo || !wup || !wdown || !g1 || !b1 || !g2 || !b2)
        return ORACLE_EINVAL;
    const int64_t d = m->d, F = m->F;
    free(m->wqkv[l]); free(m->wo[l]); free(m->wup[l]); free(m->wdown[l]); free(m->ln[l]);
    free(m->cq[l]); free(m->cs[l]);
    m->wqkv[l] = m->wo[l] = m->wup[l] = m->wdown[l] = m->ln[l] = NULL;
    m->cq[l] = NULL;
    m->cs[l] = NULL;
    if (quantize) {
        /* codes of QKV [3d, d], O [d, d], up [F, d], down [d, F], in that order */
        const int64_t nw = 4 * d * d + 2 * F * d;
        m->cq[l] = (uint8_t*)calloc((size_t)(nw / 2), 1);
        m->cs[l] = (float*)malloc(sizeof(float) * (size_t)(nw / 32));
        if (!m->cq[l] || !m->cs[l]) return ORACLE_ENOMEM;
        const float* mats[4] = {wqkv, wo, wup, wdown};
        const int64_t Ns[4] = {3 * d, d, F, d}, Ks[4] = {d, d, d, F};
        int64_t off = 0;
        for (int i = 0; i < 4; ++i) {
            oracle_quantize_int4(mats[i], Ns[i], Ks[i], m->cq[l] + off / 2, m->cs[l] + off / 32);
            off += Ns[i] * Ks[i];
        }
        m->wqkv[l] = quant_dequant(wqkv, 3 * d, d);
        m->wo[l] = quant_dequant(wo, d, d);
        m->wup[l] = quant_dequant(wup, F, d);
        m->wdown[l] = quant_dequant(wdown, d, F);
    } else {
        m->wqkv[l] = (float*)malloc(sizeof(float) * (size_t)(3 * d * d));
        m->wo[l] = (float*)malloc(sizeof(float) * (size_t)(d * d));
        m->wup[l] = (float*)malloc(sizeof(float) * (size_t)(F * d));
        m->wdown[l] = (float*)malloc(sizeof(float) * (size_t)(d * F));
        if (m->wqkv[l]) memcpy(m->wqkv[l], wqkv, sizeof(float) * (size_t)(3 * d * d));
        if (m->wo[l]) memcpy(m->wo[l], wo, sizeof(float) * (size_t)(d * d));
        if (m->wup[l]) memcpy(m->wup[l], wup, sizeof(float) * (size_t)(F * d));
        if (m->wdown[l]) memcpy(m->wdown[l], wdown, sizeof(float) * (size_t)(d * F));
    }
    m->ln[l] = (float*)malloc(sizeof(float) * (size_t)(4 * d));
    if (!m->wqkv[l] || !m->wo[l] || !m->wup[l] || !m->wdown[l] || !m->ln[l]) return ORACLE_ENOMEM;
    memcpy(m->ln[l], g1, sizeof(float) * (size_t)d);
    memcpy(m->ln[l] + d, b1, sizeof(float) * (size_t)d);
    memcpy(m->ln[l] + 2 * d, g2, sizeof(float) * (size_t)d);
    memcpy(m->ln[l] + 3 * d, b2, sizeof(float) * (size_t)d);
    return ORACLE_OK;
}

/* Position of sequence 0 (all sequences share it unless single sequences
 * were appended with oracle_model_forward_seq). */
int64_t oracle_model_position(const oracle_model* m) { return m ? m->tpos[0] : -1; }

int64_t oracle_model_position_seq(const oracle_model* m, int64_t b)
{
    return (m && b >= 0 && b < m->B) ? m->tpos[b] : -1;
}

/* 1: the four projections run the W4A8 product (needs quantised layers). */
int oracle_model_set_w4a8(oracle_model* m, int on)
{
    if (!m) return ORACLE_EINVAL;
    m->w4a8 = on ? 1 : 0;
    return ORACLE_OK;
}

/* Projection i (0 QKV, 1 O, 2 up, 3 down) of layer l applied to rows A. */
static void project(const oracle_model* m, int64_t l, int i, const float* A, int64_t rows, float* Y)
{
    const int64_t d = m->d, F = m->F;
    const int64_t Ns[4] = {3 * d, d, F, d}, Ks[4] = {d, d, d, F};
    if (m->w4a8) {
        int64_t off = 0;
        for (int j = 0; j < i; ++j) off += Ns[j] * Ks[j];
        oracle_matmul_w4a8(A, rows, Ks[i], m->cq[l] + off / 2, m->cs[l] + off / 32, Ns[i], Y);
        return;
    }
    const float* W[4] = {m->wqkv[l], m->wo[l], m->wup[l], m->wdown[l]};
    oracle_matmul(A, rows, Ks[i], W[i], Ns[i], Y);
}

void oracle_model_reset(oracle_model* m)
{
    if (m)
        for (int64_t b = 0; b < m->B; ++b) m->tpos[b] = 0;
}

int oracle_model_kv(oracle_model* m, float** k, float** v)
{
    if (!m || !k || !v) return ORACLE_EINVAL;
    *k = m->kc;
    *v = m->vc;
    return ORACLE_OK;
}

/* One decoder call for the nb sequences bsel[0 .. nb) (all B in order when
 * bsel is NULL).  tokens [nb, S] (may be NULL when S == 0), prefix
 * [nb, P, d] (may be NULL when P == 0).  The rows [prefix ; embed(tokens)]
 * of selected sequence k are appended at that sequence's own positions
 * T_k .. T_k+P+S-1 (ragged batch: each sequence attends to its own cache
 * only).  logits [nb, V] and next [nb] are those of the last appended row;
 * hidden_out, if not NULL, receives the final-LayerNorm output of that row
 * [nb, d]. */
static int forward_seqs(oracle_model* m, int64_t nb, const int64_t* bsel, const int64_t* tokens, int64_t S,
                        const float* prefix, int64_t P, float* logits, int64_t* next, float* hidden_out)
{
    if (!m || S < 0 || P < 0 || P + S < 1 || !logits || !next || nb < 1) return ORACLE_EINVAL;
    if ((S > 0 && !tokens) || (P > 0 && !prefix)) return ORACLE_EINVAL;
    for (int64_t l = 0; l < m->L; ++l)
        if (!m->wqkv[l] || !m->ln[l] || (m->w4a8 && !m->cq[l])) return ORACLE_EINVAL;
    const int64_t L = m->L, d = m->d, H = m->H, F = m->F, V = m->V, B = m->B, Tc = m->Tcap;
    const int64_t R = P + S;
    int64_t tmax = 0;
    for (int64_t k = 0; k < nb; ++k) {
        const int64_t bs = bsel ? bsel[k] : k;
        if (bs < 0 || bs >= B) return ORACLE_EINVAL;
        if (m->tpos[bs] + R > Tc) return ORACLE_EFULL;
        if (m->tpos[bs] > tmax) tmax = m->tpos[bs];
    }
    for (int64_t i = 0; i < nb * S; ++i)
        if (tokens[i] < 0 || tokens[i] >= V) return ORACLE_EINVAL;

    const int64_t rows = nb * R;
    float* r = (float*)malloc(sizeof(float) * (size_t)(rows * d));
    float* a = (float*)malloc(sizeof(float) * (size_t)(rows * d));
    float* qkv = (float*)malloc(sizeof(float) * (size_t)(rows * 3 * d));
    float* att = (float*)malloc(sizeof(float) * (size_t)(rows * d));
    float* o = (float*)malloc(sizeof(float) * (size_t)(rows * d));
    float* h1 = (float*)malloc(sizeof(float) * (size_t)(rows * F));
    if (!r || !a || !qkv || !att || !o || !h1) {
        free(r); free(a); free(qkv); free(att); free(o); free(h1);
        return ORACLE_ENOMEM;
    }

    /* Rows of selected sequence k are r[(k*R + i) * d].  Prefix rows first,
     * then the embeddings of the token ids (no scaling, no positional term). */
    for (int64_t k = 0; k < nb; ++k)
        for (int64_t i = 0; i < R; ++i) {
            const float* src = (i < P) ? prefix + (k * P + i) * d
                                       : m->tok_emb + tokens[k * S + (i - P)] * d;
            memcpy(r + (k * R + i) * d, src, sizeof(float) * (size_t)d);
        }

    for (int64_t l = 0; l < L; ++l) {
        const float* ln = m->ln[l];
        oracle_layernorm(r, rows, d, ln, ln + d, m->eps, a);
        project(m, l, 0, a, rows, qkv);
        /* cache write: K = columns [d, 2d), V = [2d, 3d); head h = 64 columns */
        for (int64_t k = 0; k < nb; ++k) {
            const int64_t bs = bsel ? bsel[k] : k, t0 = m->tpos[bs];
            for (int64_t i = 0; i < R; ++i) {
                const float* row = qkv + (k * R + i) * 3 * d;
                int64_t slot = (((l * B + bs) * Tc) + t0 + i) * d;
                memcpy(m->kc + slot, row + d, sizeof(float) * (size_t)d);
                memcpy(m->vc + slot, row + 2 * d, sizeof(float) * (size_t)d);
            }
        }
        /* causal attention: row i of a sequence at T0 sees positions [0, T0 + i] */
#pragma omp parallel
        {
            double* scratch = (double*)malloc(sizeof(double) * (size_t)(tmax + R));
#pragma omp for collapse(3) schedule(static)
            for (int64_t k = 0; k < nb; ++k)
                for (int64_t i = 0; i < R; ++i)
                    for (int64_t h = 0; h < H; ++h) {
                        const int64_t bs = bsel ? bsel[k] : k, t0 = m->tpos[bs];
                        const float* qh = qkv + (k * R + i) * 3 * d + h * 64;
                        int64_t base = ((l * B + bs) * Tc) * d + h * 64;
                        attend_row(qh, m->kc + base, m->vc + base, t0 + i + 1, d, scratch,
                                   att + (k * R + i) * d + h * 64);
                    }
            free(scratch);
        }
        project(m, l, 1, att, rows, o);
        for (int64_t j = 0; j < rows * d; ++j) r[j] = r[j] + o[j];
        oracle_layernorm(r, rows, d, ln + 2 * d, ln + 3 * d, m->eps, a);
        project(m, l, 2, a, rows, h1);
        oracle_gelu(h1, rows * F, h1);
        project(m, l, 3, h1, rows, o);
        for (int64_t j = 0; j < rows * d; ++j) r[j] = r[j] + o[j];
    }

    /* final LayerNorm and LM head on the last row of each selected sequence */
    for (int64_t k = 0; k < nb; ++k) {
        const float* last = r + (k * R + R - 1) * d;
        float* z = a + k * d;
        oracle_layernorm(last, 1, d, m->lnf, m->lnf + d, m->eps, z);
        if (hidden_out) memcpy(hidden_out + k * d, z, sizeof(float) * (size_t)d);
    }
    oracle_matmul(a, nb, d, m->lm_head, V, logits);
    for (int64_t k = 0; k < nb; ++k) {
        const float* lg = logits + k * V;
        int64_t best = 0;
        for (int64_t v = 1; v < V; ++v)
            if (lg[v] > lg[best]) best = v;
        next[k] = best;
        m->tpos[bsel ? bsel[k] : k] += R;
    }
    free(r); free(a); free(qkv); free(att); free(o); free(h1);
    return ORACLE_OK;
}

/* Every sequence: tokens [B, S], prefix [B, P, d], logits [B, V], next [B]. */
int oracle_model_forward(oracle_model* m, const int64_t* tokens, int64_t S, const float* prefix,
                         int64_t P, float* logits, int64_t* next, float* hidden_out)
{
    return m ? forward_seqs(m, m->B, NULL, tokens, S, prefix, P, logits, next, hidden_out) : ORACLE_EINVAL;
}

/* Sequence b only: tokens [S], prefix [P, d], logits [V], next [1]. */
int oracle_model_forward_seq(oracle_model* m, int64_t b, const int64_t* tokens, int64_t S, const float* prefix,
                             int64_t P, float* logits, int64_t* next)
{
    return forward_seqs(m, 1, &b, tokens, S, prefix, P, logits, next, NULL);
}

/* Sequence b starts over at position 0 (its cache rows are overwritten). */
int oracle_model_reset_seq(oracle_model* m, int64_t b)
{
    if (!m || b < 0 || b >= m->B) return ORACLE_EINVAL;
    m->tpos[b] = 0;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------ */
/* Guided logits of `pairs` row pairs: logits [2 pairs, V]; row i is the
 * conditional row and row pairs + i its unconditional partner.  guided[i, v]
 * = c + (cfg - 1) * (c - u), the difference, product and sum each a binary64
 * operation on the widened inputs, then rounded to binary32; next[i] is the
 * argmax of guided row i, lowest index on ties. */
int oracle_cfg_combine(const float* logits, int64_t pairs, int64_t V, float cfg, float* guided, int64_t* next)
{
    if (!logits || !guided || !next || pairs < 1 || V < 1) return ORACLE_EINVAL;
    const double w = (double)cfg - 1.0;
    for (int64_t i = 0; i < pairs; ++i) {
        const float* c = logits + i * V;
        const float* u = logits + (pairs + i) * V;
        float* g = guided + i * V;
        for (int64_t v = 0; v < V; ++v) {
            const double diff = (double)c[v] - (double)u[v];
            const double step = w * diff;
            g[v] = (float)((double)c[v] + step);
        }
        int64_t best = 0;
        for (int64_t v = 1; v < V; ++v)
            if (g[v] > g[best]) best = v;
        next[i] = best;
    }
    return ORACLE_OK;
}
