// Host runtime and C ABI of the MuScriptor INT4 decoder step (see include/mt.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "../../include/mt.h"
#include "mt_internal.h"

using namespace mt;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

#define HIP_TRY(expr)                                                                          \
    do {                                                                                       \
        hipError_t e_ = (expr);                                                                \
        if (e_ != hipSuccess)                                                                  \
            return fail(MT_ERR_HIP, "%s failed: %s (%s:%d)", #expr, hipGetErrorString(e_),     \
                        __FILE__, __LINE__);                                                   \
    } while (0)

constexpr int kPart = 68;      // floats per attention partial (m, l, acc[64], pad)
constexpr int kMaxSplit = 64;  // split-K bound of the decode attention
constexpr int kMaxChunk = 256; // positions per split of the decode attention
constexpr int kMaxTcap = kMaxSplit * kMaxChunk;

}  // namespace

struct mt_model {
    mt_config c{};
    int device = 0;
    hipStream_t last_stream = nullptr;
    // weights
    float* tok_emb = nullptr;
    float* lm_head = nullptr;
    float* ln = nullptr;   // [L, 4, d]
    float* lnf = nullptr;  // [2, d]
    uint8_t* wq_all = nullptr;
    float* ws_all = nullptr;
    uint8_t* wt_all = nullptr;  // the projections in the GEMV tiling
    float* wst_all = nullptr;
    std::vector<Int4Mat> proj;  // [L*4]
    // cache
    float* kc = nullptr;
    float* vc = nullptr;
    SeqPos pos{};  // positions already in the cache, per sequence
    int* err = nullptr;
    // decode scratch
    float* x = nullptr;
    float* a = nullptr;
    float* q = nullptr;
    float* att = nullptr;
    float* h = nullptr;
    float* part = nullptr;
    float* z = nullptr;
    // persistent decode
    int decode_path = MT_DECODE_AUTO;
    bool persistent_ok = false;
    void* xbuf = nullptr;
    // single-launch step for the whole batch, one XCD per sequence
    bool batched_ok = false;
    void* bxbuf = nullptr;
    void* trace = nullptr;  // phase timestamps of the last persistent step (MT_TRACE=1)
    uint32_t epoch = 0;
    // prefill workspace
    size_t pf_rows = 0;
    float* pf = nullptr;
    // this device's fixed workspace of mt_prefill_noalloc (not owned)
    float* noalloc_ws = nullptr;
};

namespace {

template <typename T>
hipError_t dmalloc(T** p, size_t count) {
    return hipMalloc(reinterpret_cast<void**>(p), std::max<size_t>(count, 1) * sizeof(T));
}

void free_model(mt_model* m) {
    if (!m) return;
    void* ptrs[] = {m->tok_emb, m->lm_head, m->ln, m->lnf, m->wq_all, m->ws_all, m->wt_all, m->wst_all, m->kc, m->vc, m->err, m->x,
                    m->a, m->q, m->att, m->h, m->part, m->z, m->xbuf, m->bxbuf, m->trace, m->pf};
    for (void* p : ptrs)
        if (p) (void)hipFree(p);
    delete m;
}

int check_config(const mt_config* c) {
    if (!c) return fail(MT_ERR_INVALID_ARG, "config is NULL");
    if (c->head_dim != 64) return fail(MT_ERR_UNSUPPORTED, "head_dim must be 64 (got %d)", c->head_dim);
    if (c->group != 32) return fail(MT_ERR_UNSUPPORTED, "group must be 32 (got %d)", c->group);
    const uint32_t known = MT_FLAG_W4A8 | MT_FLAG_DENSE_F16 | MT_FLAG_DENSE_F32;
    if (c->flags & ~known) return fail(MT_ERR_UNSUPPORTED, "unknown flags 0x%x", c->flags);
    if (__builtin_popcount(c->flags & known) > 1)
        return fail(MT_ERR_UNSUPPORTED, "W4A8, dense FP16 and dense FP32 weights exclude each other (flags 0x%x)",
                    c->flags);
    if (c->n_layers < 1 || c->n_heads < 1 || c->vocab < 1 || c->batch < 1 || c->batch > kMaxBatch ||
        c->t_cap < 1 || c->t_cap > kMaxTcap || c->d_ff < 32)
        return fail(MT_ERR_INVALID_ARG, "non-positive or out-of-range size in config");
    if (c->d_model != c->n_heads * 64)
        return fail(MT_ERR_INVALID_ARG, "d_model (%d) must equal n_heads * 64", c->d_model);
    if (c->d_model % 32 || c->d_ff % 32)
        return fail(MT_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 32");
    if (c->d_model > 2048) return fail(MT_ERR_UNSUPPORTED, "d_model above 2048 is not supported");
    if (!(c->ln_eps > 0.f) || !std::isfinite(c->ln_eps))
        return fail(MT_ERR_INVALID_ARG, "ln_eps must be positive");
    return MT_OK;
}

// Split-K layout of the decode attention over T keys: about 512 workgroups,
// chunks of 16 .. 256 positions (a multiple of 16), at most kMaxSplit splits
// (the partials buffer holds that many per sequence and head; with
// T <= kMaxTcap = kMaxSplit * kMaxChunk the chunk then stays <= 256).
void attn_split(int B, int H, int T, int* nsplit, int* chunk) {
    const int want = std::min(kMaxSplit, std::max(1, (512 + B * H - 1) / (B * H)));
    int ch = (T + want - 1) / want;
    ch = std::min(kMaxChunk, std::max(16, (ch + 15) / 16 * 16));
    *nsplit = (T + ch - 1) / ch;
    *chunk = ch;
}

// Prefill row workspace, per row (floats): x [d] | a [d] | q [d] | att [d] |
// spare [d] | h [F].  The split-K partials of the O projection go to h
// (free until FFN-up), those of FFN-down to a .. spare.
size_t prefill_row_floats(size_t d, size_t F) { return 5 * d + F; }

int ensure_prefill_ws(mt_model* m, size_t rows) {
    if (rows <= m->pf_rows) return MT_OK;
    if (m->pf) HIP_TRY(hipFree(m->pf));
    m->pf = nullptr;
    m->pf_rows = 0;
    const size_t d = m->c.d_model, F = m->c.d_ff;
    if (dmalloc(&m->pf, rows * prefill_row_floats(d, F)) != hipSuccess)
        return fail(MT_ERR_OOM, "prefill workspace of %zu rows", rows);
    m->pf_rows = rows;
    return MT_OK;
}

// Run every layer over M = B * R rows held in x (row m = b * R + i, position
// t0 + i).  `decode` selects the split-K decode attention (R == 1).
// `prefill_ws`: the buffers are the prefill workspace (prefill_row_floats),
// whose free regions hold split-K partials of the O and FFN-down GEMMs.
int run_layers(mt_model* m, float* x, float* a, float* q, float* att, float* h, int R, int b0, int nb,
               bool decode, hipStream_t st, bool prefill_ws = false) {
    const mt_config& c = m->c;
    const int d = c.d_model, F = c.d_ff, M = nb * R;
    const bool a8 = (c.flags & MT_FLAG_W4A8) != 0;
    // GEMM rows of a prefill: O and FFN-down with K split where the 64 x 64
    // tiles alone leave CUs idle, summed in a fixed order (the result does
    // not depend on scheduling)
    const bool splitk = prefill_ws && !decode && !a8 && !gemv_takes_rows(M, R);
    // with few rows (whole sequences of at most 8 rows per GEMV slice) the
    // GEMV applies both LayerNorms itself
    const bool fuse_ln = gemv_fuses_layernorm(M, d) && gemv_takes_rows(M, R);
    // a already holds the LayerNorm the next projection needs: the split-K
    // sum of the previous projection formed it with the residual update
    bool a_ready = false;
    for (int l = 0; l < c.n_layers; ++l) {
        const float* ln = m->ln + (size_t)l * 4 * d;
        QkvDest dst{q, m->kc, m->vc, d, l, c.batch, c.t_cap, b0, R, m->pos};
        if (fuse_ln) {
            HIP_TRY(launch_w4_matmul(x, d, M, m->proj[l * 4 + 0], ln, ln + d, c.ln_eps, nullptr, 0, EPI_QKV, &dst,
                                     false, st, nullptr, a8));
        } else {
            if (!a_ready) HIP_TRY(launch_layernorm(x, d, ln, ln + d, c.ln_eps, d, M, a, d, st));
            HIP_TRY(launch_w4_matmul(a, d, M, m->proj[l * 4 + 0], nullptr, nullptr, 0.f, nullptr, 0, EPI_QKV, &dst,
                                     false, st, nullptr, a8));
        }
        a_ready = false;
        if (decode) {
            // split-K attention; the O projection (GEMV) merges the partials,
            // or a merge kernel writes attention rows for the GEMM
            SeqPos T{};
            int tmax = 0;
            for (int b = 0; b < c.batch; ++b) {
                T.t[b] = m->pos.t[b] + 1;
                tmax = std::max(tmax, T.t[b]);
            }
            int ns, ch;
            attn_split(c.batch, c.n_heads, tmax, &ns, &ch);
            if (ns > kMaxSplit) return fail(MT_ERR_INVALID_ARG, "decode attention: %d splits exceed %d", ns, kMaxSplit);
            HIP_TRY(launch_attn_decode(q, m->kc, m->vc, l, c.batch, c.n_heads, c.t_cap, T, m->part, ns, ch, st));
            if (fuse_ln) {
                const AttnParts ap{m->part, c.n_heads, ns};
                HIP_TRY(launch_w4_matmul(nullptr, d, M, m->proj[l * 4 + 1], nullptr, nullptr, 0.f, x, d, EPI_RESID,
                                         nullptr, false, st, &ap, a8));
            } else {
                HIP_TRY(launch_attn_merge(m->part, c.batch, c.n_heads, ns, att, st));
                HIP_TRY(launch_w4_matmul(att, d, M, m->proj[l * 4 + 1], nullptr, nullptr, 0.f, x, d, EPI_RESID,
                                         nullptr, false, st, nullptr, a8));
            }
        } else {
            HIP_TRY(launch_attn_prefill(q, m->kc, m->vc, l, c.batch, b0, nb, c.n_heads, c.t_cap, m->pos, R, att, st));
            const int so = splitk ? splitk_plan(M, m->proj[l * 4 + 1]) : 1;
            if (so > 1 && (long)so * d <= F && !fuse_ln) {
                // the sum also forms LN2 of the updated rows into a
                HIP_TRY(launch_w4_gemm_splitk(att, d, M, m->proj[l * 4 + 1], x, d, h, so, st, ln + 2 * d, ln + 3 * d,
                                              c.ln_eps, a, d));
                a_ready = true;
            } else {
                HIP_TRY(launch_w4_matmul(att, d, M, m->proj[l * 4 + 1], nullptr, nullptr, 0.f, x, d, EPI_RESID,
                                         nullptr, false, st, nullptr, a8));
            }
        }
        if (fuse_ln) {
            HIP_TRY(launch_w4_matmul(x, d, M, m->proj[l * 4 + 2], ln + 2 * d, ln + 3 * d, c.ln_eps, h, F, EPI_GELU,
                                     nullptr, false, st, nullptr, a8));
        } else {
            if (!a_ready) HIP_TRY(launch_layernorm(x, d, ln + 2 * d, ln + 3 * d, c.ln_eps, d, M, a, d, st));
            HIP_TRY(launch_w4_matmul(a, d, M, m->proj[l * 4 + 2], nullptr, nullptr, 0.f, h, F, EPI_GELU, nullptr,
                                     false, st, nullptr, a8));
        }
        a_ready = false;
        const int sd = splitk ? splitk_plan(M, m->proj[l * 4 + 3]) : 1;
        if (sd > 1 && sd <= 4 && !fuse_ln) {
            // partials over a, q, att and the spare rows (4 M d floats); the
            // sum also forms the next layer's LN1 into a (over the first
            // partials, each row's read before it is written)
            const bool next = l + 1 < c.n_layers;
            const float* lnn = ln + 4 * d;
            HIP_TRY(launch_w4_gemm_splitk(h, F, M, m->proj[l * 4 + 3], x, d, a, sd, st, next ? lnn : nullptr,
                                          next ? lnn + d : nullptr, c.ln_eps, a, d));
            a_ready = next;
        } else {
            HIP_TRY(launch_w4_matmul(h, F, M, m->proj[l * 4 + 3], nullptr, nullptr, 0.f, x, d, EPI_RESID, nullptr,
                                     false, st, nullptr, a8));
        }
    }
    return MT_OK;
}

int run_head(mt_model* m, const float* x, int R, int nb, float* logits, int64_t* next, hipStream_t st) {
    const mt_config& c = m->c;
    const int d = c.d_model;
    // final LayerNorm of the last row of every sequence
    HIP_TRY(launch_layernorm(x + (size_t)(R - 1) * d, (long)R * d, m->lnf, m->lnf + d, c.ln_eps, d,
                             nb, m->z, d, st));
    HIP_TRY(launch_lm_head(m->z, nb, m->lm_head, c.vocab, d, logits, st));
    HIP_TRY(launch_argmax(logits, nb, c.vocab, next, st));
    return MT_OK;
}

}  // namespace

extern "C" {

const char* mt_last_error(void) { return g_last_error.c_str(); }

int mt_pack_int4(const float* W, int32_t N, int32_t K, uint8_t* q, float* s) {
    if (!W || !q || !s) return fail(MT_ERR_INVALID_ARG, "mt_pack_int4: NULL pointer");
    if (N < 0 || K <= 0 || K % 32) return fail(MT_ERR_INVALID_ARG, "mt_pack_int4: K must be a positive multiple of 32");
    const int64_t G = K / 32;
    auto work = [&](int64_t n0, int64_t n1) {
        for (int64_t n = n0; n < n1; ++n)
            for (int64_t g = 0; g < G; ++g) {
                const float* w = W + n * (int64_t)K + g * 32;
                float mx = 0.0f;
                for (int k = 0; k < 32; ++k) mx = std::max(mx, std::fabs(w[k]));
                const float sc = mx / 7.0f;
                s[n * G + g] = sc;
                uint8_t* dst = q + n * (int64_t)(K / 2) + g * 16;
                for (int j = 0; j < 16; ++j) {
                    int code[2] = {0, 0};
                    if (sc != 0.0f)
                        for (int e = 0; e < 2; ++e) {
                            float r = std::rint(w[2 * j + e] / sc);
                            r = std::min(7.0f, std::max(-8.0f, r));
                            code[e] = (int)r;
                        }
                    dst[j] = (uint8_t)((code[0] + 8) | ((code[1] + 8) << 4));
                }
            }
    };
    const int64_t nthreads = std::max<int64_t>(1, std::min<int64_t>(std::thread::hardware_concurrency(), N / 256));
    if (nthreads <= 1) {
        work(0, N);
    } else {
        std::vector<std::thread> th;
        const int64_t per = (N + nthreads - 1) / nthreads;
        for (int64_t t = 0; t < nthreads; ++t)
            th.emplace_back(work, std::min<int64_t>(N, t * per), std::min<int64_t>(N, (t + 1) * per));
        for (auto& t : th) t.join();
    }
    return MT_OK;
}

int mt_pack_f16(const float* W, int64_t n, uint16_t* out) {
    if (!W || !out || n < 0) return fail(MT_ERR_INVALID_ARG, "mt_pack_f16: NULL pointer or negative size");
    // the compiler's binary32 -> binary16 conversion rounds to nearest, ties to even
    auto work = [&](int64_t i0, int64_t i1) {
        for (int64_t i = i0; i < i1; ++i) {
            const _Float16 h = (_Float16)W[i];
            std::memcpy(out + i, &h, sizeof h);
        }
    };
    const int64_t nthreads = std::max<int64_t>(1, std::min<int64_t>(std::thread::hardware_concurrency(), n >> 20));
    if (nthreads <= 1) {
        work(0, n);
    } else {
        std::vector<std::thread> th;
        const int64_t per = (n + nthreads - 1) / nthreads;
        for (int64_t t = 0; t < nthreads; ++t)
            th.emplace_back(work, std::min<int64_t>(n, t * per), std::min<int64_t>(n, (t + 1) * per));
        for (auto& t : th) t.join();
    }
    return MT_OK;
}

int mt_create(const mt_config* cfg, const mt_weights* w, int weights_on_device, void* stream,
              mt_model** out) {
    if (!out) return fail(MT_ERR_INVALID_ARG, "mt_create: out is NULL");
    *out = nullptr;
    int rc = check_config(cfg);
    if (rc) return rc;
    const mt_config c = *cfg;
    const int fmt = (c.flags & MT_FLAG_DENSE_F16) ? WF_F16 : (c.flags & MT_FLAG_DENSE_F32) ? WF_F32 : WF_INT4;
    if (!w || !w->tok_emb || !w->lm_head || !w->ln_final || !w->ln || (fmt == WF_INT4 ? !w->proj : !w->dense))
        return fail(MT_ERR_INVALID_ARG, "mt_create: NULL weight pointer");
    const int L = c.n_layers, d = c.d_model, F = c.d_ff, V = c.vocab, B = c.batch, H = c.n_heads;
    for (int i = 0; i < L * 4; ++i)
        if (fmt == WF_INT4 ? (!w->proj[i].q || !w->proj[i].s) : !w->dense[i])
            return fail(MT_ERR_INVALID_ARG, "mt_create: NULL projection %d", i);
    // bytes of a projection's weight values per input: 1/2 (nibbles), 2, 4
    const size_t esz2 = fmt == WF_INT4 ? 1 : fmt == WF_F16 ? 4 : 8;
    hipStream_t st = (hipStream_t)stream;
    const hipMemcpyKind kind = weights_on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;

    mt_model* m = new mt_model();
    m->c = c;
    auto bail = [&](int code) {
        free_model(m);
        return code;
    };
    if (hipGetDevice(&m->device) != hipSuccess) return bail(fail(MT_ERR_HIP, "hipGetDevice failed"));
    // the fixed workspace of mt_prefill_noalloc on this device; without it
    // that entry point reports an error, the others are unaffected
    if (noalloc_scratch_setup(m->device, &m->noalloc_ws) != hipSuccess) m->noalloc_ws = nullptr;

    // projection shapes [N, K]
    size_t qbytes = 0, sfloats = 0;
    m->proj.resize((size_t)L * 4);
    for (int l = 0; l < L; ++l) {
        const int NK[4][2] = {{3 * d, d}, {d, d}, {F, d}, {d, F}};
        for (int p = 0; p < 4; ++p) {
            Int4Mat& pm = m->proj[l * 4 + p];
            pm.N = NK[p][0];
            pm.K = NK[p][1];
            pm.fmt = fmt;
            qbytes += (size_t)pm.N * pm.K / 2 * esz2;
            if (fmt == WF_INT4) sfloats += (size_t)pm.N * pm.K / 32;
        }
    }
    const size_t kv = (size_t)L * B * c.t_cap * d;
    if (dmalloc(&m->tok_emb, (size_t)V * d) || dmalloc(&m->lm_head, (size_t)V * d) ||
        dmalloc(&m->ln, (size_t)L * 4 * d) || dmalloc(&m->lnf, 2 * (size_t)d) ||
        dmalloc(&m->wq_all, qbytes) || dmalloc(&m->ws_all, std::max<size_t>(sfloats, 64)) || dmalloc(&m->kc, kv) ||
        dmalloc(&m->vc, kv) || dmalloc(&m->err, 16) || dmalloc(&m->x, (size_t)B * d) ||
        dmalloc(&m->a, (size_t)B * std::max(d, F)) || dmalloc(&m->q, (size_t)B * d) ||
        dmalloc(&m->att, (size_t)B * d) || dmalloc(&m->h, (size_t)B * F) || dmalloc(&m->part, (size_t)B * H * kMaxSplit * kPart) ||
        dmalloc(&m->z, (size_t)B * d))
        return bail(fail(MT_ERR_OOM, "mt_create: device allocation failed (KV cache %zu bytes)", 2 * kv * 4));

    auto cpy = [&](void* dst, const void* src, size_t bytes) {
        return hipMemcpyAsync(dst, src, bytes, kind, st);
    };
    if (cpy(m->tok_emb, w->tok_emb, (size_t)V * d * 4) || cpy(m->lm_head, w->lm_head, (size_t)V * d * 4) ||
        cpy(m->ln, w->ln, (size_t)L * 4 * d * 4) || cpy(m->lnf, w->ln_final, (size_t)2 * d * 4))
        return bail(fail(MT_ERR_HIP, "mt_create: weight copy failed"));
    size_t qo = 0, so = 0;
    for (int i = 0; i < L * 4; ++i) {
        Int4Mat& pm = m->proj[i];
        const size_t nb = (size_t)pm.N * pm.K / 2 * esz2, ns = fmt == WF_INT4 ? (size_t)pm.N * pm.K / 32 : 0;
        if (fmt == WF_INT4 ? (cpy(m->wq_all + qo, w->proj[i].q, nb) || cpy(m->ws_all + so, w->proj[i].s, ns * 4))
                           : cpy(m->wq_all + qo, w->dense[i], nb) != hipSuccess)
            return bail(fail(MT_ERR_HIP, "mt_create: projection copy failed"));
        pm.q = m->wq_all + qo;
        pm.s = fmt == WF_INT4 ? m->ws_all + so : nullptr;
        qo += nb;
        so += ns;
    }
    if (hipMemsetAsync(m->err, 0, 16, st)) return bail(fail(MT_ERR_HIP, "mt_create: clearing the error word failed"));
    // second copy of the projections in the GEMV tiling (decode with B <= 16)
    size_t tbytes = 0, tfloats = 0;
    for (const Int4Mat& pm : m->proj) {
        tbytes += tiled_weight_bytes(pm);
        tfloats += tiled_scale_floats(pm);
    }
    if (dmalloc(&m->wt_all, tbytes) || dmalloc(&m->wst_all, std::max<size_t>(tfloats, 64)))
        return bail(fail(MT_ERR_OOM, "mt_create: GEMV weight copy of %zu bytes", tbytes));
    size_t to = 0, tso = 0;
    for (Int4Mat& pm : m->proj) {
        if (launch_tile_weights(pm, m->wt_all + to, m->wst_all + tso, st) != hipSuccess)
            return bail(fail(MT_ERR_HIP, "mt_create: weight tiling failed"));
        pm.qt = m->wt_all + to;
        pm.st = fmt == WF_INT4 ? m->wst_all + tso : nullptr;
        to += tiled_weight_bytes(pm);
        tso += tiled_scale_floats(pm);
    }
    // the single-launch step reads nibbles only
    m->persistent_ok = fmt == WF_INT4 && persistent_supported(d, F, H, B, V);
    if (m->persistent_ok) {
        const size_t xb = persistent_xbuf_bytes(L, d, F, H, B, V);
        if (hipMalloc(&m->xbuf, xb) != hipSuccess || hipMemsetAsync(m->xbuf, 0, xb, st) != hipSuccess)
            return bail(fail(MT_ERR_OOM, "mt_create: exchange buffer of %zu bytes", xb));
        if (persistent_prepare(m->xbuf, L, d, F, st) != hipSuccess)
            return bail(fail(MT_ERR_HIP, "mt_create: persistent role table"));
    }
    m->batched_ok = fmt == WF_INT4 && batched_supported(d, F, H, B, V);
    if (m->batched_ok) {
        const size_t xb = batched_xbuf_bytes(L, d, F, std::min(B, kBatchedGroup));
        if (hipMalloc(&m->bxbuf, xb) != hipSuccess || hipMemsetAsync(m->bxbuf, 0, xb, st) != hipSuccess)
            return bail(fail(MT_ERR_OOM, "mt_create: batched exchange buffer of %zu bytes", xb));
    }
    if (m->persistent_ok || m->batched_ok) {
        const char* tr = getenv("MT_TRACE");
        if (tr && tr[0] == '1') {
            const size_t tb = persistent_trace_bytes(L);
            if (hipMalloc(&m->trace, tb) != hipSuccess || hipMemsetAsync(m->trace, 0, tb, st) != hipSuccess)
                return bail(fail(MT_ERR_OOM, "mt_create: trace buffer"));
        }
    }
    if (hipStreamSynchronize(st) != hipSuccess) return bail(fail(MT_ERR_HIP, "mt_create: synchronise failed"));
    m->last_stream = st;
    *out = m;
    return MT_OK;
}

}  // extern "C"

namespace {

// Rows [prefix ; embed(tokens)] of sequences b0 .. b0+nb-1, each appended at
// its own position.  The row workspace is the model's own (grown on demand),
// or with `fixed_ws` the device's fixed workspace of mt_prefill_noalloc.
int prefill_rows(mt_model* m, int b0, int nb, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
                 float* logits, int64_t* next, void* stream, const char* who, bool fixed_ws = false) {
    if (S < 0 || P < 0 || (int64_t)S + P < 1) return fail(MT_ERR_INVALID_ARG, "%s: need P + S >= 1 (P=%d S=%d)", who, P, S);
    if ((S > 0 && !tokens) || (P > 0 && !prefix)) return fail(MT_ERR_INVALID_ARG, "%s: NULL tokens or prefix", who);
    const mt_config& c = m->c;
    const int R = P + S;
    for (int b = b0; b < b0 + nb; ++b)
        if ((int64_t)m->pos.t[b] + R > c.t_cap)
            return fail(MT_ERR_CACHE_FULL, "%s: %d rows at position %d of sequence %d exceed capacity %d", who, R,
                        m->pos.t[b], b, c.t_cap);
    hipStream_t st = (hipStream_t)stream;
    const size_t M = (size_t)nb * R;
    const int d = c.d_model;
    float* x = nullptr;
    int rc = MT_OK;
    if (fixed_ws) {
        const size_t per = prefill_row_floats(d, c.d_ff), need = M * per, have = noalloc_scratch_floats();
        if (!m->noalloc_ws) return fail(MT_ERR_HIP, "%s: the fixed device workspace is not available", who);
        if (need > have)
            return fail(MT_ERR_UNSUPPORTED,
                        "%s: %zu rows need %zu workspace floats, the fixed workspace holds %zu (at most %zu rows)", who,
                        M, need, have, have / per);
        x = m->noalloc_ws;
    } else {
        rc = ensure_prefill_ws(m, M);
        if (rc) return rc;
        x = m->pf;
    }
    float* a = x + M * d;
    float* q = a + M * d;
    float* att = q + M * d;
    float* h = att + 2 * M * d;  // after the spare rows
    HIP_TRY(launch_embed(tokens, S, prefix, P, m->tok_emb, c.vocab, d, nb, x, m->err, st));
    rc = run_layers(m, x, a, q, att, h, R, b0, nb, false, st, true);
    if (rc) return rc;
    rc = run_head(m, x, R, nb, logits, next, st);
    if (rc) return rc;
    for (int b = b0; b < b0 + nb; ++b) m->pos.t[b] += R;
    m->last_stream = st;
    return MT_OK;
}

}  // namespace

extern "C" {

int mt_prefill(mt_model* m, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
               float* logits, int64_t* next, void* stream) {
    if (!m || !logits || !next) return fail(MT_ERR_INVALID_ARG, "mt_prefill: NULL model or output");
    return prefill_rows(m, 0, m->c.batch, tokens, S, prefix, P, logits, next, stream, "mt_prefill");
}

int mt_prefill_noalloc(mt_model* m, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
                       float* logits, int64_t* next, void* stream) {
    if (!m || !logits || !next) return fail(MT_ERR_INVALID_ARG, "mt_prefill_noalloc: NULL model or output");
    return prefill_rows(m, 0, m->c.batch, tokens, S, prefix, P, logits, next, stream, "mt_prefill_noalloc", true);
}

int mt_prefill_seq(mt_model* m, int32_t b, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
                   float* logits, int64_t* next, void* stream) {
    if (!m || !logits || !next) return fail(MT_ERR_INVALID_ARG, "mt_prefill_seq: NULL model or output");
    if (b < 0 || b >= m->c.batch) return fail(MT_ERR_INVALID_ARG, "mt_prefill_seq: sequence %d of %d", b, m->c.batch);
    return prefill_rows(m, b, 1, tokens, S, prefix, P, logits, next, stream, "mt_prefill_seq");
}

int mt_decode_step(mt_model* m, const int64_t* token, float* logits, int64_t* next, void* stream) {
    if (!m || !token || !logits || !next) return fail(MT_ERR_INVALID_ARG, "mt_decode_step: NULL argument");
    const mt_config& c = m->c;
    for (int b = 0; b < c.batch; ++b)
        if (m->pos.t[b] + 1 > c.t_cap)
            return fail(MT_ERR_CACHE_FULL, "mt_decode_step: cache of sequence %d full at position %d (capacity %d)", b,
                        m->pos.t[b], c.t_cap);
    hipStream_t st = (hipStream_t)stream;
    int tmax = 0;
    for (int b = 0; b < c.batch; ++b) tmax = std::max(tmax, m->pos.t[b]);
    const bool batched = m->batched_ok && (m->decode_path == MT_DECODE_BATCHED ||
                                            (m->decode_path == MT_DECODE_AUTO && c.batch >= kBatchedAutoSeqs));
    const bool persistent = !batched && m->persistent_ok && m->decode_path != MT_DECODE_KERNELS &&
                            m->decode_path != MT_DECODE_BATCHED && tmax <= persistent_max_position(c.d_model, c.d_ff);
    if (batched) {
        // one launch per group of up to 8 sequences (one XCD each), each on
        // its group's slice of the cache, one after the other on the stream
        for (int b0 = 0; b0 < c.batch; b0 += kBatchedGroup) {
            const int nb = std::min(kBatchedGroup, c.batch - b0);
            BatchedArgs ba{};
            ba.L = c.n_layers; ba.d = c.d_model; ba.H = c.n_heads; ba.F = c.d_ff; ba.V = c.vocab;
            ba.B = nb; ba.t_cap = c.t_cap; ba.eps = c.ln_eps;
            ba.tok_emb = m->tok_emb; ba.lm_head = m->lm_head; ba.ln = m->ln; ba.ln_final = m->lnf;
            ba.wq_base = m->wq_all; ba.ws_base = m->ws_all;
            ba.kc = m->kc + (size_t)b0 * c.t_cap * c.d_model;
            ba.vc = m->vc + (size_t)b0 * c.t_cap * c.d_model;
            ba.kv_seqs = c.batch;
            ba.token = token + b0; ba.logits = logits + (size_t)b0 * c.vocab; ba.next = next + b0;
            for (int b = 0; b < nb; ++b) ba.t0[b] = m->pos.t[b0 + b];
            ba.epoch = ++m->epoch;
            ba.xbuf = m->bxbuf; ba.err = m->err; ba.trace = m->trace;
            ba.a8 = (c.flags & MT_FLAG_W4A8) ? 1 : 0;
            HIP_TRY(launch_batched_decode(ba, st));
        }
    } else if (persistent) {
        // one launch per sequence (a batch of at most kPersistentMaxSeqs),
        // each on that sequence's slice of the cache
        for (int b = 0; b < c.batch; ++b) {
            PersistentArgs pa{};
            pa.L = c.n_layers; pa.d = c.d_model; pa.H = c.n_heads; pa.F = c.d_ff; pa.V = c.vocab;
            pa.B = 1; pa.t_cap = c.t_cap; pa.eps = c.ln_eps;
            pa.tok_emb = m->tok_emb; pa.lm_head = m->lm_head; pa.ln = m->ln; pa.ln_final = m->lnf;
            pa.wq_base = m->wq_all; pa.ws_base = m->ws_all;
            pa.kc = m->kc + (size_t)b * c.t_cap * c.d_model;
            pa.vc = m->vc + (size_t)b * c.t_cap * c.d_model;
            pa.kv_seqs = c.batch;
            pa.token = token + b; pa.logits = logits + (size_t)b * c.vocab; pa.next = next + b;
            pa.t0 = m->pos.t[b];
            pa.epoch = ++m->epoch;
            pa.a8 = (c.flags & MT_FLAG_W4A8) ? 1 : 0;
            pa.resid = m->x + (size_t)b * c.d_model; pa.xbuf = m->xbuf; pa.err = m->err; pa.trace = m->trace;
            HIP_TRY(launch_persistent_decode(pa, st));
        }
    } else {
        const int d = c.d_model;
        HIP_TRY(launch_embed(token, 1, nullptr, 0, m->tok_emb, c.vocab, d, c.batch, m->x, m->err, st));
        int rc = run_layers(m, m->x, m->a, m->q, m->att, m->h, 1, 0, c.batch, true, st);
        if (rc) return rc;
        rc = run_head(m, m->x, 1, c.batch, logits, next, st);
        if (rc) return rc;
    }
    for (int b = 0; b < c.batch; ++b) m->pos.t[b] += 1;
    m->last_stream = st;
    return MT_OK;
}

int mt_cfg_combine(const float* logits, int32_t pairs, int32_t V, float cfg, float* guided, int64_t* next,
                   int64_t* token_pair, void* stream) {
    if (!logits || !next) return fail(MT_ERR_INVALID_ARG, "mt_cfg_combine: NULL argument");
    if (pairs < 1 || V < 1) return fail(MT_ERR_INVALID_ARG, "mt_cfg_combine: %d pairs of %d logits", pairs, V);
    if (!std::isfinite(cfg)) return fail(MT_ERR_INVALID_ARG, "mt_cfg_combine: coefficient is not finite");
    HIP_TRY(launch_cfg_combine(logits, pairs, V, cfg, guided, next, token_pair, (hipStream_t)stream));
    return MT_OK;
}

int mt_reset(mt_model* m) {
    if (!m) return fail(MT_ERR_INVALID_ARG, "mt_reset: NULL model");
    m->pos = SeqPos{};
    return MT_OK;
}

int mt_reset_seq(mt_model* m, int32_t b) {
    if (!m) return fail(MT_ERR_INVALID_ARG, "mt_reset_seq: NULL model");
    if (b < 0 || b >= m->c.batch) return fail(MT_ERR_INVALID_ARG, "mt_reset_seq: sequence %d of %d", b, m->c.batch);
    m->pos.t[b] = 0;
    return MT_OK;
}

int mt_position_seq(const mt_model* m, int32_t b, int32_t* t_past) {
    if (!m || !t_past) return fail(MT_ERR_INVALID_ARG, "mt_position_seq: NULL argument");
    if (b < 0 || b >= m->c.batch) return fail(MT_ERR_INVALID_ARG, "mt_position_seq: sequence %d of %d", b, m->c.batch);
    *t_past = m->pos.t[b];
    return MT_OK;
}

int mt_position(const mt_model* m, int32_t* t_past) {
    if (!m || !t_past) return fail(MT_ERR_INVALID_ARG, "mt_position: NULL argument");
    *t_past = m->pos.t[0];
    return MT_OK;
}

int mt_kv_cache(mt_model* m, const float** k, const float** v) {
    if (!m || !k || !v) return fail(MT_ERR_INVALID_ARG, "mt_kv_cache: NULL argument");
    *k = m->kc;
    *v = m->vc;
    return MT_OK;
}

int mt_check(mt_model* m) {
    if (!m) return fail(MT_ERR_INVALID_ARG, "mt_check: NULL model");
    HIP_TRY(hipStreamSynchronize(m->last_stream));
    int h = 0;
    HIP_TRY(hipMemcpy(&h, m->err, sizeof(int), hipMemcpyDeviceToHost));
    if (h) {
        HIP_TRY(hipMemset(m->err, 0, sizeof(int)));
        if (h & 2) return fail(MT_ERR_HIP, "persistent decode step gave up waiting on an exchange");
        return fail(MT_ERR_INVALID_ARG, "a token id outside [0, vocab) reached the device");
    }
    return MT_OK;
}

int mt_set_decode_path(mt_model* m, int32_t path) {
    if (!m) return fail(MT_ERR_INVALID_ARG, "mt_set_decode_path: NULL model");
    if (path != MT_DECODE_AUTO && path != MT_DECODE_KERNELS && path != MT_DECODE_PERSISTENT &&
        path != MT_DECODE_BATCHED)
        return fail(MT_ERR_INVALID_ARG, "mt_set_decode_path: unknown path %d", path);
    if (path == MT_DECODE_PERSISTENT && !m->persistent_ok)
        return fail(MT_ERR_UNSUPPORTED, "persistent decode does not support this configuration");
    if (path == MT_DECODE_BATCHED && !m->batched_ok)
        return fail(MT_ERR_UNSUPPORTED, "batched single-launch decode does not support this configuration");
    m->decode_path = path;
    return MT_OK;
}

void mt_destroy(mt_model* m) {
    if (!m) return;
    (void)hipDeviceSynchronize();
    free_model(m);
}

int mt_debug_dequant(mt_model* m, int32_t layer, int32_t proj, float* out, void* stream) {
    if (!m || !out) return fail(MT_ERR_INVALID_ARG, "mt_debug_dequant: NULL argument");
    if (layer < 0 || layer >= m->c.n_layers || proj < 0 || proj > 3)
        return fail(MT_ERR_INVALID_ARG, "mt_debug_dequant: bad layer/projection");
    HIP_TRY(launch_dequant(m->proj[layer * 4 + proj], out, (hipStream_t)stream));
    return MT_OK;
}

int mt_debug_trace(mt_model* m, uint64_t* out, int64_t n) {
    if (!m || !out) return fail(MT_ERR_INVALID_ARG, "mt_debug_trace: NULL argument");
    if (!m->trace) return fail(MT_ERR_UNSUPPORTED, "mt_debug_trace: create the model with MT_TRACE=1");
    const size_t tb = persistent_trace_bytes(m->c.n_layers);
    if ((size_t)n * sizeof(uint64_t) < tb) return fail(MT_ERR_INVALID_ARG, "mt_debug_trace: need %zu words", tb / 8);
    HIP_TRY(hipStreamSynchronize(m->last_stream));
    HIP_TRY(hipMemcpy(out, m->trace, tb, hipMemcpyDeviceToHost));
    return MT_OK;
}

int mt_debug_matmul(mt_model* m, int32_t layer, int32_t proj, const float* x, int32_t M, float* y,
                    void* stream) {
    if (!m || !x || !y || M < 1) return fail(MT_ERR_INVALID_ARG, "mt_debug_matmul: bad argument");
    const int p = proj & 0xFF;
    const bool force_gemm = (proj & 0x100) != 0;
    if (layer < 0 || layer >= m->c.n_layers || p > 3)
        return fail(MT_ERR_INVALID_ARG, "mt_debug_matmul: bad layer/projection");
    const Int4Mat& w = m->proj[layer * 4 + p];
    HIP_TRY(launch_w4_matmul(x, w.K, M, w, nullptr, nullptr, 0.f, y, w.N, EPI_STORE, nullptr, force_gemm,
                             (hipStream_t)stream, nullptr, (m->c.flags & MT_FLAG_W4A8) != 0));
    return MT_OK;
}

}  // extern "C"
