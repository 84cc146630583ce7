/*
 * mt.h -- C ABI of the MuScriptor INT4 decoder step on MI355X (gfx950).
 *
 * The library runs the transcription decoder of MuScriptor: a decoder-only,
 * pre-norm transformer ("MuScriptor -- small" model card, "Model
 * description" and "Model variants") whose four per-layer projections are
 * stored as symmetric round-to-nearest INT4 with groups of 32 while
 * activations, the KV cache, the embeddings and the LM head stay FP32
 * ("MuScriptor Medium -- optimized W4A32 ONNX Runtime" README, "Model
 * variant").  One call appends rows to a fixed-capacity cache and returns
 * the logits of the last row; positions are implied by how many rows the
 * cache already holds ("unifolia/muscriptor-small-onnx", decoder section).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers unless stated otherwise.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All work is stream-ordered and asynchronous; outputs are valid once
 *     the stream has been synchronised.  Entry points on the decode path do
 *     not synchronise and do not allocate.
 *   - Return value: 0 on success, a negative MT_ERR_* code on failure.  On
 *     failure nothing has been launched and the cache and position are
 *     unchanged; mt_last_error() returns a message for the calling thread.
 *   - The model object is not thread-safe: calls on one model must be
 *     serialised by the caller.
 */
#ifndef MT_H
#define MT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MT_OK 0
#define MT_ERR_INVALID_ARG (-1) /* null pointer, bad size, bad config, bad token id */
#define MT_ERR_CACHE_FULL (-2)  /* T_past + rows > t_cap */
#define MT_ERR_HIP (-3)         /* a HIP runtime call failed */
#define MT_ERR_OOM (-4)         /* device or host allocation failed */
#define MT_ERR_UNSUPPORTED (-5) /* head_dim != 64, widths not multiples of 32, ... */

typedef struct mt_model mt_model;

/* Model and run configuration.  Sizes of the pages' three models:
 * small 14 x 768 x 12 heads, medium 24 x 1024 x 16, large 48 x 1536 x 24
 * (Core AI conversion table; model card "Model variants"); vocabulary 1393
 * (small ONNX conversion page); head width 64 (cache layout on the same
 * page). */
typedef struct {
    int32_t n_layers;  /* L */
    int32_t d_model;   /* d = n_heads * 64 */
    int32_t n_heads;   /* H */
    int32_t head_dim;  /* must be 64 */
    int32_t d_ff;      /* F, FFN width; multiple of 32 */
    int32_t vocab;     /* V (1393 for MT3 tokens) */
    int32_t group;     /* must be 32 */
    int32_t batch;     /* B sequences that advance in lockstep, 1..64 */
    int32_t t_cap;     /* fixed cache capacity per sequence (positions), 1..16384 */
    float ln_eps;      /* LayerNorm epsilon (1e-5) */
    uint32_t flags;    /* 0, MT_FLAG_W4A8, MT_FLAG_DENSE_F16 or MT_FLAG_DENSE_F32 */
} mt_config;

/* W4A8 variant of the four projections.  The medium ONNX README ("Model
 * variant") states that the quantised MatMuls dynamically quantise their
 * activations to INT8 and accumulate in INT32; block, scale and rounding are
 * this library's reading: for each activation row and group of 32 inputs
 * (the weight group) s_a = max|x| / 127, code = clamp(rint(x * (1 / s_a)),
 * -127, 127) with binary32 division and multiply (codes 0 for an all-zero
 * group); the group sum I = sum (u - 8) * code is exact and the projection
 * is sum_g s_w * s_a * I_g in FP32.  Attention, LayerNorm, the LM head and
 * the cache stay FP32.  Every decode path and the prefill support it. */
#define MT_FLAG_W4A8 1u

/* Dense-weight variants: the four projections are given unquantised in
 * mt_weights.dense (mt_weights.proj is not read) as row-major W [N, K] in
 * IEEE binary16 (MT_FLAG_DENSE_F16) or binary32 (MT_FLAG_DENSE_F32); each
 * value is widened exactly to FP32 and every other step is unchanged.  These
 * are the Core AI conversion's float32 files and its large float16 file,
 * whose weights are cast to half (its file table; "Faithfulness" on why
 * small fp16 is not shipped).  At most
 * one of MT_FLAG_W4A8, MT_FLAG_DENSE_F16 and MT_FLAG_DENSE_F32 may be set;
 * otherwise mt_create returns MT_ERR_UNSUPPORTED.  Dense models run the
 * multi-kernel decode step (MT_DECODE_PERSISTENT is refused). */
#define MT_FLAG_DENSE_F16 2u
#define MT_FLAG_DENSE_F32 4u

/* One INT4 projection in the canonical packed form.
 * For a matrix W [N, K] (row n = output feature n, K = input width):
 *   s[n, g]  (FP32, [N, K/32]) = max |W[n, 32g .. 32g+31]| / 7;
 *   code     = clamp(round-half-even(W / s), -8, 7), 0 for an all-zero group;
 *   q[n, j]  (uint8, [N, K/2]) = (code[2j] + 8) | (code[2j+1] + 8) << 4,
 *            i.e. the low nibble holds the even input index;
 *   dequantised weight = (float)(nibble - 8) * s  (one FP32 multiply).
 * Format: medium ONNX README, "Model variant" (symmetric RTN INT4, group
 * 32).  Nibble order, tie rule and FP32 scales are this library's reading. */
typedef struct {
    const uint8_t* q;
    const float* s;
} mt_int4;

/* Model weights.  Caller-owned and only read during mt_create; host or
 * device memory per the `weights_on_device` argument of mt_create.
 *   tok_emb  [V, d]           FP32 token embedding (not quantised)
 *   lm_head  [V, d]           FP32, row v produces logit v (untied, no bias)
 *   ln_final [2, d]           final LayerNorm gain, bias
 *   ln       [L, 4, d]        per layer: gain1, bias1, gain2, bias2 (one
 *                             contiguous array for all layers)
 *   proj     [L * 4]          per layer, in this order:
 *                               QKV  [3d, d]  rows Q | K | V, head h = rows 64h..64h+63 of each
 *                               O    [d, d]
 *                               up   [F, d]
 *                               down [d, F]
 *   dense    [L * 4]          same order; only with MT_FLAG_DENSE_F16 / _F32:
 *                               dense[i] points to W [N, K] row-major, binary16
 *                               or binary32 per the flag (proj may be NULL);
 *                               mt_pack_f16 makes the binary16 form
 * No projection has a bias. */
typedef struct {
    const float* tok_emb;
    const float* lm_head;
    const float* ln_final;
    const float* ln;
    const mt_int4* proj;
    const void* const* dense;
} mt_weights;

/* Host-side canonical packer (host pointers).  W [N, K] FP32 -> q [N, K/2],
 * s [N, K/32] as described for mt_int4.  K must be a multiple of 32.
 * Uses IEEE binary32 division and round-half-even. */
int mt_pack_int4(const float* W, int32_t N, int32_t K, uint8_t* q, float* s);

/* Host-side binary16 packer for MT_FLAG_DENSE_F16 weights (host pointers):
 * out[i] = the IEEE binary16 bits of W[i] rounded to nearest, ties to even
 * (gradual underflow, overflow to infinity), i < n.  The Core AI conversion
 * casts the large model's weights to half (its file table).  Errors: NULL
 * pointer or n < 0 -> MT_ERR_INVALID_ARG. */
int mt_pack_f16(const float* W, int64_t n, uint16_t* out);

/* Create a model: validates the config, copies the weights to the current
 * HIP device and allocates the KV cache [L, B, t_cap, H, 64] twice (K, V,
 * FP32, 2*L*B*t_cap*d*4 bytes) plus decode scratch.  The projections are the
 * INT4 group-32 MatMulNBits weights and the embeddings and LM head stay FP32
 * ("MuScriptor Medium -- optimized W4A32 ONNX Runtime" README, "Model
 * variant"); the cache has a fixed capacity chosen at deployment (the same
 * README, "Quick smoke test": a maximum cache length, 2504 by default) and is
 * owned by the model, allocated once, because past and present share one
 * buffer ("Model variant").  The projections are
 * held twice on the device: as given, and re-tiled for the batched decode
 * kernels (16-row blocks per group, so each load instruction reads one
 * contiguous block).  weights_on_device: 0 = host pointers, 1 = device
 * pointers.  The caller may free its weight buffers once mt_create
 * returns.  T_past starts at 0. */
int mt_create(const mt_config* cfg, const mt_weights* w, int weights_on_device, void* stream,
              mt_model** out);

/* Append rows to every sequence, each at its own position T_b (all equal
 * unless sequences were appended to or restarted one at a time, see
 * mt_prefill_seq), i.e. at T_b .. T_b+P+S-1:
 * first P prefix rows (the conditioner's output [B, P, d]), then the
 * embeddings of S token ids [B, S] (int64).  Either part may be empty
 * (NULL with size 0) but P + S >= 1.  Each appended row attends causally
 * to every cached position up to and including its own.  Writes the
 * logits of the last appended row [B, V] and its greedy argmax [B]
 * (int64, lowest index on ties).  T_past advances by P + S.
 * Small ONNX conversion page, decoder section: prefix rows, token rows,
 * past cache, last-position logits.  Allocates a row workspace the first
 * time a larger P + S is seen (not on the decode path).
 * Errors: MT_ERR_CACHE_FULL if T_b + P + S > t_cap for some b.  A token id outside
 * [0, V) is not checked on the host (it lives on the device): the row's
 * embedding becomes NaN and mt_check reports MT_ERR_INVALID_ARG. */
int mt_prefill(mt_model* m, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
               float* logits, int64_t* next, void* stream);

/* mt_prefill without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments, semantics and errors as
 * mt_prefill, but the row workspace is a fixed 36 MiB device array that the
 * library holds on each GPU it runs on until the process ends, instead of
 * memory grown with hipMalloc.  Calls no hipMalloc, hipFree or allocating
 * routine.  The workspace takes B * (P + S) * (5 d + d_ff) floats: at most
 * 9 Mi floats (1024 rows at d = 1024, d_ff = 4096; 682 rows at d = 1536);
 * larger calls return MT_ERR_UNSUPPORTED before any launch.  Every call on
 * one GPU uses the same array (it keeps the last call's contents; nothing in
 * it needs clearing): calls that overlap on one GPU, from different streams
 * or threads, race; serialise them. */
int mt_prefill_noalloc(mt_model* m, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
                       float* logits, int64_t* next, void* stream);

/* One greedy decode step: token[b] (int64) is appended to sequence b at
 * its own position T_b (the decoder call with one token row and no prefix
 * rows; positions are implied by the cache length: "unifolia/muscriptor-
 * small-onnx", "Files"; greedy decoding of the MT3 tokens, same section);
 * logits [B, V] and next [B] as for mt_prefill.  `next` may be passed back
 * as `token` of the following call, so greedy decoding never returns to the
 * host.  Same semantics as mt_prefill with P = 0, S = 1, on the dedicated
 * decode kernels.  No allocation, no synchronisation.
 * At B <= 2 (d_model 768/1024/1536, 256 or more CUs) the step is one
 * persistent launch per sequence that occupies every CU and whose
 * workgroups exchange data while resident: steps of different models must
 * not run concurrently on one GPU (issue them on one stream).  If workgroups cannot all become
 * resident, the step gives up after a bounded wait and mt_check reports
 * MT_ERR_HIP. */
int mt_decode_step(mt_model* m, const int64_t* token, float* logits, int64_t* next, void* stream);

/* Set every T_b to 0: the next call starts a new chunk on an empty cache
 * (positions restart because they are implied by the cache length,
 * "unifolia/muscriptor-small-onnx", "Files").  Cache contents are left as
 * they are (they are overwritten before they are read again). */
int mt_reset(mt_model* m);

/* Current position of sequence 0 (the shared T_past of a lockstep batch;
 * host pointer out). */
int mt_position(const mt_model* m, int32_t* t_past);

/* ---- Ragged batch: sequences of one batch at their own positions. ----
 * The pages' decoder is one call per chunk at a given T_past ("unifolia/
 * muscriptor-small-onnx", decoder section; positions are implied by the
 * cache length), and chunks of different tracks are independent; these calls
 * let a batch hold sequences at different positions, so a new chunk can be
 * prefilled into one slot of a running batch while the others keep decoding
 * (mt_decode_step advances every sequence, each at its own position). */

/* Append P prefix rows [P, d] and S token rows [S] (int64) to sequence b
 * only, at its position T_b; writes the logits of its last row [V] and its
 * argmax [1].  Same errors as mt_prefill (for sequence b); b outside
 * [0, batch) -> MT_ERR_INVALID_ARG.  The other sequences are untouched. */
int mt_prefill_seq(mt_model* m, int32_t b, const int64_t* tokens, int32_t S, const float* prefix, int32_t P,
                   float* logits, int64_t* next, void* stream);

/* Set T_b of sequence b to 0 (a new chunk or track starts in that slot). */
int mt_reset_seq(mt_model* m, int32_t b);

/* Current position T_b of sequence b (host pointer out). */
int mt_position_seq(const mt_model* m, int32_t b, int32_t* t_past);

/* ---- Classifier-free guidance over row pairs. ----
 * The MuScriptor model card offers optional CFG; the paper's scaling table
 * is quoted at CFG = 2; the conditioner's instrument input has a class id
 * that stands for no condition ("unifolia/muscriptor-small-onnx",
 * conditioner inputs); released models are run with the coefficient at 1.  The combining
 * rule is not on the pages; this library takes the usual guidance of logits.
 * A batch of 2 Np sequences holds Np pairs: sequence i (i < Np) is
 * conditional, sequence Np + i its unconditional partner (its prefix made
 * with the no-condition class, same length).  Both rows of a pair are fed
 * the same tokens.
 *
 * From the [2 Np, V] logits of mt_prefill or mt_decode_step:
 *   guided[i, v] = c + (cfg - 1) * (c - u),  c = logits[i, v], u = logits[Np + i, v]
 * (= u + cfg (c - u); cfg = 1 returns c bit for bit), the difference,
 * product and sum taken in binary64 and rounded once to FP32;
 *   next[i] = argmax_v guided[i, v], lowest index on ties;
 *   token_pair[i] = token_pair[Np + i] = next[i]   (when token_pair != NULL),
 * which is the `token` argument of the pair batch's next mt_decode_step.
 * All pointers are device memory on the stream's device: logits [2 Np, V]
 * FP32 (read only); guided [Np, V] FP32 or NULL (not stored); next [Np]
 * int64; token_pair [2 Np] int64 or NULL.  One launch, no allocation, no
 * synchronisation; needs no model.
 * Errors: NULL logits or next, Np < 1, V < 1 or a non-finite cfg ->
 * MT_ERR_INVALID_ARG (nothing launched); launch failure -> MT_ERR_HIP. */
int mt_cfg_combine(const float* logits, int32_t pairs, int32_t V, float cfg, float* guided, int64_t* next,
                   int64_t* token_pair, void* stream);

/* Device pointers to the cache, [L, B, t_cap, H, 64] FP32 each (the
 * decoder's past_key / past_value layout with the batch and a fixed capacity:
 * "unifolia/muscriptor-small-onnx", "Files").  The cache is updated in place:
 * past and present are the same buffer ("MuScriptor Medium -- optimized
 * W4A32 ONNX Runtime", "Model variant").  The pointers stay valid until
 * mt_destroy; the model owns the memory. */
int mt_kv_cache(mt_model* m, const float** k, const float** v);

/* Synchronise the model's last stream and report sticky device errors
 * (MT_ERR_INVALID_ARG after an out-of-range token id).  Clears the flag. */
int mt_check(mt_model* m);

/* Decode implementation selector (for measurement and parity of all):
 *   MT_DECODE_AUTO       B <= 2: one persistent launch per sequence;
 *                        3 <= B <= 16: the batched step where supported;
 *                        otherwise the kernels
 *   MT_DECODE_KERNELS    one kernel per operation
 *   MT_DECODE_PERSISTENT one persistent launch per sequence (B <= 2; past
 *                        its cache reach, 2560 to 5376 positions by width,
 *                        the kernels run)
 *   MT_DECODE_BATCHED    one launch per group of up to 8 sequences, each
 *                        sequence on its own XCD (2 <= B <= 16, INT4
 *                        weights, FP32 or MT_FLAG_W4A8 activations,
 *                        d_model 768, 1024 or 1536; any position below
 *                        t_cap);
 *                        MT_ERR_UNSUPPORTED otherwise
 * Every path computes the same decoder step ("MuScriptor Medium --
 * optimized W4A32 ONNX Runtime", "Model variant"). */
#define MT_DECODE_AUTO 0
#define MT_DECODE_KERNELS 1
#define MT_DECODE_PERSISTENT 2
#define MT_DECODE_BATCHED 3
int mt_set_decode_path(mt_model* m, int32_t path);

/* Destroy: synchronises the device, frees every buffer.  NULL is a no-op. */
void mt_destroy(mt_model* m);

/* Message for the last failing call on this thread ("" if none). */
const char* mt_last_error(void);

/* ---- Test-only entry points (stable names, unstable semantics). ---- */

/* Dequantise projection `proj` (0 QKV, 1 O, 2 up, 3 down) of layer `layer`
 * from the device copy: out [N, K] FP32 = (nibble - 8) * s, bit-exact. */
int mt_debug_dequant(mt_model* m, int32_t layer, int32_t proj, float* out, void* stream);

/* y [M, N] = x [M, K] . dequant(W)^T for one projection, on the decode
 * GEMV kernel (M <= 16, in launches of 8 rows) or the prefill GEMM kernel
 * (M > 16, or always when bit 8 of `proj` is set). */
int mt_debug_matmul(mt_model* m, int32_t layer, int32_t proj, const float* x, int32_t M, float* y,
                    void* stream);

/* Phase timestamps of the last persistent decode step (wall clock, 100 MHz
 * ticks), [256 workgroups][L + 1][24] words, copied to the host buffer `out`
 * of n words.  Only available when the model was created with the
 * environment variable MT_TRACE=1; synchronises the model's stream. */
int mt_debug_trace(mt_model* m, uint64_t* out, int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* MT_H */
