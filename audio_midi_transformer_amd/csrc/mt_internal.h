// Internal declarations shared by the host runtime and the kernel launchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mt {

// Epilogues of the INT4 matmul kernels.
enum Epilogue : int {
    EPI_STORE = 0,  // y[m, n] = acc
    EPI_GELU = 1,   // y[m, n] = GELU(acc), exact erf form
    EPI_RESID = 2,  // y[m, n] += acc (residual stream updated in place)
    EPI_QKV = 3,    // n <  d: q[m, n]; d <= n < 2d: K cache; 2d <= n: V cache
};

constexpr int kMaxBatch = 64;

// A value per sequence of the batch (positions, key counts), passed by value.
struct SeqPos {
    int t[kMaxBatch];
};

// Where the QKV epilogue scatters K and V: rows m = b * rows_per_seq + i
// (b < the number of sequences in the call) land at cache position
// pos.t[b0 + b] + i of sequence b0 + b in layer `layer`.
struct QkvDest {
    float* q;        // [M, d]
    float* kc;       // [L, batch, t_cap, H, 64]
    float* vc;
    int d;
    int layer;
    int batch;       // sequences in the cache
    int t_cap;
    int b0;          // first sequence of the rows
    int rows_per_seq;
    SeqPos pos;      // cache position of each sequence's first row
};

// Storage format of a projection's weights.
enum WeightFmt : int {
    WF_INT4 = 0,  // packed nibbles [N, K/2] + FP32 group scales [N, K/32]
    WF_F16 = 1,   // dense IEEE half [N, K]
    WF_F32 = 2,   // dense float [N, K]
};

// One projection W [N, K] (row n = output feature n).
struct Int4Mat {
    const uint8_t* q;  // INT4: nibbles [N, K/2]; dense: the values [N, K]
    const float* s;    // INT4: group scales [N, K/32]; dense: unused
    int N;
    int K;
    int fmt = WF_INT4;
    const uint8_t* qt = nullptr;  // the same weights in the GEMV tiling (launch_tile_weights)
    const float* st = nullptr;    // INT4: scales in the GEMV tiling
};

// ---- launchers (mt_kernels.hip); all return hipGetLastError() ----
hipError_t launch_embed(const int64_t* tokens, int S, const float* prefix, int P, const float* emb,
                        int V, int d, int B, float* x, int* err, hipStream_t st);
hipError_t launch_layernorm(const float* x, long ldx, const float* g, const float* b, float eps,
                            int d, int rows, float* y, long ldy, hipStream_t st);
// Prefill O / FFN-down projections (+= epilogue) with K split nsplit ways
// (splitk_plan) and a deterministic sum: the products go to part
// [nsplit][M][N] (nsplit * M * N floats), then are added to y in split order
// by one workgroup per row, which with ln_g also writes the next
// LayerNorm of the updated rows to a (row stride lda; a may be part).
int splitk_plan(int M, const Int4Mat& w);
hipError_t launch_w4_gemm_splitk(const float* x, int ldx, int M, const Int4Mat& w, float* y, int ldy, float* part,
                                 int nsplit, hipStream_t st, const float* ln_g = nullptr,
                                 const float* ln_b = nullptr, float eps = 0.f, float* a = nullptr, int lda = 0);
// Split-K partials of the decode attention, [B, H, nsplit, 68] floats.
struct AttnParts {
    const float* part;
    int H;
    int nsplit;
};

// y = x . W'^T (+ epilogue).  When ln_g is given, x is replaced by
// LayerNorm(x) inside the kernel (only where gemv_fuses_layernorm(M, K));
// when parts is given, x is the attention output merged from the partials
// (x is not read; GEMV path only).
hipError_t launch_w4_matmul(const float* x, int ldx, int M, const Int4Mat& w, const float* ln_g,
                            const float* ln_b, float eps, float* y, int ldy, Epilogue epi, const QkvDest* qkv,
                            bool force_gemm, hipStream_t st, const AttnParts* parts = nullptr, bool a8 = false);
// The GEMV takes M rows (sequences of rows_per_seq rows each) in slices of
// at most 8 rows; more rows than kGemvRowsMax go to the GEMM (a decode
// batch then merges its attention partials into rows first).
constexpr int kGemvRowsMax = 16;
bool gemv_takes_rows(int M, int rows_per_seq);
bool gemv_fuses_layernorm(int M, int K);
// Writes the split-K partials only; the O projection merges them.  Sequence
// b attends to its first T.t[b] cache positions.
hipError_t launch_attn_decode(const float* q, const float* kc, const float* vc, int layer, int B,
                              int H, int t_cap, const SeqPos& T, float* part, int nsplit, int chunk,
                              hipStream_t st);
// Attention rows out [B, H * 64] merged from the partials of launch_attn_decode.
hipError_t launch_attn_merge(const float* part, int B, int H, int nsplit, float* out, hipStream_t st);
// Causal attention of R new rows of nb sequences b0 .. b0+nb-1 (of Btot in
// the cache); sequence b0 + b's rows sit at positions t0.t[b0 + b] + i.
hipError_t launch_attn_prefill(const float* q, const float* kc, const float* vc, int layer, int Btot, int b0,
                               int nb, int H, int t_cap, const SeqPos& t0, int R, float* out, hipStream_t st);
hipError_t launch_lm_head(const float* z, int B, const float* w, int V, int d, float* logits,
                          hipStream_t st);
hipError_t launch_argmax(const float* logits, int B, int V, int64_t* next, hipStream_t st);
hipError_t launch_dequant(const Int4Mat& w, float* out, hipStream_t st);
// Guided logits of `pairs` conditional/unconditional row pairs of logits
// [2 pairs, V] (row i and row pairs + i), their argmax, and that token for
// both rows of each pair (guided and token_pair may be null).
hipError_t launch_cfg_combine(const float* logits, int pairs, int V, float cfg, float* guided, int64_t* next,
                              int64_t* token_pair, hipStream_t st);
// GEMV tiling of w.q / w.s into qt (tiled_weight_bytes(w)) and st
// (tiled_scale_floats(w) floats, INT4 only).
size_t tiled_weight_bytes(const Int4Mat& w);
size_t tiled_scale_floats(const Int4Mat& w);
hipError_t launch_tile_weights(const Int4Mat& w, uint8_t* qt, float* st, hipStream_t stream);

// Persistent single-launch decode step (mt_decode_persistent.hip).
struct PersistentPlan;
struct PersistentArgs {
    // model
    int L, d, H, F, V, B, t_cap;
    float eps;
    const float* tok_emb;
    const float* lm_head;
    const float* ln;        // [L, 4, d]
    const float* ln_final;  // [2, d]
    const uint8_t* wq_base;    // INT4 nibbles of all layers, layer after layer
    const float* ws_base;      // group scales, same order
    float* kc;             // the stepped sequence's rows of layer 0
    float* vc;
    int kv_seqs;           // sequences in the cache (its batch)
    // step
    const int64_t* token;  // [B]
    float* logits;         // [B, V]
    int64_t* next;         // [B]
    int t0;                // position of the appended row
    uint32_t epoch;        // unique per step (tags exchanged data)
    int a8;                // 1: W4A8 projections
    // workspace
    float* resid;          // [B, d] residual stream
    void* xbuf;            // exchange buffers
    int* err;
    void* trace;           // optional phase timestamps (NULL = off)
};
// Batches of up to kPersistentMaxSeqs sequences take the persistent step,
// one launch per sequence (B = 1 within each launch).
constexpr int kPersistentMaxSeqs = 2;
bool persistent_supported(int d, int F, int H, int B, int V);
size_t persistent_xbuf_bytes(int L, int d, int F, int H, int B, int V);
hipError_t launch_persistent_decode(const PersistentArgs& a, hipStream_t st);
// Writes the workgroup role table into a freshly zeroed exchange buffer.
hipError_t persistent_prepare(void* xbuf, int L, int d, int F, hipStream_t st);
int persistent_max_position(int d, int F);
size_t persistent_trace_bytes(int L);

// Single-launch decode step for a batch of 2 .. 8 sequences, one XCD per
// sequence (mt_decode_batched.hip); INT4 weights, FP32 (or W4A8 INT8)
// activations, d_model 768, 1024 or 1536.  Sequences may sit at different
// positions.
struct BatchedArgs {
    int L, d, H, F, V, B, t_cap;
    float eps;
    const float* tok_emb;
    const float* lm_head;
    const float* ln;        // [L, 4, d]
    const float* ln_final;  // [2, d]
    const uint8_t* wq_base;
    const float* ws_base;
    float* kc;              // layer 0, sequence 0 of the cache [L][kv_seqs][t_cap][d]
    float* vc;
    int kv_seqs;
    const int64_t* token;   // [B]
    float* logits;          // [B, V]
    int64_t* next;          // [B]
    int t0[8];              // T_past of each sequence (< t_cap)
    uint32_t epoch;
    void* xbuf;             // exchange words, batched_xbuf_bytes
    int* err;
    void* trace;            // optional phase timestamps (NULL = off), persistent_trace_bytes
    int a8;                 // 1: W4A8 projections
};
// MT_DECODE_AUTO takes the batched step from this batch size on (at B = 2
// the two persistent launches are faster: 0.774 against 0.839 ms per
// guided token on the medium CFG pair decoding to 2048 positions).
constexpr int kBatchedAutoSeqs = 3;
// Sequences per launch of the batched step (one per XCD); batches of up to
// kBatchedMaxSeqs run as one launch per group of this many.
constexpr int kBatchedGroup = 8;
constexpr int kBatchedMaxSeqs = 16;
bool batched_supported(int d, int F, int H, int B, int V);
size_t batched_xbuf_bytes(int L, int d, int F, int B);
hipError_t launch_batched_decode(const BatchedArgs& a, hipStream_t st);

// Fixed workspace of mt_prefill_noalloc (mt_scratch.hip): its size in
// floats, and the address of the calling device's copy (call with `device`
// current; the address is looked up once per device and kept).
size_t noalloc_scratch_floats();
hipError_t noalloc_scratch_setup(int device, float** out);

}  // namespace mt
