// Persistent single-launch decode step for B = 1 on MI355X (gfx950).
//
// One launch computes one greedy decode step of the whole decoder: token
// embedding, for every layer the pre-norm attention block (LayerNorm, fused
// QKV projection, attention over the fixed-capacity cache with the new K/V
// row written in place, O projection, residual) and the pre-norm FFN block
// (LayerNorm, FFN-up + GELU, FFN-down, residual), then the final LayerNorm,
// the FP32 LM head and the greedy argmax.  These are the decoder operations
// the pages list: four INT4 group-32 MatMulNBits projections, one
// GroupQueryAttention and two SkipLayerNormalization nodes per layer, FP32
// cache and activations ("MuScriptor Medium -- optimized W4A32 ONNX Runtime"
// README, "Model variant"); one decoder call appends a row at T_past and
// returns last-position logits ("unifolia/muscriptor-small-onnx", decoder).
//
// Execution model.  256 workgroups, one per CU, stay resident for the whole
// step.  Data moves between workgroups through exchange words of 64 bits,
// {float value, 32-bit step tag}, each written by one atomic 8-byte store;
// a consumer issues all its reads at once and re-reads only the words whose
// tag is not yet this step's.  No barrier counters, no cache flushes.  A
// vector that every workgroup reads is written once per XCD and each XCD's
// workgroups poll their own copy, which keeps the number of pollers per
// cache line low.  Every workgroup keeps its own copy of the residual
// stream in LDS and recomputes LayerNorm locally.  Weights for a phase are
// loaded into registers one phase ahead; each attention workgroup DMAs its
// K/V chunk of the next layer into LDS as soon as the current chunk is
// consumed.
//
// Roles (a table built on the host, see build_roles):
//   attention WGs  (head h, split s), 16 splits per head at small width, 8
//                  otherwise, all on one XCD.  Each recomputes q_h (at medium
//                  width: gathers it) and the softmax partial over its chunk
//                  of cached positions; splits 1.. publish (max, sum,
//                  acc[64]); split 0 (the head leader) merges them with the
//                  new position and publishes attn_h.
//   free WGs       the rest: the new K/V rows of the fused projection (to the
//                  cache slot T_past and to the exchange); at medium width
//                  also 8 q rows each; tail splits past the attention splits'
//                  reach.
//   free WGs       also the O projection (D / free WGs rows each).
//   all WGs        F/256 rows of FFN-up + GELU and D/256 rows of FFN-down.
// Per layer: A (attention partials / K,V rows) -> A2 (head merge) -> B (O)
// -> C (LN2 + up) -> D (down) -> next layer's A; after the last layer E
// (LN_f + LM-head rows + local argmax) and F (workgroup 0: global argmax,
// lowest index on ties).
//
// Every wait is bounded: past the spin limit the workgroup sets bit 2 of the
// error word and all workgroups leave; mt_check reports it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mt_internal.h"
#include "mt_pd_common.h"

namespace mt {
namespace pd {

constexpr int MAXPOS = 256;  // cached positions per attention workgroup (LDS)
constexpr int LM_ROWS = 6;   // vocabulary rows per workgroup
constexpr int TRACE_SLOTS = 24;

// Role of one workgroup (host-built table, constant for a model).
struct Role {
    int head;       // attention head, -1 if none
    int split;      // attention split (0 = head leader)
    int kv_row0;    // first row of the 2D K|V rows of the fused projection
    int kv_rows;    // number of K|V rows, 0 if none
    int o_row0;     // first of this workgroup's O-projection rows, -1 if none
    int tail_head;  // free workgroups: head of this workgroup's tail split, -1 if none
    int tail_idx;   // its index among the head's tail splits
    int q_row0;     // free workgroups with Cfg::QF: first of its Q_ROWS q rows, -1 if none
};

template <int D, int F>
struct Cfg {
    static constexpr int H = D / 64;
    static constexpr int GD = D / 32, GF = F / 32;
    static constexpr int LPR_D = lpr_for(D), CPL_D = GD / (LPR_D ? LPR_D : 1), RP_D = NT / (LPR_D ? LPR_D : 1);
    static constexpr int LPR_F = lpr_for(F), CPL_F = GF / (LPR_F ? LPR_F : 1), RP_F = NT / (LPR_F ? LPR_F : 1);
    // attention splits per head: 16 where that leaves at least 64 workgroups
    // for the new K/V rows and the O projection, else 8; each holds up to MP
    // cached positions in LDS.  (16 splits at medium width leave no such
    // workgroups: the K/V and O rows then land on the attention workgroups,
    // whose loads complete in order behind their K/V chunk DMA; measured
    // 17 % slower.)
    static constexpr int ATT_S = H * 16 + 64 <= NWG ? 16 : 8;
    static constexpr int MP = MAXPOS;
    static constexpr int NATT = H * ATT_S;
    static constexpr int NFREE = NWG - NATT;
    // Positions past ATT_S * MP go to tail splits on the free workgroups (TS
    // per head, up to MAXPOS positions each), which are idle while the
    // attention workgroups compute q_h and their partials; the head leader
    // merges them with the other partials.
    static constexpr int TS = NFREE / H;
    static constexpr int SLOTS = ATT_S + TS;  // partial slots per head
    static constexpr int REACH = ATT_S * MP + TS * MAXPOS;
    static constexpr int KV_ROWS = cdiv(2 * D, NFREE);
    // QF: the q rows are computed by the free workgroups, Q_ROWS each, next
    // to their K/V rows, and gathered by the attention workgroups, which
    // then need neither LN1 nor the head's 64 q rows (1.75 us of a medium
    // layer on the critical path, against one pass of Q_ROWS rows and an
    // exchange inside the XCD), and nor do the tail splits.  Possible where
    // every head's q rows fit on free workgroups of the head's own XCD
    // (medium width); used in the instantiation with tail splits only.
    // Measured at medium: 383 -> 391 us per step at T = 600 (the free
    // workgroups' K/V rows, which the head merge waits for, come a pass
    // later), even at T = 1100 and 2000, 458 -> 443 us at T = 2450 (the tail
    // splits skip their 64-row dot).
    static constexpr int Q_ROWS = 8;
    static constexpr bool QF = NFREE == NATT && NFREE * Q_ROWS == D;
    static constexpr int UP_ROWS = cdiv(F, NWG);
    static constexpr int O_ROWS = cdiv(D, NFREE);  // O rows: free workgroups only
    static constexpr int DN_ROWS = cdiv(D, NWG);
    static constexpr int NP_Q = cdiv(64, RP_D);
    static constexpr int NP_QF = cdiv(Q_ROWS, RP_D);
    static constexpr int NP_KV = cdiv(KV_ROWS, RP_D);
    static constexpr int NP_O = cdiv(O_ROWS, RP_D);
    static constexpr int NP_UP = cdiv(UP_ROWS, RP_D);
    static constexpr int NP_DN = cdiv(DN_ROWS, RP_F);
    // exchange layout per layer (64-bit words).  Vectors every workgroup
    // reads are written REP times; the workgroups of XCD x read copy x, so
    // no line is polled by more than 32 workgroups.
    static constexpr int XA_KV = 0;                     // new K|V row [2D]
    // q row [D], with tail splits only: with QF all of it from the free
    // workgroups, else head h's 64 rows from the head's first attention split
    static constexpr int XA_Q = XA_KV + 2 * D;
    static constexpr int XA_PART = XA_Q + D;            // partials [H][SLOTS][PW]
    static constexpr int XB_ATT = XA_PART + H * SLOTS * PW;  // merged attention [REP][D]
    static constexpr int XB_O = XB_ATT + REP * D;       // o [REP][D]
    static constexpr int XC = XB_O + REP * D;           // u [REP][F]
    static constexpr int XD = XC + REP * F;             // f [REP][D]
    static constexpr int LAYER_WORDS = rup(XD + REP * D, 2);
    // LDS layout (floats).  The K|V chunk of an attention split stays
    // resident across phases B..D (it is the next layer's chunk by then), so
    // u of phase D shares one region with the vectors of phases A..C.
    static constexpr int BIG = 2 * MP * 64;               // K|V chunk
    static constexpr int OFF_XS = BIG;                    // group sums of act [GD]
    static constexpr int OFF_US = OFF_XS + GD;            // group sums of u [GF]
    static constexpr int OFF_U = rup(OFF_US + GF, 4);     // u [F] (phase D) or:
    static constexpr int OFF_ACT = OFF_U;                 //   act [D]
    static constexpr int OFF_QH = OFF_ACT + D;            //   q_h [64]
    static constexpr int OFF_SC = OFF_QH + 64;            //   scores [MP]
    static constexpr int OFF_PART = OFF_SC + MP;          //   own partial [PW] + gathered [SLOTS-1][PW] + kv_new [128]
    // [4][64] scratch, also the staging of each phase's outputs: outside the
    // u region, because phase D writes it while other waves may still be
    // reading u
    static constexpr int OFF_COMB = rup(cmax(OFF_PART + SLOTS * PW + 128, OFF_U + F), 4);
    static constexpr int OFF_RED = rup(OFF_COMB + 4 * 64, 4);
    static constexpr int OFF_FLAG = OFF_RED + 16;
    static constexpr int LDS_FLOATS = OFF_FLAG + 16;
    static_assert(D % NT == 0 && F % NT == 0 && NT == 256, "widths");
    static_assert(LPR_D > 0 && LPR_F > 0, "width has no GEMV lane mapping");
    static_assert(NFREE >= 64 && KV_ROWS * NFREE >= 2 * D, "K/V rows need workgroups without attention duty");
    static_assert(TS >= 1 && TS * H <= NFREE, "tail splits");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
    // Regions that are live in the same phase must not overlap:
    //   all phases: the K|V chunk (BIG), xs, us, comb, red, flag;
    //   phases A, A2 (attention, head merge): act, qh, sc, the partials;
    //   phases B, C: act; phase D: u (which overlays act .. partials).
    static constexpr bool disjoint(int a, int na, int b, int nb) { return a + na <= b || b + nb <= a; }
    static_assert(disjoint(0, BIG, OFF_XS, GD) && disjoint(OFF_XS, GD, OFF_US, GF), "chunk / group sums");
    static_assert(disjoint(OFF_US, GF, OFF_U, F) && disjoint(OFF_XS, GD, OFF_U, F), "group sums / u");
    static_assert(disjoint(OFF_ACT, D, OFF_QH, 64) && disjoint(OFF_QH, 64, OFF_SC, MP) &&
                      disjoint(OFF_SC, MP, OFF_PART, SLOTS * PW + 128) &&
                      disjoint(OFF_ACT, D, OFF_PART, SLOTS * PW + 128),
                  "phase A regions");
    static_assert(disjoint(OFF_COMB, 4 * 64, OFF_U, F) && disjoint(OFF_COMB, 4 * 64, OFF_PART, SLOTS * PW + 128) &&
                      disjoint(OFF_COMB, 4 * 64, OFF_ACT, D) && disjoint(OFF_COMB, 4 * 64, 0, BIG),
                  "staging / vectors");
    static_assert(disjoint(OFF_RED, 16, OFF_COMB, 4 * 64) && disjoint(OFF_FLAG, 16, OFF_RED, 16) &&
                      OFF_FLAG + 16 <= LDS_FLOATS,
                  "reductions / flag");
    // W4A8 codes of a vector of n inputs take n bytes, followed by n / 32
    // reciprocal scales, inside the vector's own region
    static_assert(D / 4 + GD <= D && F / 4 + GF <= F, "W4A8 code layout");
};

struct Args {
    int L, V, t_cap;
    float eps;
    const float* tok_emb;
    const float* lm_head;
    const float* ln;
    const float* ln_final;
    // INT4 projections of all layers, laid out layer after layer:
    // QKV [3D, D], O [D, D], up [F, D], down [D, F] (nibbles / scales)
    const uint8_t* wq;
    const float* ws;
    long wq_layer;  // bytes per layer
    long ws_layer;  // floats per layer
    float* kc;    // this sequence's rows of layer 0: [t_cap, H, 64]
    float* vc;
    int kv_seqs;  // sequences in the cache (layer stride kv_seqs * t_cap * D)
    const int64_t* token;
    float* logits;
    int64_t* next;
    int t0;       // position of the appended row (T_past)
    int chunk;    // cached positions per attention split
    int tail0;    // first position of the tail splits (ATT_S * chunk)
    int tail_chunk;  // cached positions per tail split, 0 when T_past <= ATT_S * MP
    uint32_t epoch;
    uint64_t* x;  // exchange words
    const Role* roles;
    int* err;
    unsigned nib;     // 0x0F0F0F0F (nibble mask, see dot_u)
    int a8;           // 1: W4A8 projections (INT8 activation codes, INT32 group sums)
    uint64_t* trace;  // optional: [NWG][L + 1][TRACE_SLOTS] wall-clock stamps
};

__device__ __forceinline__ void stamp(const Args& a, int l, int k) {
    if (a.trace && threadIdx.x == 0)
        a.trace[((size_t)blockIdx.x * (a.L + 1) + l) * TRACE_SLOTS + k] = wall_clock64();
}

// The rows' dot products in the arithmetic the step runs (W4A32 or W4A8).
template <int LPR, int CPL, int NP>
__device__ __forceinline__ void dot_rows(const WBlk<CPL, NP>& w, const float* act, const float* xs, float (&out)[NP],
                                         const Args& a) {
    if (a.a8) wblk_dot8<LPR, CPL, NP>(w, reinterpret_cast<const int8_t*>(act), xs, out);
    else wblk_dot<LPR, CPL, NP>(w, act, xs, out, a.nib);
}

// K/V rows of one head at positions [p0, p0 + npos) of one layer's cache
// (npos <= MP), DMA'd into LDS: K at big[0 ..), V at big[MP * 64 ..), 64
// floats per row.  The loads are non-temporal: a step streams the whole
// live cache once, and left to the default policy it pushes the weights,
// which every step reads again, out of the caches (per step at medium:
// 395 -> 380 us at T = 1100, 415 -> 398 us at T = 2000).  Row t holds its 16-byte chunk c (dimensions 4c .. 4c+3) in slot
// (c + t) & 15, so lanes that read chunk c of consecutive rows touch
// different banks while c itself stays uniform across the wave.  One DMA
// instruction fills 4 rows: lane L lands in slot L & 15 of row L >> 4 and so
// fetches that row's chunk ((L & 15) - t) & 15.
template <int D, int MP>
__device__ __forceinline__ void kv_chunk_dma(const float* kc_l, const float* vc_l, int head, int p0,
                                             int npos, float* big) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rounds = (npos + 15) / 16;
    for (int rd = 0; rd < rounds; ++rd) {
        const int pl = rd * 16 + wave * 4;
        const int t = pl + (lane >> 4);
        const int pos = t < npos ? p0 + t : p0;  // in-range address; the slot is never read
        const size_t off = (size_t)pos * D + head * 64 + ((((lane & 15) - t) & 15) << 2);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kc_l + off),
                                         (__attribute__((address_space(3))) void*)(big + pl * 64), 16, 0, 2);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vc_l + off),
                                         (__attribute__((address_space(3))) void*)(big + MP * 64 + pl * 64),
                                         16, 0, 2);
    }
}

// Softmax partial of q over the npos cached positions in LDS (rows laid out
// by kv_chunk_dma).  Scores: thread t takes position t; each step reads four
// chunks of its K row (rotated slots, no bank conflicts) and the same four
// chunks of q (one address for the whole wave, a broadcast).
// Then lanes = dimensions for sum_t p_t V_t, four positions per step with
// two accumulator sets.  Writes (max, sum, acc[64]) to part[0], part[1],
// part[2 ..].
template <int MP>
__device__ __forceinline__ void attend_chunk(const float* big, const float* qh, int npos, float* sc,
                                             float* comb, float* red, float* part, const Args& a, int l) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float s = -INFINITY;
    if (tid < npos) {
        const float* kr = big + tid * 64;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c0 = 0; c0 < 16; c0 += 4) {
            float4 k4[4], q4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                k4[c] = *reinterpret_cast<const float4*>(kr + (((c0 + c + tid) & 15) << 2));
                q4[c] = reinterpret_cast<const float4*>(qh)[c0 + c];  // same address in every lane
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = fmaf(q4[c].x, k4[c].x, fmaf(q4[c].y, k4[c].y, fmaf(q4[c].z, k4[c].z, fmaf(q4[c].w, k4[c].w, acc[c]))));
        }
        s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * 0.125f;
    }
    stamp(a, l, 12);
    const float M = block_reduce<true>(s, red);
    const float pe = (tid < npos) ? expf(s - M) : 0.f;
    if (tid < MP) sc[tid] = pe;
    const float Ls = block_reduce<false>(pe, red + 4);
    stamp(a, l, 13);
    // sum_t p_t V_t: lane (wave w, row r, c) takes dimensions 4c .. 4c+3 of
    // positions 4w + r + 16i; the 4 rows of a wave are summed lane-wise,
    // then the 4 waves through LDS.
    const float* vbase = big + MP * 64;
    const int row = lane >> 4, c4 = lane & 15;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    auto vrow = [&](int t) { return *reinterpret_cast<const float4*>(vbase + t * 64 + (((c4 + t) & 15) << 2)); };
    auto acc4 = [](float4& acc, float p, const float4& v) {
        acc.x = fmaf(p, v.x, acc.x); acc.y = fmaf(p, v.y, acc.y); acc.z = fmaf(p, v.z, acc.z); acc.w = fmaf(p, v.w, acc.w);
    };
    int t = 4 * wave + row;
    for (; t + 48 < npos; t += 64) {
        const float p0 = sc[t], p1 = sc[t + 16], p2 = sc[t + 32], p3 = sc[t + 48];
        const float4 v0 = vrow(t), v1 = vrow(t + 16), v2 = vrow(t + 32), v3 = vrow(t + 48);
        acc4(a0, p0, v0);
        acc4(a1, p1, v1);
        acc4(a0, p2, v2);
        acc4(a1, p3, v3);
    }
    for (; t < npos; t += 16) acc4(a0, sc[t], vrow(t));
    float r4[4] = {a0.x + a1.x, a0.y + a1.y, a0.z + a1.z, a0.w + a1.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {  // lane-wise sum of the 4 rows
        r4[k] += __shfl_xor(r4[k], 16);
        r4[k] += __shfl_xor(r4[k], 32);
    }
    if (row == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) comb[wave * 64 + c4 * 4 + k] = r4[k];
    }
    stamp(a, l, 14);
    lds_barrier();
    if (tid < 64) {
        part[2 + tid] = npos > 0 ? (comb[tid] + comb[64 + tid]) + (comb[128 + tid] + comb[192 + tid]) : 0.f;
        if (tid == 0) {
            part[0] = npos > 0 ? M : -INFINITY;
            part[1] = npos > 0 ? Ls : 0.f;
        }
    }
    lds_barrier();
}

// LM-head rows of this workgroup (wave w: rows w and w + 4 of its six).
template <int D>
__device__ __forceinline__ void lm_rows_load(float4 (&wrow)[2][D / 256], const float* lm_head, int V) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int v = blockIdx.x * LM_ROWS + wave + 4 * i;
        const bool ok = v < V && wave + 4 * i < LM_ROWS;
#pragma unroll
        for (int c = 0; c < D / 256; ++c)
            wrow[i][c] = ok ? gload(reinterpret_cast<const float4*>(lm_head + (size_t)v * D) + lane + 64 * c)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// ---------------------------------------------------------------- the kernel

// LDS regions of one workgroup.
template <int D, int F>
struct Lds {
    float *big, *xs, *us, *u, *act, *qh, *sc, *own, *gpart, *knew, *vnew, *comb, *red;
    int* s_flag;
    __device__ explicit Lds(float* lds) {
        using C = Cfg<D, F>;
        big = lds;
        xs = lds + C::OFF_XS;
        us = lds + C::OFF_US;
        u = lds + C::OFF_U;
        act = lds + C::OFF_ACT;
        qh = lds + C::OFF_QH;
        sc = lds + C::OFF_SC;
        own = lds + C::OFF_PART;  // own partial [PW]
        gpart = own + PW;                   // slots 1 .. SLOTS-1 [SLOTS-1][PW]
        knew = gpart + (C::SLOTS - 1) * PW; // [64]
        vnew = knew + 64;         // [64]
        comb = lds + C::OFF_COMB; // [4][64] scratch
        red = lds + C::OFF_RED;
        s_flag = reinterpret_cast<int*>(lds + C::OFF_FLAG);
    }
};

// Byte / float offsets of the four projections inside one layer.
template <int D, int F>
struct Off {
    static constexpr long QO = 0, OO = 3L * D * D / 2, UO = 4L * D * D / 2, DO = (4L * D * D + (long)F * D) / 2;
    static constexpr long QS = 0, OS = 3L * D * D / 32, US = 4L * D * D / 32, DS = (4L * D * D + (long)F * D) / 32;
};

// Weights of phases B, C and D of one layer for this workgroup, plus LN2.
template <int D, int F>
struct BcdW {
    using C = Cfg<D, F>;
    WBlk<C::CPL_D, C::NP_O> wo;
    WBlk<C::CPL_D, C::NP_UP> wu;
    WBlk<C::CPL_F, C::NP_DN> wd;
    LnRegs<D> ln2;
};

// Loads of the O rows (orow < 0: none), the up rows and LN2 (issued during
// phase A).
template <int D, int F>
__device__ __forceinline__ void load_bc(BcdW<D, F>& w, const uint8_t* wq, const float* ws, const float* ln, int orow) {
    using C = Cfg<D, F>;
    using O = Off<D, F>;
    const int urow = blockIdx.x * C::UP_ROWS;
    if (orow >= 0)
        wblk_load<C::LPR_D, C::CPL_D, C::NP_O>(w.wo, wq + O::OO, ws + O::OS, D, orow, max(0, min(C::O_ROWS, D - orow)));
    wblk_load<C::LPR_D, C::CPL_D, C::NP_UP>(w.wu, wq + O::UO, ws + O::US, D, urow, max(0, min(C::UP_ROWS, F - urow)));
    ln_load<D>(w.ln2, ln + 2 * D, ln + 3 * D);
}

// Loads of the FFN-down rows, issued once phase C has published u: loads
// complete in order, so issued before phase C they held up its exchange
// read of o (measured 398.6 vs 402.4 us per step at T = 1100, 414 vs 424 at
// T = 2000); the u exchange that follows is long enough to hide them.
template <int D, int F>
__device__ __forceinline__ void load_d(BcdW<D, F>& w, const uint8_t* wq, const float* ws) {
    using C = Cfg<D, F>;
    using O = Off<D, F>;
    const int drow = blockIdx.x * C::DN_ROWS;
    wblk_load<C::LPR_F, C::CPL_F, C::NP_DN>(w.wd, wq + O::DO, ws + O::DS, F, drow, max(0, min(C::DN_ROWS, D - drow)));
}

// Phase B (workgroups without attention duty): attn -> O rows -> exchange.
// The attention workgroups skip it: their next-layer K/V chunk DMA, issued
// just before, would hold up their exchange reads (loads complete in order).
template <int D, int F>
__device__ __forceinline__ bool phase_b(const Args& a, const Lds<D, F>& S, uint64_t* X, const BcdW<D, F>& w, int orow,
                                        int l) {
    using C = Cfg<D, F>;
    const uint32_t ep = a.epoch;
    if (orow < 0) return true;
    if (!gather_to_lds<D / NT>(rep_of(X + C::XB_ATT, D), D, S.act, S.xs, ep, a.err, S.s_flag, a.a8)) return false;
    stamp(a, l, 6);
    float o[C::NP_O];
    dot_rows<C::LPR_D, C::CPL_D, C::NP_O>(w.wo, S.act, S.xs, o, a);
#pragma unroll
    for (int p = 0; p < C::NP_O; ++p) {
        const int rr = out_row<C::LPR_D>(p);
        if (rr >= 0 && rr < C::O_ROWS && orow + rr < D) S.comb[rr] = o[p];
    }
    publish_rep(X + C::XB_O, D, orow, S.comb, min(C::O_ROWS, D - orow), ep);
    stamp(a, l, 7);
    return true;
}

// Phase C (every workgroup): r += o; LN2; FFN-up rows + GELU -> exchange.
template <int D, int F>
__device__ __forceinline__ bool phase_c(const Args& a, const Lds<D, F>& S, uint64_t* X, const BcdW<D, F>& w,
                                        float (&r)[LnRegs<D>::PER], int l) {
    using C = Cfg<D, F>;
    const uint32_t ep = a.epoch;
    float o_in[LnRegs<D>::PER];
    if (!ll_gather_regs<LnRegs<D>::PER>(rep_of(X + C::XB_O, D), D, o_in, ep, a.err)) *S.s_flag = 1;
    stamp(a, l, 8);
    if (!residual_layernorm<D, true>(r, o_in, true, w.ln2, a.eps, S.act, S.xs, S.red, S.s_flag, a.a8)) return false;
    float o[C::NP_UP];
    dot_rows<C::LPR_D, C::CPL_D, C::NP_UP>(w.wu, S.act, S.xs, o, a);
    const int urow = blockIdx.x * C::UP_ROWS;
#pragma unroll
    for (int p = 0; p < C::NP_UP; ++p) {
        const int rr = out_row<C::LPR_D>(p);
        if (rr >= 0 && rr < C::UP_ROWS && urow + rr < F) S.comb[rr] = gelu_erf(o[p]);
    }
    publish_rep(X + C::XC, F, urow, S.comb, max(0, min(C::UP_ROWS, F - urow)), ep);
    stamp(a, l, 9);
    return true;
}

// Phase D (every workgroup): u -> FFN-down rows of this workgroup -> exchange.
template <int D, int F>
__device__ __forceinline__ bool phase_d(const Args& a, const Lds<D, F>& S, uint64_t* X, const BcdW<D, F>& w, int l) {
    using C = Cfg<D, F>;
    const uint32_t ep = a.epoch;
    if (!gather_to_lds<F / NT>(rep_of(X + C::XC, F), F, S.u, S.us, ep, a.err, S.s_flag, a.a8)) return false;
    stamp(a, l, 10);
    float o[C::NP_DN];
    dot_rows<C::LPR_F, C::CPL_F, C::NP_DN>(w.wd, S.u, S.us, o, a);
    const int drow = blockIdx.x * C::DN_ROWS;
#pragma unroll
    for (int p = 0; p < C::NP_DN; ++p) {
        const int rr = out_row<C::LPR_F>(p);
        if (rr >= 0 && rr < C::DN_ROWS && drow + rr < D) S.comb[rr] = o[p];
    }
    publish_rep(X + C::XD, D, drow, S.comb, min(C::DN_ROWS, D - drow), ep);
    stamp(a, l, 11);
    return true;
}

// Start of phase A: r += f of the previous layer (if any); LN1 into act.
template <int D, int F>
__device__ __forceinline__ bool phase_a_ln(const Args& a, const Lds<D, F>& S, const LnRegs<D>& ln1,
                                           float (&r)[LnRegs<D>::PER], int l) {
    using C = Cfg<D, F>;
    stamp(a, l, 0);
    float f[LnRegs<D>::PER] = {};
    if (l > 0) {
        const uint64_t* Xp = a.x + (size_t)(l - 1) * C::LAYER_WORDS;
        if (!ll_gather_regs<LnRegs<D>::PER>(rep_of(Xp + C::XD, D), D, f, a.epoch, a.err)) *S.s_flag = 1;
    }
    stamp(a, l, 1);
    if (!residual_layernorm<D, true>(r, f, l > 0, ln1, a.eps, S.act, S.xs, S.red, S.s_flag, a.a8)) return false;
    stamp(a, l, 2);
    return true;
}

// Start of phase A without LN1 (QF attention workgroups): r += f of the
// previous layer (if any).
template <int D, int F>
__device__ __forceinline__ bool phase_a_add(const Args& a, const Lds<D, F>& S, float (&r)[LnRegs<D>::PER], int l) {
    using C = Cfg<D, F>;
    stamp(a, l, 0);
    if (l > 0) {
        const uint64_t* Xp = a.x + (size_t)(l - 1) * C::LAYER_WORDS;
        float f[LnRegs<D>::PER];
        if (!ll_gather_regs<LnRegs<D>::PER>(rep_of(Xp + C::XD, D), D, f, a.epoch, a.err)) *S.s_flag = 1;
#pragma unroll
        for (int i = 0; i < LnRegs<D>::PER; ++i) r[i] += f[i];
        lds_barrier();
        if (*S.s_flag) return false;
    }
    stamp(a, l, 1);
    return true;
}

// Every layer for an attention workgroup (head h, split s).  TAIL: the
// cache reaches past the attention splits, and the head leader also merges
// the tail splits' partials.
template <int D, int F, bool TAIL>
__device__ __forceinline__ bool attention_role(const Args& a, const Lds<D, F>& S, const Role& role,
                                               float (&r)[LnRegs<D>::PER]) {
    using C = Cfg<D, F>;
    using O = Off<D, F>;
    const uint32_t ep = a.epoch;
    const int tid = threadIdx.x;
    constexpr int AS = C::ATT_S;
    constexpr bool QF = C::QF && TAIL;  // q rows on the free workgroups (see Cfg::QF)
    const bool leader = role.split == 0;
    const int h = role.head;
    const int p0 = role.split * a.chunk;
    const int npos = max(0, min(a.t0, p0 + a.chunk) - p0);
    const size_t lstride = (size_t)a.kv_seqs * a.t_cap * D;  // one layer of the cache
    // (with QF the head's q rows and LN1 come from the free workgroups)
    WBlk<C::CPL_D, QF ? 1 : C::NP_Q> wqh;
    BcdW<D, F> w;
    LnRegs<D> ln1;
    if (npos > 0) kv_chunk_dma<D, C::MP>(a.kc, a.vc, h, p0, npos, S.big);
    if constexpr (!QF) {
        wblk_load<C::LPR_D, C::CPL_D, C::NP_Q>(wqh, a.wq + O::QO, a.ws + O::QS, D, h * 64, 64);
        ln_load<D>(ln1, a.ln, a.ln + D);
    }
    for (int l = 0; l < a.L; ++l) {
        uint64_t* X = a.x + (size_t)l * C::LAYER_WORDS;
        const uint8_t* wq = a.wq + l * a.wq_layer;
        const float* ws = a.ws + l * a.ws_layer;
        const float* ln = a.ln + (size_t)l * 4 * D;
        const float* kc_l = a.kc + (size_t)l * lstride;
        const float* vc_l = a.vc + (size_t)l * lstride;
        const bool last = l + 1 == a.L;
        // ---- A: r += f_prev; q_h (LN1 and the dot here, or gathered);
        // softmax partial over the chunk
        if constexpr (QF) {
            if (!phase_a_add<D, F>(a, S, r, l)) return false;
            if (!ll_gather1<1, false>(X + C::XA_Q + h * 64, 64, S.qh, ep, a.err, S.s_flag)) return false;
        } else {
            if (!phase_a_ln<D, F>(a, S, ln1, r, l)) return false;
            float o[C::NP_Q];
            dot_rows<C::LPR_D, C::CPL_D, C::NP_Q>(wqh, S.act, S.xs, o, a);
#pragma unroll
            for (int p = 0; p < C::NP_Q; ++p) {
                const int rr = out_row<C::LPR_D>(p);
                if (rr >= 0 && rr < 64) {
                    S.qh[rr] = o[p];
                    // the head's tail splits gather q_h from its first split
                    if (TAIL && leader) ll_put(X + C::XA_Q + h * 64 + rr, o[p], ep);
                }
            }
        }
        stamp(a, l, 15);
        __builtin_amdgcn_s_waitcnt(0);  // the K/V chunk DMA (and every earlier load) has landed
        lds_barrier();
        stamp(a, l, 3);
        attend_chunk<C::MP>(S.big, S.qh, npos, S.sc, S.comb, S.red + 8, S.own, a, l);
        stamp(a, l, 4);
        if (!leader) {
            uint64_t* pw = X + C::XA_PART + (size_t)(h * C::SLOTS + role.split) * PW;
            if (tid < PW) ll_put(pw + tid, S.own[tid], ep);
            // the next layer's chunk: this workgroup's next exchange read
            // (phase C) is microseconds away
            if (!last && npos > 0) kv_chunk_dma<D, C::MP>(kc_l + lstride, vc_l + lstride, h, p0, npos, S.big);
        } else {
            // ---- A2: merge the splits (and the tail splits when the cache
            // reaches past them) and the new position -> attn_h
            constexpr int NS = TAIL ? C::SLOTS : AS;  // partial slots merged
            if (!ll_gather<cdiv((NS - 1) * PW + 128, NT), false>(
                    Range{X + C::XA_PART + (size_t)(h * C::SLOTS + 1) * PW, (NS - 1) * PW, S.gpart},
                    Range{X + C::XA_KV + h * 64, 64, S.knew}, Range{X + C::XA_KV + D + h * 64, 64, S.vnew}, ep,
                    a.err, S.s_flag))
                return false;
            stamp(a, l, 5);
            stamp(a, l, 16);
            if (tid < 64) {
                // every split's (sum, acc[tid]) into registers first, so the
                // LDS reads overlap; an empty split has max -inf, sum 0 and
                // acc 0, and its weight exp(-inf) is exactly 0.  The weights
                // are uniform across the wave: lane s < NS forms split s's,
                // lane NS the new position's, one exp per lane instead of
                // NS + 1 in every lane.
                static_assert(NS < 64, "one lane per partial and one for the new position");
                float pl[NS], pa[NS];
                pl[0] = S.own[1];
                pa[0] = S.own[2 + tid];
#pragma unroll
                for (int s = 1; s < NS; ++s) {
                    pl[s] = S.gpart[(s - 1) * PW + 1];
                    pa[s] = S.gpart[(s - 1) * PW + 2 + tid];
                }
                const float snew = wave_reduce<false>(S.qh[tid] * S.knew[tid]) * 0.125f;
                const float mx = tid == 0 ? S.own[0]
                                          : tid < NS ? S.gpart[(tid - 1) * PW] : tid == NS ? snew : -INFINITY;
                const float M = wave_reduce<true>(mx);
                const float wl = tid <= NS ? expf(mx - M) : 0.f;
                float Ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), NS));
                float A = Ls * S.vnew[tid];
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const float wgt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
                    Ls = fmaf(wgt, pl[s], Ls);
                    A = fmaf(wgt, pa[s], A);
                }
                ll_put_rep(X + C::XB_ATT, D, h * 64 + tid, A / Ls, ep);
            }
            stamp(a, l, 17);
            if (!last && npos > 0) kv_chunk_dma<D, C::MP>(kc_l + lstride, vc_l + lstride, h, p0, npos, S.big);
        }
        // ---- C, D (no phase B).  The FFN-up rows are requested here, behind
        // the next chunk's DMA (a few us per step faster than before the
        // attention at T <= 1100, even at T = 2000).
        load_bc<D, F>(w, wq, ws, ln, -1);
        if (!phase_c<D, F>(a, S, X, w, r, l)) return false;
        load_d<D, F>(w, wq, ws);
        if constexpr (!QF) {
            if (!last) {
                const uint8_t* wqn = wq + a.wq_layer;
                const float* wsn = ws + a.ws_layer;
                wblk_load<C::LPR_D, C::CPL_D, C::NP_Q>(wqh, wqn + O::QO, wsn + O::QS, D, h * 64, 64);
                ln_load<D>(ln1, ln + 4 * D, ln + 5 * D);
            }
        }
        if (!phase_d<D, F>(a, S, X, w, l)) return false;
    }
    return true;
}

// Every layer for a workgroup without attention duty: new K/V rows in
// phase A (with TAIL, then its tail split's partial); phases B, C, D like
// every workgroup.
template <int D, int F, bool TAIL>
__device__ __forceinline__ bool free_role(const Args& a, const Lds<D, F>& S, const Role& role,
                                          float (&r)[LnRegs<D>::PER]) {
    using C = Cfg<D, F>;
    using O = Off<D, F>;
    const uint32_t ep = a.epoch;
    const int tid = threadIdx.x;
    const size_t lstride = (size_t)a.kv_seqs * a.t_cap * D;
    // tail split: positions [tp0, tp0 + tnpos) of head th (none while the
    // cache ends within the attention splits' reach)
    const int th = TAIL ? role.tail_head : -1;
    constexpr bool QF = C::QF && TAIL;  // q rows on the free workgroups (see Cfg::QF)
    const int tp0 = a.tail0 + role.tail_idx * a.tail_chunk;
    const int tnpos = th >= 0 ? max(0, min(a.t0, tp0 + a.tail_chunk) - tp0) : 0;
    WBlk<C::CPL_D, C::NP_KV> wkv;
    WBlk<C::CPL_D, C::NP_QF> wqf;  // QF: this workgroup's q rows
    BcdW<D, F> w;
    LnRegs<D> ln1;
    if (tnpos > 0) kv_chunk_dma<D, MAXPOS>(a.kc, a.vc, th, tp0, tnpos, S.big);
    if (QF && role.q_row0 >= 0)
        wblk_load<C::LPR_D, C::CPL_D, C::NP_QF>(wqf, a.wq + O::QO, a.ws + O::QS, D, role.q_row0, C::Q_ROWS);
    if (role.kv_rows > 0)
        wblk_load<C::LPR_D, C::CPL_D, C::NP_KV>(wkv, a.wq + O::QO, a.ws + O::QS, D, D + role.kv_row0, role.kv_rows);
    ln_load<D>(ln1, a.ln, a.ln + D);
    for (int l = 0; l < a.L; ++l) {
        uint64_t* X = a.x + (size_t)l * C::LAYER_WORDS;
        const uint8_t* wq = a.wq + l * a.wq_layer;
        const float* ws = a.ws + l * a.ws_layer;
        const float* ln = a.ln + (size_t)l * 4 * D;
        float* kc_l = a.kc + (size_t)l * lstride;
        float* vc_l = a.vc + (size_t)l * lstride;
        const bool last = l + 1 == a.L;
        // ---- A: r += f_prev; LN1; (QF: q rows first, the attention
        // workgroups wait for them); new K/V rows
        if (!phase_a_ln<D, F>(a, S, ln1, r, l)) return false;
        if (QF && role.q_row0 >= 0) {
            float o[C::NP_QF];
            dot_rows<C::LPR_D, C::CPL_D, C::NP_QF>(wqf, S.act, S.xs, o, a);
#pragma unroll
            for (int p = 0; p < C::NP_QF; ++p) {
                const int rr = out_row<C::LPR_D>(p);
                if (rr >= 0 && rr < C::Q_ROWS) ll_put(X + C::XA_Q + role.q_row0 + rr, o[p], ep);
            }
        }
        if (role.kv_rows > 0) {
            float o[C::NP_KV];
            dot_rows<C::LPR_D, C::CPL_D, C::NP_KV>(wkv, S.act, S.xs, o, a);
#pragma unroll
            for (int p = 0; p < C::NP_KV; ++p) {
                const int rr = out_row<C::LPR_D>(p);
                if (rr >= 0 && rr < role.kv_rows) {
                    const int row = role.kv_row0 + rr;
                    const size_t slot = (size_t)a.t0 * D;
                    if (row < D) kc_l[slot + row] = o[p];
                    else vc_l[slot + row - D] = o[p];
                    ll_put(X + C::XA_KV + row, o[p], ep);
                }
            }
        }
        if (tnpos > 0) {
            // ---- tail split: the softmax partial over its positions, with
            // q_h gathered (from the free workgroups' q rows with QF, else
            // from the head's first attention split).  Computing q_h here
            // instead puts a 64-row dot, whose weights cannot be requested
            // ahead, on the chain to the head merge, and at large width its
            // 60 registers made the step spill.
            if (!ll_gather1<1, false>(X + C::XA_Q + th * 64, 64, S.qh, ep, a.err, S.s_flag)) return false;
            __builtin_amdgcn_s_waitcnt(0);  // the tail chunk DMA has landed
            lds_barrier();
            attend_chunk<MAXPOS>(S.big, S.qh, tnpos, S.sc, S.comb, S.red + 8, S.own, a, l);
            uint64_t* pw = X + C::XA_PART + (size_t)(th * C::SLOTS + C::ATT_S + role.tail_idx) * PW;
            if (tid < PW) ll_put(pw + tid, S.own[tid], ep);
            if (!last) kv_chunk_dma<D, MAXPOS>(kc_l + lstride, vc_l + lstride, th, tp0, tnpos, S.big);
        } else if (th >= 0) {
            // a tail split past the last position: the leader still gathers
            // every tail slot, so publish an empty partial (max -inf, sum 0)
            uint64_t* pw = X + C::XA_PART + (size_t)(th * C::SLOTS + C::ATT_S + role.tail_idx) * PW;
            if (tid < PW) ll_put(pw + tid, tid == 0 ? -INFINITY : 0.f, ep);
        }
        stamp(a, l, 18);
        load_bc<D, F>(w, wq, ws, ln, role.o_row0);
        // ---- B, C, D
        if (!phase_b<D, F>(a, S, X, w, role.o_row0, l)) return false;
        if (!phase_c<D, F>(a, S, X, w, r, l)) return false;
        load_d<D, F>(w, wq, ws);
        if (!last) {
            if (QF && role.q_row0 >= 0)
                wblk_load<C::LPR_D, C::CPL_D, C::NP_QF>(wqf, wq + a.wq_layer + O::QO, ws + a.ws_layer + O::QS, D,
                                                        role.q_row0, C::Q_ROWS);
            if (role.kv_rows > 0)
                wblk_load<C::LPR_D, C::CPL_D, C::NP_KV>(wkv, wq + a.wq_layer + O::QO, ws + a.ws_layer + O::QS, D,
                                                        D + role.kv_row0, role.kv_rows);
            ln_load<D>(ln1, ln + 4 * D, ln + 5 * D);
        }
        if (!phase_d<D, F>(a, S, X, w, l)) return false;
    }
    return true;
}

template <int D, int F, bool TAIL>
__global__ __launch_bounds__(NT, 1) void k_decode_step(Args a) {
    using C = Cfg<D, F>;
    extern __shared__ float lds[];
    const Lds<D, F> S(lds);
    const int wg = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const uint32_t ep = a.epoch;
    const Role role = a.roles[wg];
    if (tid == 0) *S.s_flag = 0;

    // embedding of the token: this workgroup's copy of the residual stream,
    // element tid + i * NT in r[i]
    float r[LnRegs<D>::PER];
    {
        const int64_t tok = gload(a.token);
        const bool bad = tok < 0 || tok >= a.V;
        if (bad && wg == 0 && tid == 0) atomicOr(a.err, 1);
#pragma unroll
        for (int i = 0; i < LnRegs<D>::PER; ++i) {
            const int k = tid + i * NT;
            r[i] = k >= D ? 0.f : (bad ? __builtin_nanf("") : gload(a.tok_emb + (size_t)tok * D + k));
        }
        lds_barrier();  // s_flag initialised
    }

    const bool ok = role.head >= 0 ? attention_role<D, F, TAIL>(a, S, role, r) : free_role<D, F, TAIL>(a, S, role, r);
    if (!ok) return;
    // LM-head rows and LN_f, loaded while the last layer's FFN-down output
    // is still in flight
    float4 wrow[2][D / 256];
    LnRegs<D> lnf;
    lm_rows_load<D>(wrow, a.lm_head, a.V);
    ln_load<D>(lnf, a.ln_final, a.ln_final + D);

    // ===================== phase E: r += f; z = LN_f(r); LM-head rows + local argmax
    uint64_t* XE = a.x + (size_t)a.L * C::LAYER_WORDS;
    {
        stamp(a, a.L, 0);
        const uint64_t* Xp = a.x + (size_t)(a.L - 1) * C::LAYER_WORDS;
        float f[LnRegs<D>::PER];
        if (!ll_gather_regs<LnRegs<D>::PER>(rep_of(Xp + C::XD, D), D, f, ep, a.err)) *S.s_flag = 1;
        stamp(a, a.L, 1);
        if (!residual_layernorm<D, false>(r, f, true, lnf, a.eps, S.act, nullptr, S.red, S.s_flag)) return;
        float* cand_v = S.comb;                              // [8]
        int* cand_i = reinterpret_cast<int*>(S.comb + 8);    // [8]
        if (tid < 8) {
            cand_v[tid] = -INFINITY;
            cand_i[tid] = 0x7fffffff;
        }
        lds_barrier();
        const int v0 = wg * LM_ROWS;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int v = v0 + wave + 4 * i;
            float acc = 0.f;
#pragma unroll
            for (int c = 0; c < D / 256; ++c) {
                const float4 z = reinterpret_cast<const float4*>(S.act)[lane + 64 * c];
                acc = fmaf(wrow[i][c].x, z.x, fmaf(wrow[i][c].y, z.y, fmaf(wrow[i][c].z, z.z, fmaf(wrow[i][c].w, z.w, acc))));
            }
            acc = wave_reduce<false>(acc);
            if (lane == 0 && v < a.V && wave + 4 * i < LM_ROWS) {
                a.logits[v] = acc;
                cand_v[wave + 4 * i] = acc;
                cand_i[wave + 4 * i] = v;
            }
        }
        lds_barrier();
        if (tid == 0) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int i = 0; i < 8; ++i) {
                const int ii = cand_i[i];
                if (ii == 0x7fffffff) continue;
                if (bi == 0x7fffffff || cand_v[i] > bv || (cand_v[i] == bv && ii < bi)) {
                    bv = cand_v[i];
                    bi = ii;
                }
            }
            ll_put(XE + 2 * wg, bv, ep);
            ll_put(XE + 2 * wg + 1, __int_as_float(bi), ep);
        }
    }

    // ===================== phase F: global argmax (workgroup 0)
    if (wg == 0) {
        float* cv = S.big;
        if (!ll_gather1<cdiv(2 * NWG, NT), false>(XE, 2 * NWG, cv, ep, a.err, S.s_flag)) return;
        if (tid < 64) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int i = tid; i < NWG; i += 64) {
                const float v = cv[2 * i];
                const int ii = __float_as_int(cv[2 * i + 1]);
                if (ii == 0x7fffffff) continue;
                if (bi == 0x7fffffff || v > bv || (v == bv && ii < bi)) {
                    bv = v;
                    bi = ii;
                }
            }
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const float ov = __shfl_xor(bv, o);
                const int oi = __shfl_xor(bi, o);
                if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (tid == 0) a.next[0] = bi == 0x7fffffff ? 0 : bi;
        }
        stamp(a, a.L, 2);
    }
}

// Role table for the shape: attention heads spread over the XCDs with the 8
// splits of a head on one XCD; O, FFN-down and K/V-row duties on the rest.
template <int D, int F>
static bool build_roles(Role* roles) {
    using C = Cfg<D, F>;
    int free_list[NWG];
    int nfree = 0;
    int nh_x[NXCD] = {0};
    for (int h = 0; h < C::H; ++h) ++nh_x[h % NXCD];
    for (int w = 0; w < NWG; ++w) {
        Role& r = roles[w];
        r = Role{-1, 0, 0, 0, -1, -1, 0, -1};
        const int x = w % NXCD, slot = w / NXCD;
        if (slot < nh_x[x] * C::ATT_S) {
            r.head = (slot / C::ATT_S) * NXCD + x;
            r.split = slot % C::ATT_S;
        } else {
            free_list[nfree++] = w;
        }
    }
    for (int i = 0; i < nfree; ++i) {
        Role& r = roles[free_list[i]];
        const int row0 = i * C::KV_ROWS;
        r.o_row0 = i * C::O_ROWS < D ? i * C::O_ROWS : -1;
        r.kv_row0 = row0;
        r.kv_rows = row0 < 2 * D ? (2 * D - row0 < C::KV_ROWS ? 2 * D - row0 : C::KV_ROWS) : 0;
    }
    // QF: head h's 64 q rows on 64 / Q_ROWS free workgroups of its XCD
    if (C::QF) {
        int next[NXCD] = {0};  // next free workgroup (index into free_list) to take, per XCD
        for (int h = 0; h < C::H; ++h) {
            const int xh = h % NXCD;
            for (int j = 0; j < 64 / C::Q_ROWS; ++j) {
                int i = next[xh];
                while (i < nfree && free_list[i] % NXCD != xh) ++i;
                if (i >= nfree) return false;
                roles[free_list[i]].q_row0 = h * 64 + j * C::Q_ROWS;
                next[xh] = i + 1;
            }
        }
    }
    // TS tail splits per head on free workgroups, first from the XCD of the
    // head (its leader's), then from any XCD
    bool used[NWG] = {};
    for (int h = 0; h < C::H; ++h) {
        const int xh = h % NXCD;
        for (int j = 0; j < C::TS; ++j) {
            int pick = -1;
            for (int pass = 0; pass < 2 && pick < 0; ++pass)
                for (int i = 0; i < nfree && pick < 0; ++i) {
                    const int w = free_list[i];
                    if (!used[w] && (pass == 1 || w % NXCD == xh)) pick = w;
                }
            used[pick] = true;  // TS * H <= NFREE: a free workgroup is always left
            roles[pick].tail_head = h;
            roles[pick].tail_idx = j;
        }
    }
    return true;
}

}  // namespace pd

// ---------------------------------------------------------------- host side

bool persistent_supported(int d, int F, int H, int B, int V) {
    if (B < 1 || B > kPersistentMaxSeqs || V > pd::NWG * pd::LM_ROWS) return false;
    const bool shape = (d == 768 && F == 3072) || (d == 1024 && F == 4096) || (d == 1536 && F == 6144);
    if (!shape) return false;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    return cus >= pd::NWG;
}

template <int D, int F>
static size_t layer_words() {
    return pd::Cfg<D, F>::LAYER_WORDS;
}

size_t persistent_xbuf_bytes(int L, int d, int F, int H, int B, int V) {
    size_t lw = 0;
    if (d == 768) lw = layer_words<768, 3072>();
    else if (d == 1024) lw = layer_words<1024, 4096>();
    else lw = layer_words<1536, 6144>();
    // exchange words + exchange E + the role table
    return 8 * (lw * L + 2 * pd::NWG) + sizeof(pd::Role) * pd::NWG + 256;
}

// The largest T_past the persistent step handles (its attention splits of
// <= MP positions and tail splits of <= MAXPOS positions;
// positions each).
int persistent_max_position(int d, int F) {
    if (d == 768 && F == 3072) return pd::Cfg<768, 3072>::REACH;
    if (d == 1024 && F == 4096) return pd::Cfg<1024, 4096>::REACH;
    if (d == 1536 && F == 6144) return pd::Cfg<1536, 6144>::REACH;
    return 0;
}

size_t persistent_trace_bytes(int L) { return sizeof(uint64_t) * pd::NWG * (L + 1) * pd::TRACE_SLOTS; }

template <int D, int F>
static pd::Role* role_table(void* xbuf, int L) {
    return reinterpret_cast<pd::Role*>(static_cast<uint64_t*>(xbuf) + pd::Cfg<D, F>::LAYER_WORDS * L + 2 * pd::NWG);
}

template <int D, int F>
static hipError_t prepare_t(void* xbuf, int L, hipStream_t st) {
    pd::Role host[pd::NWG];
    if (!pd::build_roles<D, F>(host)) return hipErrorInvalidValue;
    hipError_t e = hipMemcpyAsync(role_table<D, F>(xbuf, L), host, sizeof host, hipMemcpyHostToDevice, st);
    if (e != hipSuccess) return e;
    return hipStreamSynchronize(st);
}

hipError_t persistent_prepare(void* xbuf, int L, int d, int F, hipStream_t st) {
    if (d == 768 && F == 3072) return prepare_t<768, 3072>(xbuf, L, st);
    if (d == 1024 && F == 4096) return prepare_t<1024, 4096>(xbuf, L, st);
    if (d == 1536 && F == 6144) return prepare_t<1536, 6144>(xbuf, L, st);
    return hipErrorInvalidValue;
}

template <int D, int F>
static hipError_t launch_t(const PersistentArgs& p, hipStream_t st) {
    using C = pd::Cfg<D, F>;
    uint64_t* x = static_cast<uint64_t*>(p.xbuf);
    pd::Role* roles = role_table<D, F>(p.xbuf, p.L);
    pd::Args a{};
    a.L = p.L; a.V = p.V; a.t_cap = p.t_cap; a.eps = p.eps;
    a.tok_emb = p.tok_emb; a.lm_head = p.lm_head; a.ln = p.ln; a.ln_final = p.ln_final;
    a.wq = p.wq_base; a.ws = p.ws_base;
    a.wq_layer = (3L * D * D + (long)D * D + 2L * F * D) / 2;
    a.ws_layer = (3L * D * D + (long)D * D + 2L * F * D) / 32;
    a.kc = p.kc; a.vc = p.vc; a.kv_seqs = p.kv_seqs; a.token = p.token; a.logits = p.logits;
    a.next = p.next; a.t0 = p.t0; a.epoch = p.epoch; a.x = x; a.roles = roles; a.err = p.err;
    a.nib = 0x0F0F0F0Fu;
    a.a8 = p.a8;
    a.trace = static_cast<uint64_t*>(p.trace);
    // positions [0, t0): ATT_S splits of `chunk`; past ATT_S * MP, the rest
    // goes to TS tail splits of `tail_chunk`
    int chunk = (p.t0 + C::ATT_S - 1) / C::ATT_S;
    int tail_chunk = 0;
    if (chunk > C::MP) {
        chunk = C::MP;
        tail_chunk = (p.t0 - C::ATT_S * C::MP + C::TS - 1) / C::TS;
        if (tail_chunk > pd::MAXPOS) return hipErrorInvalidValue;
    }
    a.chunk = chunk < 1 ? 1 : chunk;
    a.tail0 = C::ATT_S * a.chunk;
    a.tail_chunk = tail_chunk;
    static bool attr_set = false;
    if (!attr_set) {
        for (const void* k : {(const void*)pd::k_decode_step<D, F, false>, (const void*)pd::k_decode_step<D, F, true>}) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(sizeof(float) * C::LDS_FLOATS));
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    // the tail-capable step only once the cache reaches past the attention
    // splits; the other keeps the registers the tail code would take
    if (tail_chunk > 0)
        pd::k_decode_step<D, F, true><<<dim3(pd::NWG), dim3(pd::NT), sizeof(float) * C::LDS_FLOATS, st>>>(a);
    else
        pd::k_decode_step<D, F, false><<<dim3(pd::NWG), dim3(pd::NT), sizeof(float) * C::LDS_FLOATS, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_persistent_decode(const PersistentArgs& p, hipStream_t st) {
    if (p.B != 1 || p.kv_seqs < 1 || p.kv_seqs > kPersistentMaxSeqs) return hipErrorInvalidValue;
    if (p.d == 768 && p.F == 3072) return launch_t<768, 3072>(p, st);
    if (p.d == 1024 && p.F == 4096) return launch_t<1024, 4096>(p, st);
    if (p.d == 1536 && p.F == 6144) return launch_t<1536, 6144>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace mt
