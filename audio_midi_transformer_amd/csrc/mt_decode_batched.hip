// Single-launch decode step for a batch of 2 .. 8 sequences on MI355X
// (gfx950): one XCD per sequence.
//
// One launch computes one greedy decode step for every sequence of the
// batch: token embedding, per layer the pre-norm attention block
// (LayerNorm, fused QKV projection, attention over the fixed-capacity cache
// with the new K/V row written in place at the sequence's own T_past, O
// projection, residual) and the pre-norm FFN block (LayerNorm, FFN-up +
// GELU, FFN-down, residual), then the final LayerNorm, the FP32 LM head and
// the greedy argmax: the decoder operations of "MuScriptor Medium --
// optimized W4A32 ONNX Runtime" README, "Model variant" (four INT4 group-32
// projections, GroupQueryAttention and two SkipLayerNormalization nodes per
// layer, FP32 cache and activations), one decoder call per step returning
// last-position logits ("unifolia/muscriptor-small-onnx", decoder).
//
// Execution model.  256 workgroups, one per CU; workgroup w runs on XCD
// w % 8 and serves sequence w % 8 (workgroups of sequences past the batch
// leave at once).  The 32 workgroups of a sequence share one L2, so every
// exchange of the step stays inside one XCD: 64-bit words {float value,
// step tag} written by one atomic store each, one copy per vector, gathered
// by re-reading only stale words (the mechanism of the B = 1 step, which
// measured 1.0 us per chained exchange inside an XCD against 1.7 us across
// the chip).  Each XCD reads every layer's weights itself; the copies after
// the first come from the memory-side cache.
//
// Per layer, for the 32 workgroups of one sequence:
//   A  r += f (previous layer); LN1; 3D/32 rows of the fused QKV projection
//      each; q, k, v to the exchange, k and v to the cache slot T_past.
//   T  attention items (head h, split s), H * NS of them, IPW per
//      workgroup: gather q_h, stream the split's cached K/V rows through LDS
//      in rounds of 128 positions (32 per wave, the next round in flight
//      while one is used; each wave keeps its own running max, sum and
//      weighted V sum), combine the four waves (the last split adds the new
//      position from the exchanged k, v) and publish (max, sum, acc[64]).
//   B  gather every partial; merge each head (the weights exp(m_s - M));
//      D/32 O rows each; o to the exchange.
//   C  r += o; LN2; F/32 FFN-up rows + GELU each; u to the exchange.
//   D  gather u; D/32 FFN-down rows each; f to the exchange.
// After the last layer: r += f, LN_f, V/32 LM-head rows each with the local
// argmax; workgroup 0 of the sequence picks the token (lowest index on
// ties).  Each phase's weight rows are requested right after the previous
// phase published its output, so they arrive during the exchange wait.
//
// Every wait is bounded: past the spin limit the workgroup sets bit 2 of the
// error word and leaves; mt_check reports it.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mt_internal.h"
#include "mt_pd_common.h"

namespace mt {
namespace px {

using namespace pd;

constexpr int NW = NWG / NXCD;  // workgroups per sequence: the CUs of one XCD
constexpr int NPASS = 8;        // cached positions per lane group and attention round
constexpr int RNDP = 16 * NPASS; // positions per attention round
constexpr int MAXB = NXCD;      // sequences per launch
constexpr int TRACE_SLOTS = 24;

template <int D, int F>
struct XCfg {
    static constexpr int H = D / 64;
    static constexpr int GD = D / 32, GF = F / 32;
    static constexpr int LPR_D = lpr_for(D), CPL_D = GD / (LPR_D ? LPR_D : 1), RP_D = NT / (LPR_D ? LPR_D : 1);
    static constexpr int LPR_F = lpr_for(F), CPL_F = GF / (LPR_F ? LPR_F : 1), RP_F = NT / (LPR_F ? LPR_F : 1);
    // attention items: NS splits per head, the fewest that spread evenly
    // over the NW workgroups (medium: 2 splits, one item per workgroup;
    // small and large: 8 and 4 splits, three items per workgroup)
    static constexpr int ns_for() {
        int s = 1;
        while ((H * s) % NW != 0) ++s;
        return s;
    }
    static constexpr int NS = ns_for();
    static constexpr int ITEMS = H * NS;
    static constexpr int IPW = ITEMS / NW;
    static constexpr int QKV_ROWS = 3 * D / NW, O_ROWS = D / NW, UP_ROWS = F / NW, DN_ROWS = D / NW;
    static constexpr int NP_QKV = cdiv(QKV_ROWS, RP_D), NP_O = cdiv(O_ROWS, RP_D);
    static constexpr int NP_UP = cdiv(UP_ROWS, RP_D), NP_DN = cdiv(DN_ROWS, RP_F);
    // each phase's rows in NCH chunks held in registers one or two at a
    // time: the whole block where it takes at most 100 registers (small and
    // medium width), else chunks of at most 50 (large: QKV 3, up and down 4)
    static constexpr int nch_for(int np, int cpl) {
        if (np * cpl * 5 <= 100) return 1;
        for (int c = 2; c <= np; ++c)
            if (np % c == 0 && (np / c) * cpl * 5 <= 50) return c;
        return np;
    }
    static constexpr int NCH_QKV = nch_for(NP_QKV, CPL_D), NCH_O = nch_for(NP_O, CPL_D);
    static constexpr int NCH_UP = nch_for(NP_UP, CPL_D), NCH_DN = nch_for(NP_DN, CPL_F);
    static_assert(NCH_QKV <= 4 && NCH_O <= 4 && NCH_UP <= 4 && NCH_DN <= 4, "chunks");
    static constexpr int STG = cmax(cmax(QKV_ROWS, UP_ROWS), cmax(O_ROWS, DN_ROWS));
    // exchange words per layer of one sequence (one copy of each vector)
    static constexpr int XQKV = 0;                   // q | k | v [3D]
    static constexpr int XPART = XQKV + 3 * D;       // partials [ITEMS][PW]
    static constexpr int XO = XPART + ITEMS * PW;    // o [D]
    static constexpr int XU = XO + D;                // u [F]
    static constexpr int XF = XU + F;                // f [D]
    static constexpr int LAYER_WORDS = rup(XF + D, 32);
    // LDS (floats).  Region 0 holds the gathered partials in phase B and u
    // with its group sums in phase D.
    static constexpr int R0 = rup(cmax(ITEMS * PW, F + GF), 4);
    static constexpr int OFF_P = 0;                     // [ITEMS * PW] (phase B)
    static constexpr int OFF_U = 0;                     // [F] (phase D)
    static constexpr int OFF_US = F;                    // [GF] (phase D)
    static constexpr int OFF_ACT = R0;                  // [D] LN output / merged attention (swizzled)
    static constexpr int OFF_XS = OFF_ACT + D;          // [GD] its group sums
    static constexpr int OFF_QH = rup(OFF_XS + GD, 4);  // q_h [64], k_new [64], v_new [64]
    static constexpr int OFF_WP = OFF_QH + 192;         // wave partials [4][PW]
    static constexpr int OFF_STG = rup(OFF_WP + 4 * PW, 4);  // outputs staged for publishing [STG]
    static constexpr int OFF_RED = OFF_STG + rup(STG, 4);    // [16]
    static constexpr int OFF_FLAG = OFF_RED + 16;
    static constexpr int LDS_FLOATS = OFF_FLAG + 4;
    static_assert(D % NT == 0 && F % NT == 0 && D % 64 == 0, "widths");
    static_assert(LPR_D > 0 && LPR_F > 0, "width has no GEMV lane mapping");
    static_assert((3 * D) % NW == 0 && D % NW == 0 && F % NW == 0, "rows per workgroup");
    static_assert(IPW >= 1 && ITEMS == IPW * NW, "attention items");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
    static_assert(H * 64 == D, "heads");
};

struct XArgs {
    int L, V, t_cap, B;
    float eps;
    const float* tok_emb;
    const float* lm_head;
    const float* ln;        // [L][4][D]: LN1 gain, bias, LN2 gain, bias
    const float* ln_final;  // [2][D]
    const uint8_t* wq;      // INT4 nibbles of all layers: QKV [3D, D], O [D, D], up [F, D], down [D, F]
    const float* ws;        // group scales, same order
    long wq_layer;          // bytes per layer
    long ws_layer;          // floats per layer
    float* kc;              // layer 0, sequence 0 of the cache [L][kv_seqs][t_cap][D]
    float* vc;
    int kv_seqs;
    const int64_t* token;   // [B]
    float* logits;          // [B][V]
    int64_t* next;          // [B]
    int t0[MAXB];           // T_past of each sequence
    uint32_t epoch;
    uint64_t* x;            // exchange words: B blocks of seq_words
    long seq_words;
    int* err;
    unsigned nib;           // 0x0F0F0F0F, see dot_u
    int a8;                 // 1: W4A8 projections (INT8 activation codes, INT32 group sums)
    uint64_t* trace;        // optional [NWG][L + 1][TRACE_SLOTS] wall-clock stamps
};

__device__ __forceinline__ void xstamp(const XArgs& a, int l, int k) {
    if (a.trace && threadIdx.x == 0)
        a.trace[((size_t)blockIdx.x * (a.L + 1) + l) * TRACE_SLOTS + k] = wall_clock64();
}

// Byte / float offsets of the four projections inside one layer.
template <int D, int F>
struct XOff {
    static constexpr long QO = 0, OO = 3L * D * D / 2, UO = 4L * D * D / 2, DO = (4L * D * D + (long)F * D) / 2;
    static constexpr long QS = 0, OS = 3L * D * D / 32, US = 4L * D * D / 32, DS = (4L * D * D + (long)F * D) / 32;
};

// Rows row0 .. row0 + NROWS - 1 of an [N, K] INT4 matrix into registers, in
// the lane layout of wblk_load (a group of LPR lanes per row, lane r
// holding groups r, r + LPR, ... of its row).  Buffer loads: the row offset
// of each pass is uniform (a scalar operand) and the lane's offset within
// it one vector register, so no per-pass addresses stay live across the
// layer loop.  Lanes of a pass past NROWS read row row0 (never used).
template <int LPR, int CPL, int NP, int NROWS>
__device__ __forceinline__ void wload(WBlk<CPL, NP>& w, const uint8_t* __restrict__ Wq, const float* __restrict__ Ws,
                                      int K, int row0) {
    constexpr int RP = NT / LPR;
    const int sub = threadIdx.x / LPR, lr = threadIdx.x % LPR;
    const int G = K / 32;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(Wq), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(Ws), 0, 0x7fffffff, 0x00020000);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const bool full = (p + 1) * RP <= NROWS;
        const int rl = full ? sub : (p * RP + sub < NROWS ? sub : -p * RP);  // row within the pass
        const int vq = rl * (K / 2) + lr * 16, vs = (rl * G + lr) * 4;
        const int sq = (row0 + p * RP) * (K / 2), ss = (row0 + p * RP) * G * 4;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rq, vq + j * LPR * 16, sq, 0);
            w.q[p][j] = make_uint4(v.x, v.y, v.z, v.w);
            w.s[p][j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, vs + j * LPR * 4, ss, 0));
        }
    }
}

// One chunk of a phase's rows: request the next chunk (NEXT) into `nxt`,
// then dot the rows in `cur` (rows rbase .. of the phase) and emit each
// output row below nrows.
template <int LPR, int CPL, int NPC, int CR, bool NEXT, typename Emit>
__device__ __forceinline__ void chunk_step(const WBlk<CPL, NPC>& cur, WBlk<CPL, NPC>& nxt, const uint8_t* Wq,
                                           const float* Ws, int K, int row_next, int rbase, int nrows,
                                           const float* act, const float* xs, unsigned nib, bool a8, Emit& emit) {
    if constexpr (NEXT) wload<LPR, CPL, NPC, CR>(nxt, Wq, Ws, K, row_next);
    float o[NPC];
    if (a8) wblk_dot8<LPR, CPL, NPC>(cur, reinterpret_cast<const int8_t*>(act), xs, o);
    else wblk_dot<LPR, CPL, NPC>(cur, act, xs, o, nib);
#pragma unroll
    for (int p = 0; p < NPC; ++p) {
        const int rr = out_row<LPR>(p);
        if (rr >= 0 && rbase + rr < nrows) emit(rbase + rr, o[p]);
    }
}

// The rows row0 .. row0 + NROWS - 1 of one projection against act (group
// sums xs), in NCH chunks of NP / NCH passes: chunk 0 is in w0 (requested
// by the caller), chunk c + 1 is requested before chunk c is used, so at
// most two chunks are in registers.  emit(row, value) for each row.
template <int LPR, int CPL, int NP, int NCH, int NROWS, typename Emit>
__device__ __forceinline__ void rows_dot(WBlk<CPL, NP / NCH>& w0, const uint8_t* Wq, const float* Ws, int K, int row0,
                                         const float* act, const float* xs, unsigned nib, bool a8, Emit emit) {
    constexpr int NPC = NP / NCH, CR = NPC * (NT / LPR);
    static_assert(NP % NCH == 0 && (NCH == 1 || NROWS % CR == 0) && NCH <= 4, "chunks");
    WBlk<CPL, NPC> w1;
    chunk_step<LPR, CPL, NPC, CR, (NCH > 1)>(w0, w1, Wq, Ws, K, row0 + CR, 0, NROWS, act, xs, nib, a8, emit);
    if constexpr (NCH > 1)
        chunk_step<LPR, CPL, NPC, CR, (NCH > 2)>(w1, w0, Wq, Ws, K, row0 + 2 * CR, CR, NROWS, act, xs, nib, a8, emit);
    if constexpr (NCH > 2)
        chunk_step<LPR, CPL, NPC, CR, (NCH > 3)>(w0, w1, Wq, Ws, K, row0 + 3 * CR, 2 * CR, NROWS, act, xs, nib, a8,
                                                 emit);
    if constexpr (NCH > 3)
        chunk_step<LPR, CPL, NPC, CR, false>(w1, w0, Wq, Ws, K, 0, 3 * CR, NROWS, act, xs, nib, a8, emit);
}

// Words i0 .. i0 + nv - 1 of a vector, staged in LDS by the lanes that
// computed them, written by consecutive threads.
__device__ __forceinline__ void publish1(uint64_t* base, int i0, const float* stg, int nv, uint32_t ep) {
    lds_barrier();
    for (int t = threadIdx.x; t < nv; t += NT) ll_put(base + i0 + t, stg[t], ep);
}

// K and V rows of one attention round into registers: lane group g =
// tid / 16 takes positions i0 + g + 16 u (u < NPASS) of the split, lane
// ql = tid % 16 dimensions 4 ql .. 4 ql + 3 of each.  Positions past n read
// the split's first row (never used).  Non-temporal: the step reads each
// cached row once.
template <int D>
__device__ __forceinline__ void round_load(const float* kc_l, const float* vc_l, int h, int p0, int n, int i0,
                                           f32x4_t (&k4)[NPASS], f32x4_t (&v4)[NPASS], int t) {
    const int g = t >> 4, ql = t & 15;
#pragma unroll
    for (int u = 0; u < NPASS; ++u) {
        const int i = i0 + g + 16 * u;
        const size_t off = (size_t)(p0 + (i < n ? i : 0)) * D + h * 64 + ql * 4;
        k4[u] = __builtin_nontemporal_load((const __attribute__((address_space(1))) f32x4_t*)(kc_l + off));
        v4[u] = __builtin_nontemporal_load((const __attribute__((address_space(1))) f32x4_t*)(vc_l + off));
    }
}

// One round into the lane group's running softmax state (m, l uniform over
// the group; acc = its lane's four dimensions of sum_t p_t V_t).
__device__ __forceinline__ void round_step(const f32x4_t (&k4)[NPASS], const f32x4_t (&v4)[NPASS], f32x4_t q4, int i0,
                                           int n, float& m, float& l, f32x4_t& acc, int t) {
    const int g = t >> 4;
    float sc[NPASS];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NPASS; ++u) {
        float d = fmaf(q4.x, k4[u].x, fmaf(q4.y, k4[u].y, fmaf(q4.z, k4[u].z, q4.w * k4[u].w)));
        d = group_reduce<16>(d) * 0.125f;
        sc[u] = i0 + g + 16 * u < n ? d : -INFINITY;
        mx = fmaxf(mx, sc[u]);
    }
    const float mn = fmaxf(m, mx);
    if (mn == -INFINITY) return;  // no valid position for this group yet
    const float al = expf(m - mn);  // 0 while m is still -inf
    float ls = l * al;
    f32x4_t a = acc * al;
#pragma unroll
    for (int u = 0; u < NPASS; ++u) {
        const float pe = sc[u] == -INFINITY ? 0.f : expf(sc[u] - mn);
        ls += pe;
        a.x = fmaf(pe, v4[u].x, a.x);
        a.y = fmaf(pe, v4[u].y, a.y);
        a.z = fmaf(pe, v4[u].z, a.z);
        a.w = fmaf(pe, v4[u].w, a.w);
    }
    m = mn;
    l = ls;
    acc = a;
}

// Softmax partial of q_h over cached positions [p0, p0 + n) of head h,
// streamed through registers in rounds of RNDP positions (round 0 already
// requested into ka / va; two register sets, the next round in flight while
// one is used).  q4 holds this lane's four dimensions of q_h.  Each wave's
// partial (max, sum, acc[64]) lands in wp[wave * PW ..]; the caller
// synchronises before reading them.
template <int D>
__device__ __forceinline__ void split_waves(const float* kc_l, const float* vc_l, int h, int p0, int n, f32x4_t q4,
                                            f32x4_t (&ka)[NPASS], f32x4_t (&va)[NPASS], float* wp_all, int tid) {
    const int lane = tid & 63, wave = tid >> 6;
    const int nr = cdiv(n, RNDP);
    f32x4_t kb[NPASS], vb[NPASS];
    float m = -INFINITY, l = 0.f;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < nr; r += 2) {
        if (r + 1 < nr) round_load<D>(kc_l, vc_l, h, p0, n, (r + 1) * RNDP, kb, vb, tid);
        round_step(ka, va, q4, r * RNDP, n, m, l, acc, tid);
        if (r + 1 < nr) {
            if (r + 2 < nr) round_load<D>(kc_l, vc_l, h, p0, n, (r + 2) * RNDP, ka, va, tid);
            round_step(kb, vb, q4, (r + 1) * RNDP, n, m, l, acc, tid);
        }
    }
    // the four lane groups of each wave (16 lanes apart)
    float M = fmaxf(m, __shfl_xor(m, 16));
    M = fmaxf(M, __shfl_xor(M, 32));
    {
        const float e = m == -INFINITY ? 0.f : expf(m - M);
        l *= e;
        acc = acc * e;
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
            l += __shfl_xor(l, o);
            acc.x += __shfl_xor(acc.x, o);
            acc.y += __shfl_xor(acc.y, o);
            acc.z += __shfl_xor(acc.z, o);
            acc.w += __shfl_xor(acc.w, o);
        }
    }
    float* wp = wp_all + wave * PW;
    if (lane == 0) {
        wp[0] = M;
        wp[1] = l;
    }
    if (lane < 16) {
        wp[2 + 4 * lane] = acc.x;
        wp[3 + 4 * lane] = acc.y;
        wp[4 + 4 * lane] = acc.z;
        wp[5 + 4 * lane] = acc.w;
    }
}

// LDS regions of one workgroup.
template <int D, int F>
struct XLds {
    float *p, *u, *us, *act, *xs, *qh, *knew, *vnew, *wp, *stg, *red;
    int* s_flag;
    __device__ explicit XLds(float* lds) {
        using C = XCfg<D, F>;
        p = lds + C::OFF_P;
        u = lds + C::OFF_U;
        us = lds + C::OFF_US;
        act = lds + C::OFF_ACT;
        xs = lds + C::OFF_XS;
        qh = lds + C::OFF_QH;
        knew = qh + 64;
        vnew = qh + 128;
        wp = lds + C::OFF_WP;
        stg = lds + C::OFF_STG;
        red = lds + C::OFF_RED;
        s_flag = reinterpret_cast<int*>(lds + C::OFF_FLAG);
    }
};

// One attention item of layer l: head h, positions [p0, p0 + n) of the
// sequence's cache (kc_l, vc_l); `with_new` adds the new position from the
// exchanged k and v of this layer.  Publishes (max, sum, acc[64]).
template <int D, int F>
__device__ __forceinline__ bool attention_item(const XArgs& a, const XLds<D, F>& S, uint64_t* X, const float* kc_l,
                                               const float* vc_l, int item, int h, int p0, int n, bool with_new,
                                               f32x4_t (&ka)[NPASS], f32x4_t (&va)[NPASS], bool pre) {
    using C = XCfg<D, F>;
    const uint32_t ep = a.epoch;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ql = tid & 15;
    // the first round is requested before q_h is waited for (pre: already
    // requested by the caller)
    if (n > 0 && !pre) round_load<D>(kc_l, vc_l, h, p0, n, 0, ka, va, tid);
    const Range rq{X + C::XQKV + h * 64, 64, S.qh};
    const Range rk{X + C::XQKV + D + h * 64, with_new ? 64 : 0, S.knew};
    const Range rv{X + C::XQKV + 2 * D + h * 64, with_new ? 64 : 0, S.vnew};
    if (!ll_gather<1, false>(rq, rk, rv, ep, a.err, S.s_flag)) return false;
    split_waves<D>(kc_l, vc_l, h, p0, n, *reinterpret_cast<const f32x4_t*>(S.qh + 4 * ql), ka, va, S.wp, tid);
    lds_barrier();
    if (wave == 0) {
        float mw[5], lw[5];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            mw[w] = S.wp[w * PW];
            lw[w] = S.wp[w * PW + 1];
        }
        mw[4] = -INFINITY;
        lw[4] = 0.f;
        if (with_new) {
            mw[4] = wave_reduce<false>(S.qh[lane] * S.knew[lane]) * 0.125f;
            lw[4] = 1.f;
        }
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 5; ++w) M = fmaxf(M, mw[w]);
        float Ls = 0.f, A = 0.f;
#pragma unroll
        for (int w = 0; w < 5; ++w) {
            const float e = mw[w] == -INFINITY ? 0.f : expf(mw[w] - M);
            Ls = fmaf(e, lw[w], Ls);
            const float aw = w < 4 ? S.wp[w * PW + 2 + lane] : (with_new ? S.vnew[lane] : 0.f);
            A = fmaf(e, aw, A);
        }
        uint64_t* pw = X + C::XPART + (size_t)item * PW;
        ll_put(pw + 2 + lane, A, ep);
        if (lane == 0) {
            ll_put(pw, M, ep);
            ll_put(pw + 1, Ls, ep);
        }
    }
    // the wave partials and q_h are reused by the next item
    lds_barrier();
    return true;
}

// Phase B: every partial -> merged attention (swizzled, group sums) -> O rows.
template <int D, int F, bool A8>
__device__ __forceinline__ bool phase_merge(const XArgs& a, const XLds<D, F>& S, uint64_t* X) {
    using C = XCfg<D, F>;
    if (!ll_gather1<cdiv(C::ITEMS * PW, NT), false>(X + C::XPART, C::ITEMS * PW, S.p, a.epoch, a.err, S.s_flag))
        return false;
    float v[D / NT];
#pragma unroll
    for (int i = 0; i < D / NT; ++i) {
        const int k = threadIdx.x + i * NT;
        const int h = k >> 6, d = k & 63;
        const float* P = S.p + h * C::NS * PW;
        float M = -INFINITY;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) M = fmaxf(M, P[s * PW]);
        float Ls = 0.f, A = 0.f;
#pragma unroll
        for (int s = 0; s < C::NS; ++s) {
            const float ms = P[s * PW];
            const float e = ms == -INFINITY ? 0.f : expf(ms - M);
            Ls = fmaf(e, P[s * PW + 1], Ls);
            A = fmaf(e, P[s * PW + 2 + d], A);
        }
        v[i] = A / Ls;
    }
    if constexpr (A8) {
        // W4A8: codes at cpos(k) and the group scales, the layout the
        // LayerNorm and the gathers give (group maxima to xs, then scales
        // and reciprocals once per group, then the codes)
        lds_barrier();  // the partials are read above; the codes overlay them
        int8_t* a8p = reinterpret_cast<int8_t*>(S.act);
        float* rr = S.act + D / 4;
#pragma unroll
        for (int i = 0; i < D / NT; ++i) {
            const int k = threadIdx.x + i * NT;
            const float am = max32_hi(fabsf(v[i]));
            if ((threadIdx.x & 31) == res_lane(32)) S.xs[k >> 5] = am;
        }
        lds_barrier();
        group_scales(S.xs, rr, D / 32);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < D / NT; ++i) {
            const int k = threadIdx.x + i * NT;
            a8p[cpos(k)] = code8r(v[i], rr[k >> 5]);
        }
    } else {
#pragma unroll
        for (int i = 0; i < D / NT; ++i) {
            const int k = threadIdx.x + i * NT;
            S.act[swz(k)] = v[i];
            const float t = group_reduce<32>(v[i]);
            if ((threadIdx.x & 31) == res_lane(32)) S.xs[k >> 5] = t;
        }
    }
    lds_barrier();
    return true;
}

template <int D, int F, bool A8>
__global__ __launch_bounds__(NT, 1) void k_decode_xcd(XArgs a) {
    using C = XCfg<D, F>;
    using O = XOff<D, F>;
    constexpr int PER = LnRegs<D>::PER;
    extern __shared__ float lds_raw[];
    const XLds<D, F> S(lds_raw);
    const int b = blockIdx.x % NXCD, j = blockIdx.x / NXCD;
    if (b >= a.B) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t ep = a.epoch;
    const int t0 = a.t0[b];
    uint64_t* XS = a.x + (size_t)b * a.seq_words;
    const size_t lstride = (size_t)a.kv_seqs * a.t_cap * D;  // one layer of the cache
    float* kc_b = a.kc + (size_t)b * a.t_cap * D;
    float* vc_b = a.vc + (size_t)b * a.t_cap * D;
    // positions [0, t0) in NS splits of `chunk`; the last split also takes the new one
    const int chunk = t0 > 0 ? cdiv(t0, C::NS) : 1;
    if (tid == 0) *S.s_flag = 0;

    // embedding: this workgroup's copy of the residual stream, element
    // tid + i * NT in r[i]
    float r[PER];
    {
        const int64_t tok = gload(a.token + b);
        const bool bad = tok < 0 || tok >= a.V;
        if (bad && j == 0 && tid == 0) atomicOr(a.err, 1);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int k = tid + i * NT;
            r[i] = bad ? __builtin_nanf("") : gload(a.tok_emb + (size_t)tok * D + k);
        }
        lds_barrier();  // s_flag initialised
    }

    const int qrow = j * C::QKV_ROWS, orow = j * C::O_ROWS, urow = j * C::UP_ROWS, drow = j * C::DN_ROWS;
    // the first chunk of each phase's rows (the whole block at small and
    // medium width)
    constexpr int QC = C::NP_QKV / C::NCH_QKV, OC = C::NP_O / C::NCH_O;
    constexpr int UC = C::NP_UP / C::NCH_UP, DC = C::NP_DN / C::NCH_DN;
    constexpr int QR0 = C::NCH_QKV == 1 ? C::QKV_ROWS : QC * C::RP_D, OR0 = C::NCH_O == 1 ? C::O_ROWS : OC * C::RP_D;
    constexpr int UR0 = C::NCH_UP == 1 ? C::UP_ROWS : UC * C::RP_D, DR0 = C::NCH_DN == 1 ? C::DN_ROWS : DC * C::RP_F;
    WBlk<C::CPL_D, QC> wqkv;
    WBlk<C::CPL_D, OC> wo;
    WBlk<C::CPL_D, UC> wu;
    WBlk<C::CPL_F, DC> wd;
    LnRegs<D> ln1, ln2;
    wload<C::LPR_D, C::CPL_D, QC, QR0>(wqkv, a.wq + O::QO, a.ws + O::QS, D, qrow);
    ln_load<D>(ln1, a.ln, a.ln + D);
    for (int l = 0; l < a.L; ++l) {
        uint64_t* X = XS + (size_t)l * C::LAYER_WORDS;
        const uint8_t* wq = a.wq + l * a.wq_layer;
        const float* ws = a.ws + l * a.ws_layer;
        const float* ln = a.ln + (size_t)l * 4 * D;
        float* kc_l = kc_b + (size_t)l * lstride;
        float* vc_l = vc_b + (size_t)l * lstride;
        const bool last = l + 1 == a.L;
        f32x4_t ka[NPASS], va[NPASS];  // the first attention round of an item
        // ---- A: r += f; LN1; QKV rows -> exchange, k / v -> cache slot t0
        xstamp(a, l, 0);
        {
            float f[PER] = {};
            if (l > 0 && !ll_gather_regs<PER>(XS + (size_t)(l - 1) * C::LAYER_WORDS + C::XF, D, f, ep, a.err))
                *S.s_flag = 1;
            if (!residual_layernorm<D, true>(r, f, l > 0, ln1, a.eps, S.act, S.xs, S.red, S.s_flag, A8)) return;
            xstamp(a, l, 1);
            // the first attention round of the first item is requested
            // here, so it lands during the QKV dot (763 -> 739 us per step
            // at B = 8, T = 520, medium; the O, FFN-up, FFN-down and next
            // QKV weights requested a phase earlier than below were slower,
            // 787 .. 789 us)
            {
                const int h0 = j / C::NS, p00 = (j % C::NS) * chunk;
                const int n0 = max(0, min(t0, p00 + chunk) - p00);
                if (n0 > 0) round_load<D>(kc_l, vc_l, h0, p00, n0, 0, ka, va, tid);
            }
            rows_dot<C::LPR_D, C::CPL_D, C::NP_QKV, C::NCH_QKV, C::QKV_ROWS>(
                wqkv, wq + O::QO, ws + O::QS, D, qrow, S.act, S.xs, a.nib, A8, [&](int rr, float v) { S.stg[rr] = v; });
            lds_barrier();
            for (int t = tid; t < C::QKV_ROWS; t += NT) {
                const int g = qrow + t;
                const float v = S.stg[t];
                ll_put(X + C::XQKV + g, v, ep);
                if (g >= 2 * D) vc_l[(size_t)t0 * D + (g - 2 * D)] = v;
                else if (g >= D) kc_l[(size_t)t0 * D + (g - D)] = v;
            }
        }
        xstamp(a, l, 2);
        // ---- T: attention items
#pragma unroll 1
        for (int it = 0; it < C::IPW; ++it) {
            const int item = j + it * NW;
            const int h = item / C::NS, s = item % C::NS;
            const int p0 = s * chunk;
            const int n = max(0, min(t0, p0 + chunk) - p0);
            if (!attention_item<D, F>(a, S, X, kc_l, vc_l, item, h, p0, n, s == C::NS - 1, ka, va, it == 0))
                return;
        }
        xstamp(a, l, 3);
        // ---- B: merge the heads; O rows -> exchange
        wload<C::LPR_D, C::CPL_D, OC, OR0>(wo, wq + O::OO, ws + O::OS, D, orow);
        if (!phase_merge<D, F, A8>(a, S, X)) return;
        xstamp(a, l, 4);

        {
            rows_dot<C::LPR_D, C::CPL_D, C::NP_O, C::NCH_O, C::O_ROWS>(
                wo, wq + O::OO, ws + O::OS, D, orow, S.act, S.xs, a.nib, A8, [&](int rr, float v) { S.stg[rr] = v; });
            publish1(X + C::XO, orow, S.stg, C::O_ROWS, ep);
        }
        xstamp(a, l, 5);
        // ---- C: r += o; LN2; FFN-up rows + GELU -> exchange
        wload<C::LPR_D, C::CPL_D, UC, UR0>(wu, wq + O::UO, ws + O::US, D, urow);
        ln_load<D>(ln2, ln + 2 * D, ln + 3 * D);
        {
            float oi[PER];
            if (!ll_gather_regs<PER>(X + C::XO, D, oi, ep, a.err)) *S.s_flag = 1;
            xstamp(a, l, 6);
            if (!residual_layernorm<D, true>(r, oi, true, ln2, a.eps, S.act, S.xs, S.red, S.s_flag, A8)) return;
            rows_dot<C::LPR_D, C::CPL_D, C::NP_UP, C::NCH_UP, C::UP_ROWS>(
                wu, wq + O::UO, ws + O::US, D, urow, S.act, S.xs, a.nib, A8,
                [&](int rr, float v) { S.stg[rr] = gelu_erf(v); });
            publish1(X + C::XU, urow, S.stg, C::UP_ROWS, ep);
        }
        xstamp(a, l, 7);
        // ---- D: u -> FFN-down rows -> exchange
        wload<C::LPR_F, C::CPL_F, DC, DR0>(wd, wq + O::DO, ws + O::DS, F, drow);
        if (!gather_to_lds<F / NT>(X + C::XU, F, S.u, S.us, ep, a.err, S.s_flag, A8)) return;
        xstamp(a, l, 8);

        {
            rows_dot<C::LPR_F, C::CPL_F, C::NP_DN, C::NCH_DN, C::DN_ROWS>(
                wd, wq + O::DO, ws + O::DS, F, drow, S.u, S.us, a.nib, A8, [&](int rr, float v) { S.stg[rr] = v; });
            publish1(X + C::XF, drow, S.stg, C::DN_ROWS, ep);
        }
        xstamp(a, l, 9);
        if (!last) {
            wload<C::LPR_D, C::CPL_D, QC, QR0>(wqkv, wq + a.wq_layer + O::QO, ws + a.ws_layer + O::QS, D, qrow);
            ln_load<D>(ln1, ln + 4 * D, ln + 5 * D);
        }
    }

    // ===================== E: r += f; z = LN_f(r); this workgroup's LM-head rows + local argmax
    uint64_t* XE = XS + (size_t)a.L * C::LAYER_WORDS;
    {
        xstamp(a, a.L, 0);
        LnRegs<D> lnf;
        ln_load<D>(lnf, a.ln_final, a.ln_final + D);
        float f[PER];
        if (!ll_gather_regs<PER>(XS + (size_t)(a.L - 1) * C::LAYER_WORDS + C::XF, D, f, ep, a.err)) *S.s_flag = 1;
        if (!residual_layernorm<D, false>(r, f, true, lnf, a.eps, S.act, nullptr, S.red, S.s_flag)) return;
        xstamp(a, a.L, 1);
        const int lmr = cdiv(a.V, NW);
        const int v0 = j * lmr, v1 = min(a.V, v0 + lmr);
        float* logits = a.logits + (size_t)b * a.V;
        float bv = -INFINITY;
        int bi = 0x7fffffff;
        // rows v0 + wave + 4 i, four at a time per wave
        for (int vb = v0 + wave; vb < v1; vb += 16) {
            float4 w4[4][D / 256];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = vb + 4 * u;
#pragma unroll
                for (int c = 0; c < D / 256; ++c)
                    w4[u][c] = v < v1 ? gload(reinterpret_cast<const float4*>(a.lm_head + (size_t)v * D) + lane + 64 * c)
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int v = vb + 4 * u;
                float acc = 0.f;
#pragma unroll
                for (int c = 0; c < D / 256; ++c) {
                    const float4 z = reinterpret_cast<const float4*>(S.act)[lane + 64 * c];
                    acc = fmaf(w4[u][c].x, z.x, fmaf(w4[u][c].y, z.y, fmaf(w4[u][c].z, z.z, fmaf(w4[u][c].w, z.w, acc))));
                }
                acc = wave_reduce<false>(acc);
                if (v < v1) {
                    if (lane == 0) logits[v] = acc;
                    // rows rise within a wave: a tie keeps the earlier (lower) index
                    if (bi == 0x7fffffff || acc > bv) {
                        bv = acc;
                        bi = v;
                    }
                }
            }
        }
        float* cand_v = S.red;                             // [4]
        int* cand_i = reinterpret_cast<int*>(S.red + 4);   // [4]
        if (lane == 0) {
            cand_v[wave] = bv;
            cand_i[wave] = bi;
        }
        lds_barrier();
        if (tid == 0) {
            float best = -INFINITY;
            int besti = 0x7fffffff;
            for (int w = 0; w < 4; ++w) {
                const int ii = cand_i[w];
                if (ii == 0x7fffffff) continue;
                if (besti == 0x7fffffff || cand_v[w] > best || (cand_v[w] == best && ii < besti)) {
                    best = cand_v[w];
                    besti = ii;
                }
            }
            ll_put(XE + 2 * j, best, ep);
            ll_put(XE + 2 * j + 1, __int_as_float(besti), ep);
        }
    }

    // ===================== F: the sequence's argmax (its workgroup 0)
    if (j == 0) {
        float* cv = S.p;
        if (!ll_gather1<1, false>(XE, 2 * NW, cv, ep, a.err, S.s_flag)) return;
        if (tid < 64) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            if (tid < NW) {
                bv = cv[2 * tid];
                bi = __float_as_int(cv[2 * tid + 1]);
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
            if (tid == 0) a.next[b] = bi == 0x7fffffff ? 0 : bi;
        }
        xstamp(a, a.L, 2);
    }
}

}  // namespace px

// ---------------------------------------------------------------- host side

static bool xcd_shape(int d, int F) {
    return (d == 768 && F == 3072) || (d == 1024 && F == 4096) || (d == 1536 && F == 6144);
}

bool batched_supported(int d, int F, int H, int B, int V) {
    if (B < 2 || B > kBatchedMaxSeqs || V < 1 || H * 64 != d || !xcd_shape(d, F)) return false;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    return cus >= pd::NWG;
}

static long seq_words(int L, int d, int F) {
    long lw = 0;
    if (d == 768 && F == 3072) lw = px::XCfg<768, 3072>::LAYER_WORDS;
    else if (d == 1024 && F == 4096) lw = px::XCfg<1024, 4096>::LAYER_WORDS;
    else if (d == 1536 && F == 6144) lw = px::XCfg<1536, 6144>::LAYER_WORDS;
    else return 0;
    return pd::rup((int)(lw * L + 2 * px::NW), 32);
}

size_t batched_xbuf_bytes(int L, int d, int F, int B) { return 8 * (size_t)seq_words(L, d, F) * B + 256; }

template <int D, int F>
static hipError_t launch_xcd_t(const BatchedArgs& p, hipStream_t st) {
    using C = px::XCfg<D, F>;
    px::XArgs a{};
    a.L = p.L; a.V = p.V; a.t_cap = p.t_cap; a.B = p.B; a.eps = p.eps;
    a.tok_emb = p.tok_emb; a.lm_head = p.lm_head; a.ln = p.ln; a.ln_final = p.ln_final;
    a.wq = p.wq_base; a.ws = p.ws_base;
    a.wq_layer = (3L * D * D + (long)D * D + 2L * F * D) / 2;
    a.ws_layer = (3L * D * D + (long)D * D + 2L * F * D) / 32;
    a.kc = p.kc; a.vc = p.vc; a.kv_seqs = p.kv_seqs;
    a.token = p.token; a.logits = p.logits; a.next = p.next;
    for (int b = 0; b < px::MAXB; ++b) a.t0[b] = b < p.B ? p.t0[b] : 0;
    a.epoch = p.epoch;
    a.x = static_cast<uint64_t*>(p.xbuf);
    a.seq_words = seq_words(p.L, D, F);
    a.err = p.err;
    a.nib = 0x0F0F0F0Fu;
    a.a8 = p.a8;
    a.trace = static_cast<uint64_t*>(p.trace);
    static bool attr_set = false;
    if (!attr_set) {
        for (const void* k : {(const void*)px::k_decode_xcd<D, F, false>, (const void*)px::k_decode_xcd<D, F, true>}) {
            hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)(sizeof(float) * C::LDS_FLOATS));
            if (e != hipSuccess) return e;
        }
        attr_set = true;
    }
    if (p.a8)
        px::k_decode_xcd<D, F, true><<<dim3(pd::NWG), dim3(pd::NT), sizeof(float) * C::LDS_FLOATS, st>>>(a);
    else
        px::k_decode_xcd<D, F, false><<<dim3(pd::NWG), dim3(pd::NT), sizeof(float) * C::LDS_FLOATS, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_batched_decode(const BatchedArgs& p, hipStream_t st) {
    if (p.B < 1 || p.B > px::MAXB || p.kv_seqs < p.B || p.L < 1) return hipErrorInvalidValue;
    for (int b = 0; b < p.B; ++b)
        if (p.t0[b] < 0 || p.t0[b] >= p.t_cap) return hipErrorInvalidValue;
    if (p.d == 768 && p.F == 3072) return launch_xcd_t<768, 3072>(p, st);
    if (p.d == 1024 && p.F == 4096) return launch_xcd_t<1024, 4096>(p, st);
    if (p.d == 1536 && p.F == 6144) return launch_xcd_t<1536, 6144>(p, st);
    return hipErrorInvalidValue;
}

}  // namespace mt
