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
//                  otherwise, all on one XCD.  Each recomputes q_h and the
//                  softmax partial over its chunk of cached positions; splits
//                  1.. publish (max, sum, acc[64]); split 0 (the head leader)
//                  merges them with the new position and publishes attn_h.
//   free WGs       the rest: the new K/V rows of the fused projection (to the
//                  cache slot T_past and to the exchange).
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

namespace mt {
namespace pd {

constexpr int NT = 256;      // threads per workgroup
constexpr int NWG = 256;     // workgroups (one per CU)
constexpr int NXCD = 8;      // workgroup w runs on XCD w % 8
constexpr int REP = NXCD;    // copies of each broadcast vector, one per XCD
constexpr int PW = 66;       // words per attention partial: m, l, acc[64]
constexpr int MAXPOS = 256;  // cached positions per attention workgroup (LDS)
constexpr int LM_ROWS = 6;   // vocabulary rows per workgroup
constexpr uint32_t SPIN_LIMIT = 1u << 21;
constexpr int TRACE_SLOTS = 24;

constexpr int lpr_for(int K) {
    const int G = K / 32;
    for (int c = 1; c <= 4; ++c) {
        if (G % c) continue;
        const int l = G / c;
        if (l <= 64 && (l & (l - 1)) == 0) return l;
    }
    return 0;
}
constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
constexpr int rup(int a, int b) { return cdiv(a, b) * b; }
constexpr int cmax(int a, int b) { return a > b ? a : b; }
// lane of an LPR-lane group that holds the group sum after group_reduce
constexpr int res_lane(int lpr) { return lpr == 64 ? 48 : (lpr == 32 ? 16 : 0); }

// Role of one workgroup (host-built table, constant for a model).
struct Role {
    int head;     // attention head, -1 if none
    int split;    // attention split (0 = head leader)
    int kv_row0;  // first row of the 2D K|V rows of the fused projection
    int kv_rows;  // number of K|V rows, 0 if none
    int o_row0;   // first of this workgroup's O-projection rows, -1 if none
    int pad0, pad1, pad2;
};

template <int D, int F>
struct Cfg {
    static constexpr int H = D / 64;
    static constexpr int GD = D / 32, GF = F / 32;
    static constexpr int LPR_D = lpr_for(D), CPL_D = GD / (LPR_D ? LPR_D : 1), RP_D = NT / (LPR_D ? LPR_D : 1);
    static constexpr int LPR_F = lpr_for(F), CPL_F = GF / (LPR_F ? LPR_F : 1), RP_F = NT / (LPR_F ? LPR_F : 1);
    // attention splits per head: 16 where that leaves at least 64 workgroups
    // for the new K/V rows, else 8 (16 splits at medium width measured slower:
    // the q projection is recomputed by twice as many workgroups and the head
    // merge gathers twice as many partials)
    static constexpr int ATT_S = H * 16 + 64 <= NWG ? 16 : 8;
    static constexpr int NATT = H * ATT_S;
    static constexpr int NFREE = NWG - NATT;
    static constexpr int KV_ROWS = cdiv(2 * D, NFREE);
    static constexpr int UP_ROWS = cdiv(F, NWG);
    static constexpr int O_ROWS = cdiv(D, NFREE);  // O rows: free workgroups only
    static constexpr int DN_ROWS = cdiv(D, NWG);
    static constexpr int NP_Q = cdiv(64, RP_D);
    static constexpr int NP_KV = cdiv(KV_ROWS, RP_D);
    static constexpr int NP_O = cdiv(O_ROWS, RP_D);
    static constexpr int NP_UP = cdiv(UP_ROWS, RP_D);
    static constexpr int NP_DN = cdiv(DN_ROWS, RP_F);
    // exchange layout per layer (64-bit words).  Vectors every workgroup
    // reads are written REP times; the workgroups of XCD x read copy x, so
    // no line is polled by more than 32 workgroups.
    static constexpr int XA_KV = 0;                     // new K|V row [2D]
    static constexpr int XA_PART = XA_KV + 2 * D;       // partials [H][ATT_S][PW]
    static constexpr int XB_ATT = XA_PART + NATT * PW;  // merged attention [REP][D]
    static constexpr int XB_O = XB_ATT + REP * D;       // o [REP][D]
    static constexpr int XC = XB_O + REP * D;           // u [REP][F]
    static constexpr int XD = XC + REP * F;             // f [REP][D]
    static constexpr int LAYER_WORDS = rup(XD + REP * D, 2);
    // LDS layout (floats).  The K|V chunk of an attention split stays
    // resident across phases B..D (it is the next layer's chunk by then), so
    // u of phase D shares one region with the vectors of phases A..C.
    static constexpr int BIG = 2 * MAXPOS * 64;           // K|V chunk
    static constexpr int OFF_XS = BIG;                    // group sums of act [GD]
    static constexpr int OFF_US = OFF_XS + GD;            // group sums of u [GF]
    static constexpr int OFF_U = rup(OFF_US + GF, 4);     // u [F] (phase D) or:
    static constexpr int OFF_ACT = OFF_U;                 //   act [D]
    static constexpr int OFF_QH = OFF_ACT + D;            //   q_h [64]
    static constexpr int OFF_SC = OFF_QH + 64;            //   scores [MAXPOS]
    static constexpr int OFF_PART = OFF_SC + MAXPOS;      //   own partial [PW] + gathered [ATT_S-1][PW] + kv_new [128]
    // [4][64] scratch, also the staging of each phase's outputs: outside the
    // u region, because phase D writes it while other waves may still be
    // reading u
    static constexpr int OFF_COMB = rup(cmax(OFF_PART + ATT_S * PW + 128, OFF_U + F), 4);
    static constexpr int OFF_RED = rup(OFF_COMB + 4 * 64, 4);
    static constexpr int OFF_FLAG = OFF_RED + 16;
    static constexpr int LDS_FLOATS = OFF_FLAG + 16;
    static_assert(D % NT == 0 && F % NT == 0 && NT == 256, "widths");
    static_assert(LPR_D > 0 && LPR_F > 0, "width has no GEMV lane mapping");
    static_assert(NFREE >= 64 && KV_ROWS * NFREE >= 2 * D, "K/V rows need workgroups without attention duty");
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "LDS budget");
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

// Loads through the global address space.  The weight pointers come from a
// device-side table; without the cast the compiler emits flat loads, which
// also count against the LDS wait counter.
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
    return *(const __attribute__((address_space(1))) T*)(p);
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload(const uint4* p) {
    const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)(p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 gload(const float4* p) {
    const f32x4_t v = *(const __attribute__((address_space(1))) f32x4_t*)(p);
    return make_float4(v.x, v.y, v.z, v.w);
}

// Workgroup barrier that orders LDS only.  Exchange data goes through
// agent-scope atomics, so no barrier here needs to wait for global memory;
// a full __syncthreads() would also wait for every outstanding global load
// and store (prefetches included) before it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------- cross-lane sums (DPP)

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over groups of W consecutive lanes.  W <= 16: every lane of the group
// holds the sum; W = 32: lanes 16..31 of the group; W = 64: lanes 48..63.
template <int W>
__device__ __forceinline__ float group_reduce(float v) {
    if (W >= 2) v += dpp<0xB1>(v);         // quad_perm [1,0,3,2]
    if (W >= 4) v += dpp<0x4E>(v);         // quad_perm [2,3,0,1]
    if (W >= 8) v += dpp<0x141>(v);        // row_half_mirror
    if (W >= 16) v += dpp<0x140>(v);       // row_mirror
    if (W >= 32) v += dpp<0x142, 0xA>(v);  // row_bcast15 into rows 1, 3
    if (W >= 64) v += dpp<0x143, 0x8>(v);  // row_bcast31 into row 3
    return v;
}

template <bool MAX>
__device__ __forceinline__ float row_reduce16(float v) {
    if (MAX) {
        v = fmaxf(v, dpp<0xB1>(v));
        v = fmaxf(v, dpp<0x4E>(v));
        v = fmaxf(v, dpp<0x141>(v));
        v = fmaxf(v, dpp<0x140>(v));
    } else {
        v = group_reduce<16>(v);
    }
    return v;
}

// Whole-wave sum / max, returned in every lane.
template <bool MAX>
__device__ __forceinline__ float wave_reduce(float v) {
    v = row_reduce16<MAX>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return MAX ? fmaxf(fmaxf(a, b), fmaxf(c, d)) : (a + b) + (c + d);
}

// Whole-workgroup sum / max; `red` holds 4 floats owned by this call site.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
    v = wave_reduce<MAX>(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    lds_barrier();
    return MAX ? fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])) : (red[0] + red[1]) + (red[2] + red[3]);
}

// ---------------------------------------------------------------- W4A8 codes

// Maximum over each group of 32 consecutive lanes, valid in lanes 16..31 of
// the group (the layout of group_reduce<32>).
__device__ __forceinline__ float max32_hi(float v) {
    v = fmaxf(v, dpp<0xB1>(v));        // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));        // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));       // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));       // row_mirror: the 16-lane row
    return fmaxf(v, dpp<0x142, 0xA>(v));  // row_bcast15 into rows 1, 3
}

// Group scales from group maxima: thread g turns xs[g] (max |x| of group g)
// into s = max / 127 (kept in xs) and its reciprocal rr[g]; ng groups.
__device__ __forceinline__ void group_scales(float* xs, float* rr, int ng) {
    for (int g = threadIdx.x; g < ng; g += NT) {
        const float sc = xs[g] / 127.0f;
        xs[g] = sc;
        rr[g] = sc != 0.f ? 1.0f / sc : 0.f;
    }
}

// The INT8 code of x with reciprocal scale r.
__device__ __forceinline__ int8_t code8r(float x, float r) {
    return (int8_t)(int)fminf(fmaxf(rintf(__fmul_rn(x, r)), -127.f), 127.f);
}

// Byte position of input k in the W4A8 code layout: in each block of 8
// inputs the even ones first, then the odd ones, the order in which the
// low and high nibbles of a weight dword come apart.
__device__ __forceinline__ int cpos(int k) {
    const int j = k & 7;
    return (k & ~7) | ((j & 1) << 2) | (j >> 1);
}


// ---------------------------------------------------------------- exchange words

__device__ __forceinline__ void ll_put(uint64_t* p, float v, uint32_t ep) {
    __hip_atomic_store(p, ((uint64_t)ep << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ll_get(const uint64_t* p) {
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ bool aborted(int* err) {
    return (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) & 2) != 0;
}

// Position of element k of a vector in the swizzled LDS layout: the eight
// 16-byte sub-blocks of each 32-element group are rotated by the group index
// so that lanes reading different groups hit different banks.
__device__ __forceinline__ int swz(int k) {
    const int c = k >> 5, j = (k >> 2) & 7;
    return (c << 5) + (((j + c) & 7) << 2) + (k & 3);
}

struct Range {
    const uint64_t* src;
    int n;
    float* dst;
};

// Wait for up to three ranges of exchange words (n0 + n1 + n2 <= NT * U) and
// store their values to LDS (range 0 optionally swizzled).  All first reads
// are issued together; re-reads of stale words too.
template <int U, bool SWZ0>
__device__ bool ll_gather_single(Range r0, Range r1, Range r2, uint32_t ep, int* err, int* s_flag) {
    const int n01 = r0.n + r1.n, n = n01 + r2.n;
    auto src = [&](int i) -> const uint64_t* {
        return i < r0.n ? r0.src + i : (i < n01 ? r1.src + (i - r0.n) : r2.src + (i - n01));
    };
    uint64_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = u * NT + threadIdx.x;
        w[u] = (i < n) ? ll_get(src(i)) : ((uint64_t)ep << 32);
    }
    bool ok = true;
    for (uint32_t it = 0;; ++it) {
        bool all = true;
#pragma unroll
        for (int u = 0; u < U; ++u) all &= (uint32_t)(w[u] >> 32) == ep;
        if (all) break;
        if (it > SPIN_LIMIT || ((it & 255u) == 255u && aborted(err))) {
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((uint32_t)(w[u] >> 32) != ep) w[u] = ll_get(src(u * NT + threadIdx.x));
    }
    // the destination may still be read by other waves of the previous phase
    lds_barrier();
    if (ok) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = u * NT + threadIdx.x;
            const float v = __uint_as_float((uint32_t)w[u]);
            if (i < r0.n) r0.dst[SWZ0 ? swz(i) : i] = v;
            else if (i < n01) r1.dst[i - r0.n] = v;
            else if (i < n) r2.dst[i - n01] = v;
        }
    } else {
        atomicOr(err, 2);
        *s_flag = 1;
    }
    lds_barrier();
    return *s_flag == 0;
}

template <int U, bool SWZ0>
__device__ __forceinline__ bool ll_gather(Range r0, Range r1, Range r2, uint32_t ep, int* err, int* s_flag) {
    return ll_gather_single<U, SWZ0>(r0, r1, r2, ep, err, s_flag);
}

// Word i of all REP copies of a broadcast vector of n words.
__device__ __forceinline__ void ll_put_rep(uint64_t* base, int n, int i, float v, uint32_t ep) {
#pragma unroll
    for (int r = 0; r < REP; ++r) ll_put(base + (size_t)r * n + i, v, ep);
}

// Publish nv consecutive words i0 .. i0 + nv - 1 of a broadcast vector of n
// words to all REP copies.  The values were staged in LDS (stg) by the lanes
// that computed them; thread t then writes word t % nv of copy t / nv, so
// each copy goes out as contiguous stores of one wave instead of scattered
// single words.
__device__ __forceinline__ void publish_rep(uint64_t* base, int n, int i0, const float* stg, int nv, uint32_t ep) {
    lds_barrier();
    for (int t = threadIdx.x; t < nv * REP; t += NT) ll_put(base + (size_t)(t / nv) * n + i0 + t % nv, stg[t % nv], ep);
}

// The copy of a broadcast vector this workgroup reads (its XCD's).
__device__ __forceinline__ const uint64_t* rep_of(const uint64_t* base, int n) {
    return base + (size_t)(blockIdx.x % REP) * n;
}

template <int U, bool SWZ>
__device__ __forceinline__ bool ll_gather1(const uint64_t* src, int n, float* dst, uint32_t ep, int* err,
                                           int* s_flag) {
    return ll_gather<U, SWZ>(Range{src, n, dst}, Range{src, 0, dst}, Range{src, 0, dst}, ep, err, s_flag);
}

// Wait for words t + i * NT (i < U) of an n-word vector and return their
// values in registers (thread t), the element mapping of the LayerNorm.  On
// a failed wait the error bit is set and false returned; the caller flags
// the workgroup.
struct StrideIdx {  // word u of thread t: t + u * NT
    __device__ int operator()(int u) const { return u * NT + (int)threadIdx.x; }
};

template <int U, typename Idx = StrideIdx>
__device__ __forceinline__ bool ll_gather_regs(const uint64_t* src, int n, float (&v)[U], uint32_t ep, int* err,
                                               Idx idx = Idx()) {
    uint64_t w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int i = idx(u);
        w[u] = (i < n) ? ll_get(src + i) : ((uint64_t)ep << 32);
    }
    bool ok = true;
    for (uint32_t it = 0;; ++it) {
        bool all = true;
#pragma unroll
        for (int u = 0; u < U; ++u) all &= (uint32_t)(w[u] >> 32) == ep;
        if (all) break;
        if (it > SPIN_LIMIT || ((it & 255u) == 255u && aborted(err))) {
            ok = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((uint32_t)(w[u] >> 32) != ep) w[u] = ll_get(src + idx(u));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __uint_as_float((uint32_t)w[u]);
    if (!ok) atomicOr(err, 2);
    return ok;
}

// Word order of a vector gathered as W4A8 codes: dword q = rho * NT + t of the
// code layout (thread t, rho < U / 4) holds the codes of inputs 8 (q / 2) +
// (q % 2) + 2 j, j < 4 (the even or the odd inputs of one block of 8), so a
// thread's four values make one code dword and the 32 inputs of a group are
// eight consecutive lanes.
struct CodeIdx {
    __device__ int operator()(int u) const {
        const int q = (u >> 2) * NT + (int)threadIdx.x;
        return 8 * (q >> 1) + (q & 1) + 2 * (u & 3);
    }
};

// ---------------------------------------------------------------- LayerNorm

// Wait for an n-word vector (n a multiple of NT), store it swizzled to LDS
// (dst) with the sums of its 32-element groups (xs).  Thread t holds words
// t + i NT, so each group lies in 32 consecutive lanes and its sum is a lane
// reduction.  False (for the whole workgroup) if a wait failed.
// With a8 the vector is stored as W4A8 codes (bytes at cpos(i) of dst) and
// xs receives the group scales instead.
template <int U>
__device__ __forceinline__ bool gather_to_lds(const uint64_t* src, int n, float* dst, float* xs, uint32_t ep,
                                              int* err, int* s_flag, bool a8) {
    float v[U];
    if (a8 && U % 4 == 0) {
        // codes: one dword per four gathered values (CodeIdx order); group
        // maxima over eight lanes by DPP, scales and reciprocals (after the
        // n code bytes) once per group
        if (!ll_gather_regs<U>(src, n, v, ep, err, CodeIdx())) *s_flag = 1;
        lds_barrier();  // dst and xs may still be read by other waves of the previous phase
        unsigned* d32 = reinterpret_cast<unsigned*>(dst);
        float* rr = dst + n / 4;
#pragma unroll
        for (int rho = 0; rho < U / 4; ++rho) {
            float am = fmaxf(fmaxf(fabsf(v[4 * rho]), fabsf(v[4 * rho + 1])),
                             fmaxf(fabsf(v[4 * rho + 2]), fabsf(v[4 * rho + 3])));
            am = fmaxf(am, dpp<0xB1>(am));   // quad_perm [1,0,3,2]
            am = fmaxf(am, dpp<0x4E>(am));   // quad_perm [2,3,0,1]
            am = fmaxf(am, dpp<0x141>(am));  // row_half_mirror: the 8 lanes
            const int q = rho * NT + threadIdx.x;
            if ((threadIdx.x & 7) == 0) xs[q >> 3] = am;
        }
        lds_barrier();
        group_scales(xs, rr, n / 32);
        lds_barrier();
#pragma unroll
        for (int rho = 0; rho < U / 4; ++rho) {
            const int q = rho * NT + threadIdx.x;
            const float r = rr[q >> 3];
            unsigned wd = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) wd |= ((unsigned)(uint8_t)code8r(v[4 * rho + j], r)) << (8 * j);
            d32[q] = wd;
        }
        lds_barrier();
        return *s_flag == 0;
    }
    if (!ll_gather_regs<U>(src, n, v, ep, err)) *s_flag = 1;
    lds_barrier();  // dst and xs may still be read by other waves of the previous phase
    if (a8) {
        // codes byte by byte (vectors whose length is not a multiple of 4 NT):
        // group maxima to xs, scales and reciprocals once per group
        int8_t* d8 = reinterpret_cast<int8_t*>(dst);
        float* rr = dst + n / 4;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float am = max32_hi(fabsf(v[u]));
            if ((threadIdx.x & 31) == res_lane(32)) xs[(u * NT + threadIdx.x) >> 5] = am;
        }
        lds_barrier();
        group_scales(xs, rr, n / 32);
        lds_barrier();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = u * NT + threadIdx.x;
            d8[cpos(i)] = code8r(v[u], rr[i >> 5]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = u * NT + threadIdx.x;
            dst[swz(i)] = v[u];
            const float t = group_reduce<32>(v[u]);
            if ((threadIdx.x & 31) == res_lane(32)) xs[i >> 5] = t;
        }
    }
    lds_barrier();
    return *s_flag == 0;
}

// LayerNorm gain and bias held in registers (element k = threadIdx.x + i*NT).
template <int D>
struct LnRegs {
    static constexpr int PER = (D + NT - 1) / NT;
    float g[PER], b[PER];
};

template <int D>
__device__ __forceinline__ void ln_load(LnRegs<D>& p, const float* __restrict__ g, const float* __restrict__ b) {
#pragma unroll
    for (int i = 0; i < LnRegs<D>::PER; ++i) {
        const int k = threadIdx.x + i * NT;
        p.g[i] = k < D ? gload(g + k) : 0.f;
        p.b[i] = k < D ? gload(b + k) : 0.f;
    }
}

// r += delta (if add); y = LN(r) * g + b into act (swizzled when SWZ),
// plus the group sums of y into xs (if given).  Biased variance, two
// passes.  Thread t holds elements t + i * NT of r and delta in registers;
// with this mapping the 32 elements of a group sit in 32 consecutive lanes,
// so group sums are lane reductions.  Returns false (for every thread) if
// a thread of the workgroup flagged a failed exchange before the call.
template <int D, bool SWZ>
__device__ __forceinline__ bool residual_layernorm(float (&r)[LnRegs<D>::PER], const float (&delta)[LnRegs<D>::PER],
                                                   bool add, const LnRegs<D>& p, float eps, float* act, float* xs, float* red,
                                                   const int* s_flag, bool a8 = false) {
    constexpr int PER = LnRegs<D>::PER;
    // mean and sum of squared deviations of each wave's 64 PER elements
    // (two passes within the wave), then combined across the four waves:
    // M2 = sum_w M2_w + n_w sum_w (mean_w - mean)^2 (exact combination).
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        if (add) r[i] += delta[i];
        s += r[i];
    }
    constexpr float NW = 64.f * PER;
    const float mw = wave_reduce<false>(s) / NW;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float c = r[i] - mw;
        q = fmaf(c, c, q);
    }
    q = wave_reduce<false>(q);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[2 * wave] = mw;
        red[2 * wave + 1] = q;
    }
    lds_barrier();
    if (*s_flag) return false;
    const float mean = ((red[0] + red[2]) + (red[4] + red[6])) * 0.25f;
    const float d0 = red[0] - mean, d1 = red[2] - mean, d2 = red[4] - mean, d3 = red[6] - mean;
    const float m2 = ((red[1] + red[3]) + (red[5] + red[7])) +
                     NW * ((d0 * d0 + d1 * d1) + (d2 * d2 + d3 * d3));
    const float var = m2 / (float)D;
    const float rstd = 1.0f / sqrtf(var + eps);
    if (a8 && xs) {
        // W4A8: codes and group scales of y (D is a multiple of NT); group
        // maxima to xs, scales and reciprocals (after the D code bytes) once
        // per group, then the codes
        int8_t* a8p = reinterpret_cast<int8_t*>(act);
        float* rr = act + D / 4;
        float y[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int k = threadIdx.x + i * NT;
            y[i] = (r[i] - mean) * rstd * p.g[i] + p.b[i];
            const float am = max32_hi(fabsf(y[i]));
            if ((threadIdx.x & 31) == res_lane(32)) xs[k >> 5] = am;
        }
        lds_barrier();
        group_scales(xs, rr, D / 32);
        lds_barrier();
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int k = threadIdx.x + i * NT;
            a8p[cpos(k)] = code8r(y[i], rr[k >> 5]);
        }
        lds_barrier();
        return true;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int k = threadIdx.x + i * NT;
        const float y = k < D ? (r[i] - mean) * rstd * p.g[i] + p.b[i] : 0.f;
        if (k < D) act[SWZ ? swz(k) : k] = y;
        if (xs) {
            const float t = group_reduce<32>(y);
            if ((threadIdx.x & 31) == res_lane(32) && k < D) xs[k >> 5] = t;
        }
    }
    lds_barrier();
    return true;
}

// ---------------------------------------------------------------- INT4 rows held in registers

template <int CPL, int NP>
struct WBlk {
    uint4 q[NP][CPL];
    float s[NP][CPL];
};

// Rows row0 .. row0+nrows-1 of an [N, K] INT4 matrix; a lane group of LPR
// lanes per row, lane r holding groups r, r + LPR, ... of its row.
template <int LPR, int CPL, int NP>
__device__ __forceinline__ void wblk_load(WBlk<CPL, NP>& w, const uint8_t* __restrict__ Wq,
                                          const float* __restrict__ Ws, int K, int row0, int nrows) {
    constexpr int RP = NT / LPR;
    const int sub = threadIdx.x / LPR, lr = threadIdx.x % LPR;
    const int G = K / 32;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int r = p * RP + sub;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lr + LPR * j;
            if (r < nrows) {
                const size_t row = (size_t)(row0 + r);
                w.q[p][j] = gload(reinterpret_cast<const uint4*>(Wq + row * (K / 2) + (size_t)c * 16));
                w.s[p][j] = gload(Ws + row * G + c);
            } else {
                w.q[p][j] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
                w.s[p][j] = 0.f;
            }
        }
    }
}

// Activation group c (32 floats) from the swizzled LDS vector, in input order.
__device__ __forceinline__ void load_group(const float* act, int c, float (&x)[32]) {
    const float* base = act + (c << 5);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float4 v = *reinterpret_cast<const float4*>(base + (((j + c) & 7) << 2));
        x[4 * j + 0] = v.x;
        x[4 * j + 1] = v.y;
        x[4 * j + 2] = v.z;
        x[4 * j + 3] = v.w;
    }
}

// Unsigned byte N of x as float: one v_cvt_f32_ubyte<N> per weight.
template <int N>
__device__ __forceinline__ float ubyte(unsigned x) {
    return (float)(uint8_t)(x >> (8 * N));
}

// sum_k u_k x_k over one group.  Byte j of the group holds input 2j (low
// nibble) and 2j+1 (high nibble).  `m` is 0x0F0F0F0F, passed in at run time:
// with a literal mask the compiler knows the upper bits of each byte are
// zero and extracts every nibble with a bit-field instruction before the
// conversion instead of converting bytes directly.
__device__ __forceinline__ float dot_u(uint4 w, const float (&x)[32], unsigned m) {
    const unsigned wd[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned lo = wd[k] & m;
        const unsigned hi = (wd[k] >> 4) & m;
        const float* xm = x + 8 * k;
        acc = fmaf(ubyte<0>(lo), xm[0], acc);
        acc = fmaf(ubyte<0>(hi), xm[1], acc);
        acc = fmaf(ubyte<1>(lo), xm[2], acc);
        acc = fmaf(ubyte<1>(hi), xm[3], acc);
        acc = fmaf(ubyte<2>(lo), xm[4], acc);
        acc = fmaf(ubyte<2>(hi), xm[5], acc);
        acc = fmaf(ubyte<3>(lo), xm[6], acc);
        acc = fmaf(ubyte<3>(hi), xm[7], acc);
    }
    return acc;
}

// out[p] = row . a, valid in lane res_lane(LPR) of each row group.  The
// stored nibble is code + 8, so row . a = s * (sum u a - 8 sum a) per group.
// A lane holds the same groups for all of its rows, so each activation group
// is read from LDS once and used for every row.
template <int LPR, int CPL, int NP>
__device__ __forceinline__ void wblk_dot(const WBlk<CPL, NP>& w, const float* act, const float* xs,
                                         float (&out)[NP], unsigned m) {
    const int lr = threadIdx.x % LPR;
    float acc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[p] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        float x[32];
        load_group(act, c, x);
        const float x8 = -8.f * xs[c];
#pragma unroll
        for (int p = 0; p < NP; ++p) acc[p] = fmaf(w.s[p][j], dot_u(w.q[p][j], x, m) + x8, acc[p]);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) out[p] = group_reduce<LPR>(acc[p]);
}

// W4A8 form of wblk_dot: per group the exact INT32 sum of code * 16 (u - 8)
// with v_dot4 (nibbles sign-flipped by xor 8, even inputs from the low and
// odd inputs from the high nibbles, against the codes stored in that order),
// then out += I * s_a * s_w / 16.  `sa` holds the group scales of the codes.
template <int LPR, int CPL, int NP>
__device__ __forceinline__ void wblk_dot8(const WBlk<CPL, NP>& w, const int8_t* act8, const float* sa,
                                          float (&out)[NP]) {
    const int lr = threadIdx.x % LPR;
    float acc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[p] = 0.f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lr + LPR * j;
        const uint4 a0 = *reinterpret_cast<const uint4*>(act8 + c * 32);
        const uint4 a1 = *reinterpret_cast<const uint4*>(act8 + c * 32 + 16);
        const unsigned av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float s16 = sa[c] * 0.0625f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const unsigned wd[4] = {w.q[p][j].x, w.q[p][j].y, w.q[p][j].z, w.q[p][j].w};
            int I = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const unsigned x8 = wd[i] ^ 0x88888888u;
                I = __builtin_amdgcn_sdot4((int)((x8 << 4) & 0xF0F0F0F0u), (int)av[2 * i], I, false);
                I = __builtin_amdgcn_sdot4((int)(x8 & 0xF0F0F0F0u), (int)av[2 * i + 1], I, false);
            }
            acc[p] = fmaf((float)I, s16 * w.s[p][j], acc[p]);
        }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) out[p] = group_reduce<LPR>(acc[p]);
}

// The rows' dot products in the arithmetic the step runs (W4A32 or W4A8).
template <int LPR, int CPL, int NP>
__device__ __forceinline__ void dot_rows(const WBlk<CPL, NP>& w, const float* act, const float* xs, float (&out)[NP],
                                         const Args& a) {
    if (a.a8) wblk_dot8<LPR, CPL, NP>(w, reinterpret_cast<const int8_t*>(act), xs, out);
    else wblk_dot<LPR, CPL, NP>(w, act, xs, out, a.nib);
}

// Row handled by this lane in pass p, or -1 if this lane does not write.
template <int LPR>
__device__ __forceinline__ int out_row(int p) {
    constexpr int RP = NT / LPR;
    return (threadIdx.x % LPR) == res_lane(LPR) ? p * RP + threadIdx.x / LPR : -1;
}

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// K/V rows of one head at positions [p0, p0 + npos) of one layer's cache,
// DMA'd into LDS: K at big[0 ..), V at big[MAXPOS * 64 ..), 64 floats each.
template <int D>
__device__ __forceinline__ void kv_chunk_dma(const float* kc_l, const float* vc_l, int head, int p0,
                                             int npos, float* big) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rounds = (npos + 15) / 16;
    for (int rd = 0; rd < rounds; ++rd) {
        const int pl = rd * 16 + wave * 4;
        int pos = p0 + pl + (lane >> 4);
        if (pos >= p0 + npos) pos = p0;  // in-range address; the slot is never read
        const size_t off = (size_t)pos * D + head * 64 + (lane & 15) * 4;
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(kc_l + off),
                                         (__attribute__((address_space(3))) void*)(big + pl * 64), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(vc_l + off),
                                         (__attribute__((address_space(3))) void*)(big + MAXPOS * 64 + pl * 64),
                                         16, 0, 0);
    }
}

// Softmax partial of q over the npos cached positions in LDS: one lane per
// position for the scores (rotated 16-byte reads, four in flight, no
// cross-lane reduction), then lanes = dimensions for sum_t p_t V_t.  Writes
// (max, sum, acc[64]) to part[0], part[1], part[2 ..].
__device__ __forceinline__ void attend_chunk(const float* big, const float* qh, int npos, float* sc,
                                             float* comb, float* red, float* part, const Args& a, int l) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float s = -INFINITY;
    if (tid < npos) {
        const float* kr = big + tid * 64;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int c0 = 0; c0 < 16; c0 += 4) {
            float4 k4[4], q4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int cc = (c0 + c + tid) & 15;
                k4[c] = *reinterpret_cast<const float4*>(kr + cc * 4);
                q4[c] = *reinterpret_cast<const float4*>(qh + cc * 4);
            }
#pragma unroll
            for (int c = 0; c < 4; c += 2) {
                acc0 = fmaf(q4[c].x, k4[c].x, fmaf(q4[c].y, k4[c].y, fmaf(q4[c].z, k4[c].z, fmaf(q4[c].w, k4[c].w, acc0))));
                acc1 = fmaf(q4[c + 1].x, k4[c + 1].x,
                            fmaf(q4[c + 1].y, k4[c + 1].y, fmaf(q4[c + 1].z, k4[c + 1].z, fmaf(q4[c + 1].w, k4[c + 1].w, acc1))));
            }
        }
        s = (acc0 + acc1) * 0.125f;
    }
    stamp(a, l, 12);
    const float M = block_reduce<true>(s, red);
    const float pe = (tid < npos) ? expf(s - M) : 0.f;
    if (tid < MAXPOS) sc[tid] = pe;
    const float Ls = block_reduce<false>(pe, red + 4);
    stamp(a, l, 13);
    // sum_t p_t V_t: lane (wave w, row r, c) takes dims 4c..4c+3 of positions
    // 4w + r + 16i; the 4 rows of a wave are summed lane-wise, then the 4
    // waves through LDS.
    const float* vbase = big + MAXPOS * 64;
    const int row = lane >> 4, c4 = lane & 15;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    int t = 4 * wave + row;
    for (; t + 16 < npos; t += 32) {
        const float p0 = sc[t], p1 = sc[t + 16];
        const float4 v0 = *reinterpret_cast<const float4*>(vbase + t * 64 + c4 * 4);
        const float4 v1 = *reinterpret_cast<const float4*>(vbase + (t + 16) * 64 + c4 * 4);
        a0.x = fmaf(p0, v0.x, a0.x); a0.y = fmaf(p0, v0.y, a0.y); a0.z = fmaf(p0, v0.z, a0.z); a0.w = fmaf(p0, v0.w, a0.w);
        a1.x = fmaf(p1, v1.x, a1.x); a1.y = fmaf(p1, v1.y, a1.y); a1.z = fmaf(p1, v1.z, a1.z); a1.w = fmaf(p1, v1.w, a1.w);
    }
    for (; t < npos; t += 16) {
        const float p0 = sc[t];
        const float4 v0 = *reinterpret_cast<const float4*>(vbase + t * 64 + c4 * 4);
        a0.x = fmaf(p0, v0.x, a0.x); a0.y = fmaf(p0, v0.y, a0.y); a0.z = fmaf(p0, v0.z, a0.z); a0.w = fmaf(p0, v0.w, a0.w);
    }
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
        gpart = own + PW;                   // splits 1 .. ATT_S-1 [ATT_S-1][PW]
        knew = gpart + (C::ATT_S - 1) * PW; // [64]
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

// Loads of the FFN-down rows (issued after phase B).
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

// Every layer for an attention workgroup (head h, split s).
template <int D, int F>
__device__ __forceinline__ bool attention_role(const Args& a, const Lds<D, F>& S, const Role& role,
                                               float (&r)[LnRegs<D>::PER]) {
    using C = Cfg<D, F>;
    using O = Off<D, F>;
    const uint32_t ep = a.epoch;
    const int tid = threadIdx.x;
    constexpr int AS = C::ATT_S;
    const bool leader = role.split == 0;
    const int h = role.head;
    const int p0 = role.split * a.chunk;
    const int npos = max(0, min(a.t0, p0 + a.chunk) - p0);
    const size_t lstride = (size_t)a.kv_seqs * a.t_cap * D;  // one layer of the cache
    WBlk<C::CPL_D, C::NP_Q> wqh;
    BcdW<D, F> w;
    LnRegs<D> ln1;
    if (npos > 0) kv_chunk_dma<D>(a.kc, a.vc, h, p0, npos, S.big);
    wblk_load<C::LPR_D, C::CPL_D, C::NP_Q>(wqh, a.wq + O::QO, a.ws + O::QS, D, h * 64, 64);
    ln_load<D>(ln1, a.ln, a.ln + D);
    for (int l = 0; l < a.L; ++l) {
        uint64_t* X = a.x + (size_t)l * C::LAYER_WORDS;
        const uint8_t* wq = a.wq + l * a.wq_layer;
        const float* ws = a.ws + l * a.ws_layer;
        const float* ln = a.ln + (size_t)l * 4 * D;
        const float* kc_l = a.kc + (size_t)l * lstride;
        const float* vc_l = a.vc + (size_t)l * lstride;
        const bool last = l + 1 == a.L;
        // ---- A: r += f_prev; LN1; q_h; softmax partial over the chunk
        if (!phase_a_ln<D, F>(a, S, ln1, r, l)) return false;
        {
            float o[C::NP_Q];
            dot_rows<C::LPR_D, C::CPL_D, C::NP_Q>(wqh, S.act, S.xs, o, a);
#pragma unroll
            for (int p = 0; p < C::NP_Q; ++p) {
                const int rr = out_row<C::LPR_D>(p);
                if (rr >= 0 && rr < 64) S.qh[rr] = o[p];
            }
        }
        stamp(a, l, 15);
        __builtin_amdgcn_s_waitcnt(0);  // the K/V chunk DMA (and every earlier load) has landed
        lds_barrier();
        stamp(a, l, 3);
        // phase B and C weights load behind the attention
        load_bc<D, F>(w, wq, ws, ln, -1);
        attend_chunk(S.big, S.qh, npos, S.sc, S.comb, S.red + 8, S.own, a, l);
        stamp(a, l, 4);
        if (!leader) {
            uint64_t* pw = X + C::XA_PART + (size_t)(h * AS + role.split) * PW;
            if (tid < PW) ll_put(pw + tid, S.own[tid], ep);
            // the next layer's chunk: this workgroup's next exchange read
            // (phase C) is microseconds away
            if (!last && npos > 0) kv_chunk_dma<D>(kc_l + lstride, vc_l + lstride, h, p0, npos, S.big);
        } else {
            // ---- A2: merge the splits and the new position -> attn_h
            if (!ll_gather<cdiv((AS - 1) * PW + 128, NT), false>(
                    Range{X + C::XA_PART + (size_t)(h * AS + 1) * PW, (AS - 1) * PW, S.gpart},
                    Range{X + C::XA_KV + h * 64, 64, S.knew}, Range{X + C::XA_KV + D + h * 64, 64, S.vnew}, ep,
                    a.err, S.s_flag))
                return false;
            stamp(a, l, 5);
            if (tid < 64) {
                const float snew = wave_reduce<false>(S.qh[tid] * S.knew[tid]) * 0.125f;
                float M = fmaxf(snew, S.own[0]);
                for (int s = 0; s < AS - 1; ++s) M = fmaxf(M, S.gpart[s * PW]);
                float Ls = expf(snew - M);
                float A = Ls * S.vnew[tid];
                if (S.own[0] != -INFINITY) {
                    const float wgt = expf(S.own[0] - M);
                    Ls = fmaf(wgt, S.own[1], Ls);
                    A = fmaf(wgt, S.own[2 + tid], A);
                }
                for (int s = 0; s < AS - 1; ++s) {
                    const float ms = S.gpart[s * PW];
                    if (ms == -INFINITY) continue;
                    const float wgt = expf(ms - M);
                    Ls = fmaf(wgt, S.gpart[s * PW + 1], Ls);
                    A = fmaf(wgt, S.gpart[s * PW + 2 + tid], A);
                }
                ll_put_rep(X + C::XB_ATT, D, h * 64 + tid, A / Ls, ep);
            }
            if (!last && npos > 0) kv_chunk_dma<D>(kc_l + lstride, vc_l + lstride, h, p0, npos, S.big);
        }
        // ---- C, D (no phase B)
        load_d<D, F>(w, wq, ws);
        if (!phase_c<D, F>(a, S, X, w, r, l)) return false;
        if (!last) {
            const uint8_t* wqn = wq + a.wq_layer;
            const float* wsn = ws + a.ws_layer;
            wblk_load<C::LPR_D, C::CPL_D, C::NP_Q>(wqh, wqn + O::QO, wsn + O::QS, D, h * 64, 64);
            ln_load<D>(ln1, ln + 4 * D, ln + 5 * D);
        }
        if (!phase_d<D, F>(a, S, X, w, l)) return false;
    }
    return true;
}

// Every layer for a workgroup without attention duty: new K/V rows in
// phase A; phases B, C, D like every workgroup.
template <int D, int F>
__device__ __forceinline__ bool free_role(const Args& a, const Lds<D, F>& S, const Role& role,
                                          float (&r)[LnRegs<D>::PER]) {
    using C = Cfg<D, F>;
    using O = Off<D, F>;
    const uint32_t ep = a.epoch;
    const size_t lstride = (size_t)a.kv_seqs * a.t_cap * D;
    WBlk<C::CPL_D, C::NP_KV> wkv;
    BcdW<D, F> w;
    LnRegs<D> ln1;
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
        // ---- A: r += f_prev; LN1; new K/V rows
        if (!phase_a_ln<D, F>(a, S, ln1, r, l)) return false;
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
        load_bc<D, F>(w, wq, ws, ln, role.o_row0);
        // ---- B, C, D
        if (!phase_b<D, F>(a, S, X, w, role.o_row0, l)) return false;
        load_d<D, F>(w, wq, ws);
        if (!phase_c<D, F>(a, S, X, w, r, l)) return false;
        if (!last) {
            if (role.kv_rows > 0)
                wblk_load<C::LPR_D, C::CPL_D, C::NP_KV>(wkv, wq + a.wq_layer + O::QO, ws + a.ws_layer + O::QS, D,
                                                        D + role.kv_row0, role.kv_rows);
            ln_load<D>(ln1, ln + 4 * D, ln + 5 * D);
        }
        if (!phase_d<D, F>(a, S, X, w, l)) return false;
    }
    return true;
}

template <int D, int F>
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

    const bool ok = role.head >= 0 ? attention_role<D, F>(a, S, role, r) : free_role<D, F>(a, S, role, r);
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
static void build_roles(Role* roles) {
    using C = Cfg<D, F>;
    int free_list[NWG];
    int nfree = 0;
    int nh_x[NXCD] = {0};
    for (int h = 0; h < C::H; ++h) ++nh_x[h % NXCD];
    for (int w = 0; w < NWG; ++w) {
        Role& r = roles[w];
        r = Role{-1, 0, 0, 0, -1, 0, 0, 0};
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

// The largest T_past the persistent step handles (its splits of <= MAXPOS
// positions each).
int persistent_max_position(int d, int F) {
    if (d == 768 && F == 3072) return pd::Cfg<768, 3072>::ATT_S * pd::MAXPOS;
    if (d == 1024 && F == 4096) return pd::Cfg<1024, 4096>::ATT_S * pd::MAXPOS;
    if (d == 1536 && F == 6144) return pd::Cfg<1536, 6144>::ATT_S * pd::MAXPOS;
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
    pd::build_roles<D, F>(host);
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
    const int chunk = (p.t0 + C::ATT_S - 1) / C::ATT_S;
    if (chunk > pd::MAXPOS) return hipErrorInvalidValue;
    a.chunk = chunk < 1 ? 1 : chunk;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)pd::k_decode_step<D, F>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)(sizeof(float) * C::LDS_FLOATS));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    pd::k_decode_step<D, F><<<dim3(pd::NWG), dim3(pd::NT), sizeof(float) * C::LDS_FLOATS, st>>>(a);
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
