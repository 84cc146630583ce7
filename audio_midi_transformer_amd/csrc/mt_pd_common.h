// Device helpers shared by the single-launch decode steps (gfx950): the
// exchange words between workgroups, LayerNorm with the residual held in
// registers, and INT4 group-32 rows held in registers with their dot
// products against activations in LDS.
#pragma once
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace mt {
namespace pd {

constexpr int NT = 256;      // threads per workgroup
constexpr int NWG = 256;     // workgroups (one per CU)
constexpr int NXCD = 8;      // workgroup w runs on XCD w % 8
constexpr int REP = NXCD;    // copies of each broadcast vector, one per XCD
constexpr int PW = 66;       // words per attention partial: m, l, acc[64]
constexpr uint32_t SPIN_LIMIT = 1u << 21;

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

// Loads through the global address space.  The weight pointers come from a
// device-side table; without the cast the compiler emits flat loads, which
// also count against the LDS wait counter.
template <typename T>
__device__ __forceinline__ T gload(const T* p) {
    return *(const __attribute__((address_space(1))) T*)(p);
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
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

// Two nibble values (0 .. 15, one per byte, bytes 2 sel and 2 sel + 1 of x)
// as floats, u * 2^-9, in one v_cvt_pk_f32_fp8: an FP8 E4M3 byte whose sign
// and upper exponent bits are zero encodes u * 2^-9 exactly (u < 8
// subnormal, 8 <= u < 16 the first binade; u * 2^-10 in the variant with
// exponent bias 8), so the conversion takes two weights per instruction
// instead of one v_cvt_f32_ubyte each.  u4_unit() gives the factor back.
template <bool SEL>
__device__ __forceinline__ f32x2_t u4_pair(unsigned x) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)x, SEL);
}
// 1 / (the float u4_pair gives for u = 1): a power of two.
__device__ __forceinline__ float u4_unit() {
    return 8.0f / u4_pair<false>(8u).x;
}

// sum_k u_k x_k / u4_unit() over one group.  Byte j of the group holds
// input 2j (low nibble) and 2j+1 (high nibble).  Every product is the exact
// power-of-two multiple of the one with integer u, and the sum is formed in
// the same order, so after the factor the result is the integer form's bit
// for bit.  `m` is 0x0F0F0F0F, passed in at run time so that the compiler
// does not turn the mask and shift into bit-field extracts.
__device__ __forceinline__ float dot_u(uint4 w, const float (&x)[32], unsigned m) {
    const unsigned wd[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const unsigned lo = wd[k] & m;
        const unsigned hi = (wd[k] >> 4) & m;
        const f32x2_t l01 = u4_pair<false>(lo), l23 = u4_pair<true>(lo);
        const f32x2_t h01 = u4_pair<false>(hi), h23 = u4_pair<true>(hi);
        const float* xm = x + 8 * k;
        acc = fmaf(l01.x, xm[0], acc);
        acc = fmaf(h01.x, xm[1], acc);
        acc = fmaf(l01.y, xm[2], acc);
        acc = fmaf(h01.y, xm[3], acc);
        acc = fmaf(l23.x, xm[4], acc);
        acc = fmaf(h23.x, xm[5], acc);
        acc = fmaf(l23.y, xm[6], acc);
        acc = fmaf(h23.y, xm[7], acc);
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
    const float unit = u4_unit();
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
        for (int p = 0; p < NP; ++p) acc[p] = fmaf(w.s[p][j], fmaf(dot_u(w.q[p][j], x, m), unit, x8), acc[p]);
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

// Row handled by this lane in pass p, or -1 if this lane does not write.
template <int LPR>
__device__ __forceinline__ int out_row(int p) {
    constexpr int RP = NT / LPR;
    return (threadIdx.x % LPR) == res_lane(LPR) ? p * RP + threadIdx.x / LPR : -1;
}

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

}  // namespace pd
}  // namespace mt
