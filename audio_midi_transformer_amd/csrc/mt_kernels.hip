// HIP kernels (gfx950) for the MuScriptor INT4 decoder step: one kernel per
// operation.  Used for prefill at every batch size and for decode when the
// persistent single-launch step is not selected.
//
// Operations and the passages that define them:
//   embed / prefix concat      small ONNX conversion page, decoder inputs
//   INT4 dequant matmul        medium ONNX README, "Model variant"
//                              (symmetric RTN INT4, group 32, FP32 activations)
//   causal attention, cache    small ONNX conversion page (cache [L,B,T,H,64],
//                              positions implied by T_past)
//   residual + LayerNorm       medium ONNX README, "Model variant"
//                              (SkipLayerNormalization nodes)
//   LM head + greedy argmax    medium ONNX README table (FP32 LM head); small
//                              ONNX conversion page (greedy decoding)
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include <algorithm>
#include <stdint.h>

#include "mt_internal.h"

namespace mt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Sum over the `width` consecutive lanes of a lane group (width power of 2).
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Max / sum over each row of 16 lanes (DPP row = 16 lanes), in every lane.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dppf<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dppf<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dppf<0x141>(v));  // row_half_mirror
    return fmaxf(v, dppf<0x140>(v));  // row_mirror
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dppf<0xB1>(v);
    v += dppf<0x4E>(v);
    v += dppf<0x141>(v);
    return v + dppf<0x140>(v);
}

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

struct EpiArgs {
    Epilogue epi;
    QkvDest qkv;
    // split K with a deterministic sum (k_gemm_w4_bf3 only): workgroup z
    // of the K split stores its products to part[z][m][n]; k_splitk_add adds
    // them to y in the order z = 0, 1, ...
    float* part = nullptr;
};

__device__ __forceinline__ void epilogue(const EpiArgs& e, float* __restrict__ y, int ldy, int m, int n,
                                         float v) {
    switch (e.epi) {
        case EPI_STORE: y[(size_t)m * ldy + n] = v; break;
        case EPI_GELU: y[(size_t)m * ldy + n] = gelu_erf(v); break;
        case EPI_RESID: y[(size_t)m * ldy + n] += v; break;
        case EPI_QKV: {
            const QkvDest& q = e.qkv;
            if (n < q.d) {
                q.q[(size_t)m * q.d + n] = v;
            } else {
                const int b = q.b0 + m / q.rows_per_seq, i = m % q.rows_per_seq;
                const size_t slot = ((size_t)(q.layer * q.batch + b) * q.t_cap + q.pos.t[b] + i) * q.d;
                if (n < 2 * q.d) q.kc[slot + (n - q.d)] = v;
                else q.vc[slot + (n - 2 * q.d)] = v;
            }
        } break;
    }
}

// ---------------------------------------------------------------- embed

// x rows of sequence b: [prefix_b (P rows) ; E[tokens_b] (S rows)].
__global__ __launch_bounds__(256) void k_embed(const int64_t* __restrict__ tokens, int S,
                                               const float* __restrict__ prefix, int P,
                                               const float* __restrict__ emb, int V, int d,
                                               float* __restrict__ x, int* err) {
    const int R = P + S;
    const int row = blockIdx.x;  // b * R + i
    const int b = row / R, i = row % R;
    float* dst = x + (size_t)row * d;
    if (i < P) {
        const float* src = prefix + ((size_t)b * P + i) * d;
        for (int j = threadIdx.x; j < d; j += blockDim.x) dst[j] = src[j];
    } else {
        const int64_t tok = tokens[(size_t)b * S + (i - P)];
        if (tok < 0 || tok >= V) {
            if (threadIdx.x == 0) atomicOr(err, 1);
            for (int j = threadIdx.x; j < d; j += blockDim.x) dst[j] = __builtin_nanf("");
            return;
        }
        const float* src = emb + (size_t)tok * d;
        for (int j = threadIdx.x; j < d; j += blockDim.x) dst[j] = src[j];
    }
}

// ---------------------------------------------------------------- LayerNorm

// One block per row: y = (x - mean) / sqrt(var + eps) * g + b, biased var.
__global__ __launch_bounds__(256) void k_layernorm(const float* __restrict__ x, long ldx,
                                                   const float* __restrict__ g,
                                                   const float* __restrict__ bta, float eps, int d,
                                                   float* __restrict__ y, long ldy) {
    __shared__ float red[4];
    const float* xr = x + (size_t)blockIdx.x * ldx;
    float* yr = y + (size_t)blockIdx.x * ldy;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float v[8];
    int n = 0;
    float s = 0.f;
    for (int j = tid; j < d; j += 256, ++n) {
        v[n] = xr[j];
        s += v[n];
    }
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    const float mean = ((red[0] + red[1]) + (red[2] + red[3])) / (float)d;
    __syncthreads();
    float q = 0.f;
    for (int k = 0; k < n; ++k) {
        const float c = v[k] - mean;
        q = fmaf(c, c, q);
    }
    q = wave_sum(q);
    if (lane == 0) red[wave] = q;
    __syncthreads();
    const float var = ((red[0] + red[1]) + (red[2] + red[3])) / (float)d;
    const float rstd = 1.0f / sqrtf(var + eps);
    n = 0;
    for (int j = tid; j < d; j += 256, ++n) yr[j] = (v[n] - mean) * rstd * g[j] + bta[j];
}

// Decode-attention partial of one (sequence, head, split): max score, sum of
// exp, two pad floats, then sum of exp * V (16-byte aligned).
constexpr int PART = 68;
constexpr int PART_ACC = 4;

// ---------------------------------------------------------------- INT4 GEMV (M <= 8) on MFMA

constexpr int GV_MAXSPAN = 2048;  // activation columns staged in LDS at a time
constexpr int GV_M = 8;           // activation rows held in LDS

// Source of the activation rows (a template parameter, so that every load
// of a variant is straight-line code and each wait counts exactly the loads
// it needs).
enum GemvSrc : int { GS_ROWS = 0, GS_LN = 1, GS_PARTS = 2 };

// Sum over each group of 32 lanes in every lane: DPP within rows of 16, one
// swap between the two rows.
__device__ __forceinline__ float sum32(float v) {
    v = row_sum16(v);
    return v + __shfl_xor(v, 16);
}

// Y[m, n] = sum_k W'[n, k] x[m, k] for M <= 8 rows with v_mfma_f32_16x16x4f32
// (A = 16 output rows of W' x 4 columns, B = 4 columns x 16 activation rows,
// 8 of them used).  x is read from X, or (part != NULL) merged from
// decode-attention partials of H heads and ns splits; optionally replaced
// by LayerNorm(x) (gain ln_g, bias ln_b, biased variance; whole rows).
// Workgroup (n block, k split): 16 output rows over columns
// [ks * kspan, (ks + 1) * kspan), staged through LDS in chunks of <=
// GV_MAXSPAN columns; the four waves take interleaved quarters of each
// chunk's groups (at most NG each) and their 16 x 16 tiles are summed in
// LDS.  With more than one k split the results are added to Y atomically
// (the += epilogue only).
//
// Lane l = 16 kq + r works on weight row n0 + r and, in every group of 32
// columns, on the 8 contiguous columns 8 kq .. 8 kq + 7: INT4 weights are one
// dword of nibbles per lane and group (converted as s * u - 8 s, one
// rounding, equal to (u - 8) * s), dense weights one or two 16-byte pieces,
// and the matching activations two 16-byte LDS reads, fetched one group
// ahead.  The weights come from the GEMV tiling (launch_tile_weights): per
// (16-row block, group) the 64 lanes' pieces are consecutive, so every load
// instruction reads one contiguous block.  Loads are issued activations
// first, then every weight group (addresses clamped, never predicated), so
// that staging waits only for the activations while the weights are still in
// flight, and each group's MFMAs wait only for that group.  Rows past N are
// zero padding in the tiling; their results are dropped.
//
// A8 (W4A8 variant): after staging, each (row, group of 32) of the staged
// activations is coded to INT8 (s_a = max|x| / 127, code = clamp(rint(x *
// (1 / s_a)), +-127)) in LDS, and each group is one v_mfma_i32_16x16x32_i8
// with A = activation codes (16 rows, 8 used) and B = 16 (u - 8) of 16
// weight rows; the INT32 tile is exact and is added to the FP32 result as
// I * s_a * s_w / 16.
//
// NG: groups per wave and chunk at most (4, 8, 12 or 16); SRC: GemvSrc.
template <int WF, bool A8, int NG, int SRC>
__global__ __launch_bounds__(256) void k_gemv_w4(const float* __restrict__ X, int ldx, int M, int K, int kspan,
                                                 const float* __restrict__ ln_g, const float* __restrict__ ln_b,
                                                 float eps, const float* __restrict__ part, int H, int ns,
                                                 const uint8_t* __restrict__ Wq, const float* __restrict__ Ws,
                                                 int N, float* __restrict__ Y, int ldy, EpiArgs ep) {
    extern __shared__ float xt[];  // [GV_M][chunk + 4]
    __shared__ float dred[4][16][17];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 16;
    const int G = K / 32;
    const int kb0 = blockIdx.y * kspan;
    const int kq = lane >> 4;
    const int bm = lane & 15;  // activation row this lane feeds into B
    const int xm = tid >> 5, xr = tid & 31;  // staging: row, thread in row (32 per row)
    const bool xrow = xm < M;
    const int xmc = min(xm, M - 1);  // rows past M load row M - 1 and store zeros
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
    for (int c0 = 0; c0 < kspan; c0 += GV_MAXSPAN) {
        const int cw = min(GV_MAXSPAN, kspan - c0);  // columns in this chunk
        const int XS = cw + 4;                       // LDS row stride
        const int kbase = kb0 + c0;
        const int gch = cw / 32, gbase = kbase / 32;
        // this wave's groups of the chunk: g = wave, wave + 4, ...; ngw <= NG
        // of them, uniform over the wave
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const int ngw = (gch - wv + 3) / 4;
        const int nf4 = (cw / 4 + 31) / 32;  // float4 per staging thread, <= NG
        // ---- activations first (plain rows only), with the LayerNorm gain
        // and bias of the chunk when it is fused: float4 f < cw / 4 of the
        // gain, then of the bias, spread over the workgroup
        float4 v[NG];
        float4 gb[NG / 4];
        if constexpr (SRC != GS_PARTS) {
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int k = min((xr + i * 32) * 4, cw - 4);
                v[i] = *reinterpret_cast<const float4*>(X + (size_t)xmc * ldx + kbase + k);
            }
            if constexpr (SRC == GS_LN) {
#pragma unroll
                for (int j = 0; j < NG / 4; ++j) {
                    const int f = min(tid + 256 * j, cw / 2 - 1);
                    gb[j] = *reinterpret_cast<const float4*>(f < cw / 4 ? ln_g + kbase + 4 * f
                                                                         : ln_b + kbase + 4 * (f - cw / 4));
                }
            }
        }
        // ---- then every weight group of this wave (INT4: nibble dword kq
        // and the group scale; F16: 8 halves; F32: 8 floats' bits)
        unsigned w4[WF == WF_INT4 ? NG : 1];
        float sc[WF == WF_INT4 ? NG : 1];
        uint4 wq[WF == WF_INT4 ? 1 : NG];
        uint4 wq2[WF == WF_F32 ? NG : 1];
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            // tile (row block, group): lane l's piece at unit l, so a wave
            // reads one contiguous block (256 B INT4, 1 KB half, 2 KB float)
            const size_t tg = (size_t)blockIdx.x * G + gbase + min(wv + 4 * i, gch - 1);
            if constexpr (WF == WF_INT4) {
                w4[i] = reinterpret_cast<const unsigned*>(Wq)[tg * 64 + lane];
                sc[i] = Ws[tg * 16 + (lane & 15)];
            } else if constexpr (WF == WF_F16) {
                wq[i] = reinterpret_cast<const uint4*>(Wq)[tg * 64 + lane];
            } else {
                wq[i] = reinterpret_cast<const uint4*>(Wq)[tg * 128 + lane];
                wq2[i] = reinterpret_cast<const uint4*>(Wq)[tg * 128 + 64 + lane];
            }
        }
        if (c0) __syncthreads();
        // ---- stage x[m][kbase .. kbase + cw) into xt[m][k]
        if constexpr (SRC == GS_PARTS) {
            // attention output merged from the partials: first the weight
            // e^(m_s - M) / sum_s e^(m_s - M) l_s of every (row, head, split),
            // one (row, head) per thread, then the weighted sums of acc_s
            const int nh = cw / 64, h0 = kbase / 64;
            float* wts = xt + (size_t)XS * GV_M;  // [M][nh][ns]
            if (tid < M * nh) {
                const int m = tid / nh, hl = tid % nh;
                const float* pp = part + (size_t)(m * H + h0 + hl) * ns * PART;
                float* wr = wts + (size_t)(m * nh + hl) * ns;
                float Mx = -INFINITY;
#pragma unroll 8
                for (int sp = 0; sp < ns; ++sp) {
                    wr[sp] = pp[sp * PART];
                    Mx = fmaxf(Mx, wr[sp]);
                }
                float L = 0.f;
#pragma unroll 8
                for (int sp = 0; sp < ns; ++sp) {
                    const float e = wr[sp] == -INFINITY ? 0.f : expf(wr[sp] - Mx);
                    wr[sp] = e;
                    L = fmaf(e, pp[sp * PART + 1], L);
                }
                const float inv = 1.0f / L;
                for (int sp = 0; sp < ns; ++sp) wr[sp] *= inv;
            }
            __syncthreads();
            for (int i = 0; i < nf4; ++i) {
                const int k = (xr + i * 32) * 4;
                if (k < cw) {
                    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
                    if (xrow) {
                        const int hl = k >> 6, j = k & 63;
                        const float* pp = part + (size_t)(xm * H + h0 + hl) * ns * PART + PART_ACC + j;
                        const float* wr = wts + (size_t)(xm * nh + hl) * ns;
#pragma unroll 8
                        for (int sp = 0; sp < ns; ++sp) {
                            const float4 a = *reinterpret_cast<const float4*>(pp + sp * PART);
                            const float wgt = wr[sp];
                            v.x = fmaf(wgt, a.x, v.x);
                            v.y = fmaf(wgt, a.y, v.y);
                            v.z = fmaf(wgt, a.z, v.z);
                            v.w = fmaf(wgt, a.w, v.w);
                        }
                    }
                    *reinterpret_cast<float4*>(xt + xm * XS + k) = v;
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int k = (xr + i * 32) * 4;
                if (!(i < nf4 && k < cw && xrow)) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
            if constexpr (SRC == GS_LN) {  // one chunk holds the whole row
                // gain [cw] and bias [cw] go to LDS past the activation rows
                float* lnb = xt + (size_t)XS * GV_M;
#pragma unroll
                for (int j = 0; j < NG / 4; ++j) {
                    const int f = tid + 256 * j;
                    if (f < cw / 2) *reinterpret_cast<float4*>(lnb + 4 * f) = gb[j];
                }
                float sm = 0.f;
#pragma unroll
                for (int i = 0; i < NG; ++i) sm += (v[i].x + v[i].y) + (v[i].z + v[i].w);
                const float mean = sum32(sm) / (float)K;
                float q = 0.f;
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const int k = (xr + i * 32) * 4;
                    if (i < nf4 && k < cw) {
                        const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
                        q = fmaf(a0, a0, fmaf(a1, a1, fmaf(a2, a2, fmaf(a3, a3, q))));
                    }
                }
                const float var = sum32(q) / (float)K;
                const float rstd = 1.0f / sqrtf(var + eps);
                __syncthreads();  // gain and bias in LDS
#pragma unroll
                for (int i = 0; i < NG; ++i) {
                    const int k = (xr + i * 32) * 4;
                    if (i < nf4 && k < cw && xrow) {
                        const float4 gg = *reinterpret_cast<const float4*>(lnb + k);
                        const float4 bb = *reinterpret_cast<const float4*>(lnb + cw + k);
                        v[i].x = (v[i].x - mean) * rstd * gg.x + bb.x;
                        v[i].y = (v[i].y - mean) * rstd * gg.y + bb.y;
                        v[i].z = (v[i].z - mean) * rstd * gg.z + bb.z;
                        v[i].w = (v[i].w - mean) * rstd * gg.w + bb.w;
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                const int k = (xr + i * 32) * 4;
                if (i < nf4 && k < cw) *reinterpret_cast<float4*>(xt + xm * XS + k) = v[i];
            }
        }
        __syncthreads();
        if constexpr (A8 && WF == WF_INT4) {
            // ---- INT8 codes of the staged rows, one (row, group) per thread
            // and pass: codes [GV_M][cw] bytes, scales [gch][GV_M]
            const size_t wfl = SRC == GS_PARTS ? (size_t)M * (cw / 64) * ns : 0;
            int8_t* xq = reinterpret_cast<int8_t*>(xt + (size_t)XS * GV_M + ((wfl + 3) & ~(size_t)3));
            float* xsa = reinterpret_cast<float*>(xq + (size_t)GV_M * cw);
            for (int p = tid; p < GV_M * gch; p += 256) {
                const int m = p & (GV_M - 1), g = p / GV_M;
                const float* src = xt + m * XS + g * 32;
                float v[32];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float4 t = *reinterpret_cast<const float4*>(src + 4 * j);
                    v[4 * j] = t.x;
                    v[4 * j + 1] = t.y;
                    v[4 * j + 2] = t.z;
                    v[4 * j + 3] = t.w;
                }
                float amax = 0.f;
#pragma unroll
                for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
                const float sa = amax / 127.0f;
                const float ra = sa != 0.f ? 1.0f / sa : 0.f;
                unsigned pk[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    unsigned w = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float c = fminf(fmaxf(rintf(__fmul_rn(v[4 * j + b], ra)), -127.f), 127.f);
                        w |= ((unsigned)(int)c & 0xFFu) << (8 * b);
                    }
                    pk[j] = w;
                }
                uint4* dst = reinterpret_cast<uint4*>(xq + (size_t)m * cw + g * 32);
                dst[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
                dst[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
                xsa[g * GV_M + m] = sa;
            }
            __syncthreads();
            // ---- one INT8 MFMA per group.  A: lane l gives codes k = 8 kq ..
            // 8 kq + 7 of activation row l % 16 (zero for rows >= GV_M); B:
            // 16 (u - 8) of weight row n0 + l % 16 at the same k, built from
            // dword kq of the group (low nibbles = even k) by sign-flipping
            // the nibbles and interleaving the two halves with v_perm.
            const bool avalid = bm < GV_M;
            const int8_t* xa = xq + (size_t)(bm & (GV_M - 1)) * cw + 8 * kq;
#pragma unroll
            for (int i = 0; i < NG; ++i) {
                if (i < ngw) {
                    const int gi = wv + 4 * i;
                    const unsigned x8 = w4[i] ^ 0x88888888u;
                    const unsigned lo = (x8 << 4) & 0xF0F0F0F0u, hi = x8 & 0xF0F0F0F0u;
                    const unsigned b0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
                    const unsigned b1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
                    const long bop = (long)(((unsigned long)b1 << 32) | b0);
                    const long aop = avalid ? *reinterpret_cast<const long*>(xa + gi * 32) : 0L;
                    const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x32_i8(aop, bop, i32x4{0, 0, 0, 0}, 0, 0, 0);
                    const float sw = sc[i] * 0.0625f;
                    const float4 sa = *reinterpret_cast<const float4*>(xsa + gi * GV_M + 4 * (kq & 1));
                    f32x4& ac = (i & 1) ? acc1 : acc0;
                    ac[0] = fmaf((float)d[0], sa.x * sw, ac[0]);
                    ac[1] = fmaf((float)d[1], sa.y * sw, ac[1]);
                    ac[2] = fmaf((float)d[2], sa.z * sw, ac[2]);
                    ac[3] = fmaf((float)d[3], sa.w * sw, ac[3]);
                }
            }
            continue;
        }
        // ---- MFMA over this wave's groups, alternate groups into two
        // accumulators.  Step s of a group takes column 8 kq + s; the lanes
        // feeding B columns 8..15 read row bm - 8, whose products land in
        // D columns that are never read.
        const float* xb = xt + (bm & (GV_M - 1)) * XS + 8 * kq;
        float4 nb0 = make_float4(0.f, 0.f, 0.f, 0.f), nb1 = nb0;
        if (ngw > 0) {
            nb0 = *reinterpret_cast<const float4*>(xb + wv * 32);
            nb1 = *reinterpret_cast<const float4*>(xb + wv * 32 + 4);
        }
#pragma unroll
        for (int i = 0; i < NG; ++i) {
            if (i < ngw) {
                const float bv[8] = {nb0.x, nb0.y, nb0.z, nb0.w, nb1.x, nb1.y, nb1.z, nb1.w};
                if (i + 1 < ngw) {
                    nb0 = *reinterpret_cast<const float4*>(xb + (wv + 4 * i + 4) * 32);
                    nb1 = *reinterpret_cast<const float4*>(xb + (wv + 4 * i + 4) * 32 + 4);
                }
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    float a;
                    if constexpr (WF == WF_INT4) {
                        a = fmaf(sc[i], (float)((w4[i] >> (4 * s)) & 15u), -8.f * sc[i]);
                    } else if constexpr (WF == WF_F16) {
                        const unsigned hw[4] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w};
                        a = __half2float(__ushort_as_half((unsigned short)(hw[s >> 1] >> (16 * (s & 1)))));
                    } else {
                        const unsigned fw[8] = {wq[i].x, wq[i].y, wq[i].z, wq[i].w,
                                                wq2[i].x, wq2[i].y, wq2[i].z, wq2[i].w};
                        a = __uint_as_float(fw[s]);
                    }
                    if (i & 1) acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv[s], acc1, 0, 0, 0);
                    else acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a, bv[s], acc0, 0, 0, 0);
                }
            }
        }
    }
    const f32x4 acc = acc0 + acc1;
    // ---- sum the four waves' tiles; lane l holds D[4 (l / 16) + r][l % 16]
    // (weight row x activation row; transposed in the A8 form)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if (A8) dred[wave][lane & 15][4 * kq + r] = acc[r];
        else dred[wave][4 * kq + r][lane & 15] = acc[r];
    }
    __syncthreads();
    const int n = tid >> 4, m = tid & 15;
    if (m < M && n0 + n < N) {
        const float v = (dred[0][n][m] + dred[1][n][m]) + (dred[2][n][m] + dred[3][n][m]);
        if (gridDim.y > 1) atomicAdd(Y + (size_t)m * ldy + n0 + n, v);
        else epilogue(ep, Y, ldy, m, n0 + n, v);
    }
}

// ---------------------------------------------------------------- INT4 GEMM (FP32 MFMA)

// Y[M, N] = X[M, K] . W'^T with W' = (u - 8) * s dequantised exactly into LDS.
// Tile TM x 64 per workgroup, K step GK per LDS stage, the next stage's
// activations and nibbles loaded into registers while the current one is
// multiplied.  Two shapes: TM = 64 with GK = 64 for long inputs (many
// workgroups, four per CU by LDS), TM = 32 with GK = 128 for short prompts,
// where 64-row tiles would leave CUs idle and each workgroup needs more MFMA
// work per stage to cover the load latency.  Four waves as 2 x 2, each a
// (TM / 2) x 32 sub-tile of (TM / 32) x 2 v_mfma_f32_16x16x4f32 blocks.
// Operand layout of that instruction: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; it receives D[4 (l / 16) + r][l % 16], r = 0..3.
// blockIdx.z splits K into kspan-column ranges whose results are added
// atomically (+= epilogue only).
constexpr int GN = 64;
constexpr size_t gemm_lds(int tm, int gk) { return sizeof(float) * (tm + GN) * (gk + 4); }

template <int TM, int GK, int WF>
__global__ __launch_bounds__(256) void k_gemm_w4(const float* __restrict__ X, int ldx, int M, int K,
                                                 const uint8_t* __restrict__ Wq,
                                                 const float* __restrict__ Ws, int N,
                                                 float* __restrict__ Y, int ldy, EpiArgs ep, int kspan) {
    constexpr int GS = GK + 4;   // LDS row stride in floats
    constexpr int MI = TM / 32;  // 16-row MFMA blocks per wave
    extern __shared__ float gsm[];
    float* As = gsm;            // [TM][GS]
    float* Bs = gsm + TM * GS;  // [64][GS]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * GN;
    const int G = K / 32;
    const int kb = blockIdx.z * kspan, ke = min(K, kb + kspan);
    f32x4 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // stage loads.  Activations: TM rows x GK columns, TM * GK / 1024 float4
    // per thread.  Nibbles: thread t takes quarter t % 4 (GK / 4 columns,
    // inside one group) of weight row t / 4, with that group's scale.
    constexpr int NA = TM * GK / 4 / 256;
    // weight dwords per thread: GK / 4 columns as nibbles, halves or floats
    constexpr int NW = WF == WF_INT4 ? GK / 32 : WF == WF_F16 ? GK / 8 : GK / 4;
    constexpr int ESZ2 = WF == WF_INT4 ? 1 : WF == WF_F16 ? 4 : 8;  // bytes per 2 columns
    // The next stage is loaded into registers while the current one is
    // multiplied.  Every load is issued (addresses clamped into the matrix,
    // out-of-range values replaced afterwards), so each wait counts exactly
    // one stage's loads.
    struct Stage {
        float4 a[NA];
        unsigned w[NW];
        float s;
    };
    Stage st;
    const int wrow = tid >> 2, wq = tid & 3;
    const int klast = ke - 1;  // any column of the range, for clamping
    auto load_stage = [&](int k0, Stage& S) {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + e * 256;
            const int r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
            const bool ok = m0 + r < M && k0 + c < ke;
            const int rr = min(m0 + r, M - 1), cc = min(k0 + c, (klast & ~3));
            const float4 t = *reinterpret_cast<const float4*>(X + (size_t)rr * ldx + cc);
            S.a[e] = ok ? t : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        const int c0 = k0 + wq * (GK / 4);
        const bool ok = n0 + wrow < N && c0 < ke;
        const int cc0 = min(c0, (klast & ~(GK / 4 - 1)));
        const int rw = min(n0 + wrow, N - 1);
        const uint8_t* wrow_p = Wq + ((size_t)rw * K + cc0) / 2 * ESZ2;
        const unsigned fill = WF == WF_INT4 ? 0x88888888u : 0u;
        if constexpr (NW % 4 == 0) {
#pragma unroll
            for (int i = 0; i < NW; i += 4) {
                const uint4 t = *reinterpret_cast<const uint4*>(wrow_p + 4 * i);
                S.w[i] = ok ? t.x : fill, S.w[i + 1] = ok ? t.y : fill;
                S.w[i + 2] = ok ? t.z : fill, S.w[i + 3] = ok ? t.w : fill;
            }
        } else {
#pragma unroll
            for (int i = 0; i < NW; i += 2) {
                const uint2 t = *reinterpret_cast<const uint2*>(wrow_p + 4 * i);
                S.w[i] = ok ? t.x : fill, S.w[i + 1] = ok ? t.y : fill;
            }
        }
        if constexpr (WF == WF_INT4) {
            const float sv = Ws[(size_t)rw * G + cc0 / 32];
            S.s = ok ? sv : 0.f;
        }
    };
    // one stage: stage S into LDS, refill S with stage k0 + GK, multiply
    auto run_stage = [&](int k0, Stage& S) {
        if (k0 != kb) __syncthreads();  // the previous stage has been multiplied
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + e * 256;
            *reinterpret_cast<float4*>(As + (idx / (GK / 4)) * GS + (idx % (GK / 4)) * 4) = S.a[e];
        }
        {
            float* dst = Bs + wrow * GS + wq * (GK / 4);
            if constexpr (WF == WF_INT4) {
                // dword d holds inputs 8 d .. 8 d + 7 of the quarter, low
                // nibble first.  The four threads of a row write their
                // quarters GK / 4 floats apart, i.e. on the same banks at
                // GK = 128; each thread therefore starts at dword rot and
                // goes round, so one write instruction covers all 32 banks.
                const int rot = GK == 128 ? wq : (wq >> 1);
#pragma unroll
                for (int t = 0; t < NW; ++t) {
                    const int d = (t + rot) & (NW - 1);
                    unsigned w = S.w[0];
#pragma unroll
                    for (int i = 1; i < NW; ++i) w = d == i ? S.w[i] : w;
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float v[4];
#pragma unroll
                        for (int b = 0; b < 2; ++b) {
                            const unsigned byte = (w >> (8 * (2 * h + b))) & 0xFFu;
                            v[2 * b] = (float)((int)(byte & 15u) - 8) * S.s;
                            v[2 * b + 1] = (float)((int)(byte >> 4) - 8) * S.s;
                        }
                        *reinterpret_cast<float4*>(dst + d * 8 + h * 4) = make_float4(v[0], v[1], v[2], v[3]);
                    }
                }
            } else if constexpr (WF == WF_F16) {
                // dword i holds inputs 2 i, 2 i + 1
#pragma unroll
                for (int i = 0; i < NW; i += 2) {
                    const float2 a = __half22float2(*reinterpret_cast<const __half2*>(&S.w[i]));
                    const float2 b = __half22float2(*reinterpret_cast<const __half2*>(&S.w[i + 1]));
                    *reinterpret_cast<float4*>(dst + 2 * i) = make_float4(a.x, a.y, b.x, b.y);
                }
            } else {
#pragma unroll
                for (int i = 0; i < NW; i += 4)
                    *reinterpret_cast<float4*>(dst + i) = make_float4(__uint_as_float(S.w[i]), __uint_as_float(S.w[i + 1]),
                                                                      __uint_as_float(S.w[i + 2]), __uint_as_float(S.w[i + 3]));
            }
        }
        __syncthreads();
        load_stage(k0 + GK, S);  // past the range: clamped loads, values unused
        // all GK / 4 steps, also in a partial last stage: its missing columns
        // were staged as zero activations and zero weights.  In each block of
        // 16 columns lane l takes columns 4 (l / 16) .. + 3 with one 16-byte
        // LDS read per operand and feeds them to four consecutive steps (the
        // same permutation of k on both operands).
#pragma unroll
        for (int kc = 0; kc < GK / 16; ++kc) {
            const int k = kc * 16 + 4 * (lane >> 4);
            float4 a[MI], b[2];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                a[i] = *reinterpret_cast<const float4*>(As + (wm * (TM / 2) + i * 16 + (lane & 15)) * GS + k);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const float4*>(Bs + (wn * 32 + j * 16 + (lane & 15)) * GS + k);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int i = 0; i < MI; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
        }
    };
    load_stage(kb, st);
    for (int k0 = kb; k0 < ke; k0 += GK) run_stage(k0, st);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * (TM / 2) + i * 16 + 4 * (lane >> 4) + r;
                const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                if (m < M && n < N) {
                    if (gridDim.z > 1) atomicAdd(Y + (size_t)m * ldy + n, acc[i][j][r]);
                    else epilogue(ep, Y, ldy, m, n, acc[i][j][r]);
                }
            }
}

// W4A8 form of the GEMM: Y[M, N] = sum_g s_w s_a I_g, I_g the exact INT32
// product of a group's activation codes (coded per row and group of 32 while
// staged: s_a = max|x| / 127, code = clamp(rint(x * (1 / s_a)), +-127)) and
// the weights' (u - 8).  Tile TM x 64, K stages of GK columns, four waves as
// 2 x 2 of (TM / 2) x 32; per group one v_mfma_i32_16x16x32_i8 per 16 x 16
// block, A = activation codes (lane l: row l % 16, k = 8 (l / 16) .. + 7),
// B = 16 (u - 8) (lane l: weight row l % 16, same k), D[4 (l / 16) + r][l % 16];
// the INT32 block is added to the FP32 result as I * s_a * s_w / 16.
// blockIdx.z takes the kspan-column range of K whose results are added
// atomically (+= epilogue only), as in the FP32 GEMM.
constexpr int QS = 8;  // LDS row padding (bytes) of the code tiles

template <int TM, int GK>
__global__ __launch_bounds__(256) void k_gemm_w4a8(const float* __restrict__ X, int ldx, int M, int K,
                                                   const uint8_t* __restrict__ Wq,
                                                   const float* __restrict__ Ws, int N,
                                                   float* __restrict__ Y, int ldy, EpiArgs ep, int kspan) {
    constexpr int MI = TM / 32;
    constexpr int NG = GK / 32;       // groups per stage
    constexpr int RS = GK + QS;       // code row stride (bytes)
    __shared__ __align__(16) int8_t Aq[TM * RS];
    __shared__ __align__(16) int8_t Bq[GN * RS];
    __shared__ __align__(16) float As_s[NG][TM];  // activation scales [group][row]
    __shared__ float Bs_s[NG][GN];    // weight scales / 16 [group][row]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * GN;
    const int G = K / 32;
    const int kb = blockIdx.z * kspan, ke = min(K, kb + kspan);  // this workgroup's K range
    f32x4 acc[MI][2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stage loads as in the FP32 GEMM: TM * GK / 1024 float4 of X per thread;
    // thread t: quarter t % 4 of weight row t / 4 (GK / 4 columns in one group)
    constexpr int NA = TM * GK / 4 / 256;
    constexpr int NW = GK / 32;
    float4 pa[NA];
    unsigned pw[NW];
    float ps = 0.f;
    const int wrow = tid >> 2, wq = tid & 3;
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + e * 256;
            const int r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
            pa[e] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + r < M && k0 + c < ke) pa[e] = *reinterpret_cast<const float4*>(X + (size_t)(m0 + r) * ldx + k0 + c);
        }
        const int c0 = k0 + wq * (GK / 4), g = c0 / 32;
        const bool ok = n0 + wrow < N && c0 < ke;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            pw[i] = ok ? *reinterpret_cast<const unsigned*>(Wq + (size_t)(n0 + wrow) * (K / 2) + c0 / 2 + 4 * i)
                       : 0x88888888u;
        ps = ok ? Ws[(size_t)(n0 + wrow) * G + g] : 0.f;
    };
    load_stage(kb);
    for (int k0 = kb; k0 < ke; k0 += GK) {
        if (k0 != kb) __syncthreads();  // the previous stage has been multiplied
        // activation codes: the 8 float4 of a (row, group) sit in 8
        // consecutive lanes; their maximum by DPP within the 8 lanes
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + e * 256;
            const int r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
            float am = fmaxf(fmaxf(fabsf(pa[e].x), fabsf(pa[e].y)), fmaxf(fabsf(pa[e].z), fabsf(pa[e].w)));
            am = fmaxf(am, dppf<0xB1>(am));   // quad_perm [1,0,3,2]
            am = fmaxf(am, dppf<0x4E>(am));   // quad_perm [2,3,0,1]
            am = fmaxf(am, dppf<0x141>(am));  // row_half_mirror: the 8-lane group
            const float sa = am / 127.0f;
            const float ra = sa != 0.f ? 1.0f / sa : 0.f;
            const float v[4] = {pa[e].x, pa[e].y, pa[e].z, pa[e].w};
            unsigned w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float cd = fminf(fmaxf(rintf(__fmul_rn(v[b], ra)), -127.f), 127.f);
                w |= ((unsigned)(int)cd & 0xFFu) << (8 * b);
            }
            *reinterpret_cast<unsigned*>(Aq + r * RS + c) = w;
            if ((c & 31) == 0) As_s[c >> 5][r] = sa;
        }
        // weight codes 16 (u - 8): sign-flip the nibbles, split even / odd
        // k, interleave back to k order with v_perm
        {
            int8_t* dst = Bq + wrow * RS + wq * (GK / 4);
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const unsigned x8 = pw[i] ^ 0x88888888u;
                const unsigned lo = (x8 << 4) & 0xF0F0F0F0u, hi = x8 & 0xF0F0F0F0u;
                *reinterpret_cast<uint2*>(dst + 8 * i) =
                    make_uint2(__builtin_amdgcn_perm(hi, lo, 0x05010400u), __builtin_amdgcn_perm(hi, lo, 0x07030602u));
            }
            if (((wq * (GK / 4)) & 31) == 0) Bs_s[(wq * (GK / 4)) >> 5][wrow] = ps * 0.0625f;
        }
        __syncthreads();
        if (k0 + GK < ke) load_stage(k0 + GK);
        const int kq = lane >> 4, l16 = lane & 15;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            long a[MI], b[2];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                a[i] = *reinterpret_cast<const long*>(Aq + (wm * (TM / 2) + i * 16 + l16) * RS + g * 32 + 8 * kq);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                b[j] = *reinterpret_cast<const long*>(Bq + (wn * 32 + j * 16 + l16) * RS + g * 32 + 8 * kq);
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const float4 sa = *reinterpret_cast<const float4*>(&As_s[g][wm * (TM / 2) + i * 16 + 4 * kq]);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const i32x4 d = __builtin_amdgcn_mfma_i32_16x16x32_i8(a[i], b[j], i32x4{0, 0, 0, 0}, 0, 0, 0);
                    const float sw = Bs_s[g][wn * 32 + j * 16 + l16];
                    acc[i][j][0] = fmaf((float)d[0], sa.x * sw, acc[i][j][0]);
                    acc[i][j][1] = fmaf((float)d[1], sa.y * sw, acc[i][j][1]);
                    acc[i][j][2] = fmaf((float)d[2], sa.z * sw, acc[i][j][2]);
                    acc[i][j][3] = fmaf((float)d[3], sa.w * sw, acc[i][j][3]);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * (TM / 2) + i * 16 + 4 * (lane >> 4) + r;
                const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                if (m < M && n < N) {
                    if (gridDim.z > 1) atomicAdd(Y + (size_t)m * ldy + n, acc[i][j][r]);
                    else epilogue(ep, Y, ldy, m, n, acc[i][j][r]);
                }
            }
}

// INT4 GEMM on BF16 matrix cores with FP32 results (W4A32).  Per group g
// of 32 inputs the partial sum P = sum_k x_k (u_k - 8) is formed with exact
// products: every activation is split into three bf16 pieces
// x = x1 + x2 + x3 (x1 = bf16(x), x2 = bf16(x - x1), x3 = x - x1 - x2; each
// remainder is exact in FP32 and the last one has at most 8 significant
// bits, so the split is exact), u - 8 is a bf16 integer, and a product of
// the two has at most 12 significant bits.  Three v_mfma_f32_16x16x32_bf16
// per group and 16 x 16 block accumulate the pieces against the codes in
// FP32, then acc += s_w * P.  The products are those of the FP32 form
// (x (u - 8) s with the scale applied per group instead of per weight); only
// the accumulation order differs, inside the same FP32 error bound.  BF16
// MFMA runs 16x16x32 in 16 cycles where FP32 MFMA needs 8 x 16x16x4 at 32.
// Tile TM x NT per workgroup (NT = 64, or 32 where 64-column tiles would
// leave fewer than two workgroups per CU, as for the 504-row O and FFN-down
// projections), K stages of GK columns, four waves as 2 x 2 of
// (TM / 2) x (NT / 2).  Operand layout (as the INT8 16x16x32 form): lane l
// supplies A row l % 16, k = 8 (l / 16) .. + 7, and B row (output column)
// l % 16, same k; it receives D[4 (l / 16) + r][l % 16].  blockIdx.z takes
// the kspan-column range of K whose results are added atomically (+=
// epilogue only), as in the other GEMMs.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// bf16 bits of (a, b), round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
    const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
    return __builtin_bit_cast(unsigned, h);
}
__device__ __forceinline__ float bf16_lo(unsigned p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(unsigned p) { return __uint_as_float(p & 0xFFFF0000u); }

template <int TM, int GK, int NT>
__global__ __launch_bounds__(256) void k_gemm_w4_bf3(const float* __restrict__ X, int ldx, int M, int K,
                                                     const uint8_t* __restrict__ Wq,
                                                     const float* __restrict__ Ws, int N,
                                                     float* __restrict__ Y, int ldy, EpiArgs ep, int kspan) {
    constexpr int MI = TM / 32;
    constexpr int NJ = NT / 32;      // 16-column blocks per wave
    constexpr int WPR = 256 / NT;    // threads per weight row (each GK / WPR columns)
    constexpr int NG = GK / 32;      // groups per stage
    constexpr int RS = GK + 8;       // row stride in bf16 (16-byte rows, shifted 4 banks per row)
    static_assert((GK / WPR) % 8 == 0 && 32 % (GK / WPR) == 0 || (GK / WPR) % 32 == 0, "weight part inside one group");
    __shared__ __align__(16) unsigned short Ap[3][TM * RS];  // activation pieces x1, x2, x3
    __shared__ __align__(16) unsigned short Bu[NT * RS];     // codes u - 8
    __shared__ float Bs_s[NG][NT];                           // weight scales [group][row]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * TM, n0 = blockIdx.x * NT;
    const int G = K / 32;
    const int kb = blockIdx.z * kspan, ke = min(K, kb + kspan);  // this workgroup's K range
    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // stage loads: TM * GK / 1024 float4 of X per thread; thread t takes
    // part t % WPR of weight row t / WPR (GK / WPR columns in one group) and
    // that group's scale
    constexpr int NA = TM * GK / 4 / 256;
    constexpr int NW = GK / WPR / 8;  // nibble dwords per thread
    float4 pa[NA];
    unsigned pw[NW];
    float ps = 0.f;
    const int wrow = tid / WPR, wq = tid % WPR;
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + e * 256;
            const int r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
            pa[e] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + r < M && k0 + c < ke) pa[e] = *reinterpret_cast<const float4*>(X + (size_t)(m0 + r) * ldx + k0 + c);
        }
        const int c0 = k0 + wq * (GK / WPR), g = c0 / 32;
        const bool ok = n0 + wrow < N && c0 < ke;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            pw[i] = ok ? *reinterpret_cast<const unsigned*>(Wq + (size_t)(n0 + wrow) * (K / 2) + c0 / 2 + 4 * i)
                       : 0x88888888u;
        ps = ok ? Ws[(size_t)(n0 + wrow) * G + g] : 0.f;
    };
    load_stage(kb);
    for (int k0 = kb; k0 < ke; k0 += GK) {
        if (k0 != kb) __syncthreads();  // the previous stage has been multiplied
        // activations: three bf16 pieces of every value
#pragma unroll
        for (int e = 0; e < NA; ++e) {
            const int idx = tid + e * 256;
            const int r = idx / (GK / 4), c = (idx % (GK / 4)) * 4;
            const float v[4] = {pa[e].x, pa[e].y, pa[e].z, pa[e].w};
            unsigned p1[2], p2[2], p3[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float a = v[2 * h], b = v[2 * h + 1];
                p1[h] = pk_bf16(a, b);
                const float ra = a - bf16_lo(p1[h]), rb = b - bf16_hi(p1[h]);
                p2[h] = pk_bf16(ra, rb);
                p3[h] = pk_bf16(ra - bf16_lo(p2[h]), rb - bf16_hi(p2[h]));
            }
            *reinterpret_cast<uint2*>(&Ap[0][r * RS + c]) = make_uint2(p1[0], p1[1]);
            *reinterpret_cast<uint2*>(&Ap[1][r * RS + c]) = make_uint2(p2[0], p2[1]);
            *reinterpret_cast<uint2*>(&Ap[2][r * RS + c]) = make_uint2(p3[0], p3[1]);
        }
        // weights: u - 8 as bf16 (exact), inputs in k order (low nibble of
        // byte j is input 2 j)
        {
            unsigned short* dst = Bu + wrow * RS + wq * (GK / WPR);
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                unsigned o[4];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const unsigned byte = (pw[i] >> (8 * b)) & 0xFFu;
                    o[b] = pk_bf16((float)(int)(byte & 15u) - 8.f, (float)(int)(byte >> 4) - 8.f);
                }
                *reinterpret_cast<uint4*>(dst + 8 * i) = make_uint4(o[0], o[1], o[2], o[3]);
            }
            if (((wq * (GK / WPR)) & 31) == 0) Bs_s[(wq * (GK / WPR)) >> 5][wrow] = ps;
        }
        __syncthreads();
        if (k0 + GK < ke) load_stage(k0 + GK);
        const int kq = lane >> 4, l16 = lane & 15;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            bf16x8 a[3][MI], b[NJ];
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int i = 0; i < MI; ++i)
                    a[p][i] = *reinterpret_cast<const bf16x8*>(&Ap[p][(wm * (TM / 2) + i * 16 + l16) * RS + g * 32 + 8 * kq]);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                b[j] = *reinterpret_cast<const bf16x8*>(&Bu[(wn * (NT / 2) + j * 16 + l16) * RS + g * 32 + 8 * kq]);
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0][i], b[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[1][i], b[j], d, 0, 0, 0);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[2][i], b[j], d, 0, 0, 0);
                    const float sw = Bs_s[g][wn * (NT / 2) + j * 16 + l16];
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sw, d[r], acc[i][j][r]);
                }
        }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * (TM / 2) + i * 16 + 4 * (lane >> 4) + r;
                const int n = n0 + wn * (NT / 2) + j * 16 + (lane & 15);
                if (m < M && n < N) {
                    if (ep.part) ep.part[((size_t)blockIdx.z * M + m) * N + n] = acc[i][j][r];
                    else if (gridDim.z > 1) atomicAdd(Y + (size_t)m * ldy + n, acc[i][j][r]);
                    else epilogue(ep, Y, ldy, m, n, acc[i][j][r]);
                }
            }
}

// Row blockIdx.x of y (row stride ldy, N <= 2048 columns):
// y[m, n] += part[0][m][n] + part[1][m][n] + ... (nsplit terms, added in
// that order); then, with g given, a[m, :] = LayerNorm(y[m, :]) * g + b
// with the statistics formed exactly as k_layernorm forms them (so a is
// bit-identical to a separate k_layernorm launch).  a may alias
// part[0]: each thread reads its own elements of the row before writing them.
__global__ __launch_bounds__(256) void k_splitk_add(float* __restrict__ y, int ldy, const float* part, int nsplit,
                                                    int M, int N, const float* __restrict__ g,
                                                    const float* __restrict__ bta, float eps, float* a, int lda) {
    __shared__ float red[4];
    const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float v[8];
    int n = 0;
    float s = 0.f;
    for (int j = tid; j < N; j += 256, ++n) {
        float p = part[(size_t)m * N + j];
        for (int z = 1; z < nsplit; ++z) p += part[((size_t)z * M + m) * N + j];
        const float x = y[(size_t)m * ldy + j] + p;
        y[(size_t)m * ldy + j] = x;
        v[n] = x;
        s += x;
    }
    if (!g) return;
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    const float mean = ((red[0] + red[1]) + (red[2] + red[3])) / (float)N;
    __syncthreads();
    float q = 0.f;
    for (int k = 0; k < n; ++k) {
        const float c = v[k] - mean;
        q = fmaf(c, c, q);
    }
    q = wave_sum(q);
    if (lane == 0) red[wave] = q;
    __syncthreads();
    const float var = ((red[0] + red[1]) + (red[2] + red[3])) / (float)N;
    const float rstd = 1.0f / sqrtf(var + eps);
    n = 0;
    for (int j = tid; j < N; j += 256, ++n) a[(size_t)m * lda + j] = (v[n] - mean) * rstd * g[j] + bta[j];
}

// ---------------------------------------------------------------- decode attention

// Split-K decode attention.  Workgroup (split, h, b) covers positions
// [split * chunk, min(T, (split + 1) * chunk)), chunk <= 256, of head h of
// sequence b and writes the unnormalised partial: max score, sum of exp, and
// sum of exp * V at offset PART_ACC.  16 lane groups of 16 lanes: group g
// takes positions g, g + 16, ... of the split, lane l of the group the
// dimensions 4l .. 4l + 3.  Every K and V row of the split is requested
// before the first is used.  The splits are merged where the attention
// output is read (the O projection's activation staging).
__global__ __launch_bounds__(256) void k_attn_decode(const float* __restrict__ q,
                                                     const float* __restrict__ kc,
                                                     const float* __restrict__ vc, int layer,
                                                     int B, int H, int t_cap, SeqPos Tn, int chunk,
                                                     float* __restrict__ part) {
    __shared__ float red[8];
    __shared__ float sacc[4][64];
    const int split = blockIdx.x, ns = gridDim.x, h = blockIdx.y, b = blockIdx.z;
    const int T = Tn.t[b];
    const int d = H * 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = tid >> 4, ql = tid & 15;
    const float4 q4 = *reinterpret_cast<const float4*>(q + (size_t)b * d + h * 64 + ql * 4);
    const size_t base = ((size_t)(layer * B + b) * t_cap) * d + h * 64 + ql * 4;
    const int t0 = split * chunk;
    const int n = max(0, min(T - t0, chunk));
    float4 k4[16], v4[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = g + 16 * i;
        k4[i] = v4[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < n) {
            // non-temporal: the step reads each cached row once, and the
            // weights the next launches read again should stay cached
            const f32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(kc + base + (size_t)(t0 + t) * d));
            const f32x4 vv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vc + base + (size_t)(t0 + t) * d));
            k4[i] = make_float4(kv[0], kv[1], kv[2], kv[3]);
            v4[i] = make_float4(vv[0], vv[1], vv[2], vv[3]);
        }
    }
    float sc[16];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float s = q4.x * k4[i].x + q4.y * k4[i].y + q4.z * k4[i].z + q4.w * k4[i].w;
        s = group_sum<16>(s) * 0.125f;
        sc[i] = g + 16 * i < n ? s : -INFINITY;
        mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float ls = 0.f;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (M != -INFINITY) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = sc[i] == -INFINITY ? 0.f : expf(sc[i] - M);
            ls += p;
            a.x = fmaf(p, v4[i].x, a.x);
            a.y = fmaf(p, v4[i].y, a.y);
            a.z = fmaf(p, v4[i].z, a.z);
            a.w = fmaf(p, v4[i].w, a.w);
        }
    }
#pragma unroll
    for (int o = 16; o <= 32; o <<= 1) {
        ls += __shfl_xor(ls, o);
        a.x += __shfl_xor(a.x, o);
        a.y += __shfl_xor(a.y, o);
        a.z += __shfl_xor(a.z, o);
        a.w += __shfl_xor(a.w, o);
    }
    if (lane < 16) {
        *reinterpret_cast<float4*>(&sacc[wave][ql * 4]) = a;
        if (ql == 0) red[4 + wave] = ls;
    }
    __syncthreads();
    float* pp = part + ((size_t)(b * H + h) * ns + split) * PART;
    if (tid < 64) {
        pp[PART_ACC + tid] = (sacc[0][tid] + sacc[1][tid]) + (sacc[2][tid] + sacc[3][tid]);
        if (tid == 0) {
            pp[0] = M;
            pp[1] = (red[4] + red[5]) + (red[6] + red[7]);
        }
    }
}

// Merge of the decode attention's split-K partials into attention rows, for
// batches whose O projection runs on the GEMM: workgroup (h, b), lane j
// forms out[b, 64 h + j] = sum_s e^(m_s - M) acc_s[j] / sum_s e^(m_s - M) l_s
// (M the largest m_s; splits with no keys have m_s = -inf and weigh 0), the
// same weights as the GEMV's merged-partials staging.
__global__ __launch_bounds__(64) void k_attn_merge(const float* __restrict__ part, int H, int ns,
                                                   float* __restrict__ out) {
    const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
    const float* pp = part + (size_t)(b * H + h) * ns * PART;
    float Mx = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) Mx = fmaxf(Mx, pp[sp * PART]);
    float L = 0.f, acc = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
        const float m = pp[sp * PART];
        const float e = m == -INFINITY ? 0.f : expf(m - Mx);
        L = fmaf(e, pp[sp * PART + 1], L);
        acc = fmaf(e, pp[sp * PART + PART_ACC + j], acc);
    }
    out[(size_t)b * H * 64 + h * 64 + j] = acc * (1.0f / L);
}

// ---------------------------------------------------------------- prefill attention

// Causal attention of R new rows per sequence (positions t0 .. t0+R-1) over
// the cache, on v_mfma_f32_16x16x4f32 (A = 16 rows x 4 columns, B = 4 x 16,
// lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and receives
// D[4 (l / 16) + r][l % 16]).  Workgroup (x, h, b): the 16 query rows of
// row block x, then those of row block nrb - 1 - x (nrb = ceil(R / 16)),
// so that the short and the long rows of a causal prompt pair up.
// The keys the block sees are cut into blocks of 32; wave w takes blocks w,
// w + 4, ..., so the long rows at the end of a prompt are shared by four
// waves instead of one.  Per key block a wave stages K and V in its own LDS
// tiles, computes S = Q K^T / 8 (two 16 x 16 tiles), updates each row's
// running max and sum of exp (a row's scores sit in one 16-lane DPP row),
// rescales its output, stores P = e^(S - m) in LDS (the D layout of S is not
// the A layout P needs) and adds P V.  At the end the four waves' (max, sum,
// output) are merged through LDS.
constexpr int PS = 68;   // LDS row stride (floats) of the K, V and P tiles
constexpr int PKB = 32;  // keys per block (two 16-key S tiles)
constexpr size_t kAttnPrefillLds = sizeof(float) * 4 * (2 * PKB + 16) * PS;

__global__ __launch_bounds__(256) void k_attn_prefill(const float* __restrict__ q,
                                                      const float* __restrict__ kc,
                                                      const float* __restrict__ vc, int layer,
                                                      int Btot, int b0, int H, int t_cap, SeqPos tp, int R,
                                                      float* __restrict__ out) {
    extern __shared__ float asm_lds[];
    const int d = H * 64;
    const int h = blockIdx.y, b = blockIdx.z;
    const int bs = b0 + b, t0 = tp.t[bs];  // sequence in the cache, its first new position
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    float* Kw = asm_lds + wave * (2 * PKB + 16) * PS;  // [PKB][PS]
    float* Vw = Kw + PKB * PS;                          // [PKB][PS]
    float* P = Vw + PKB * PS;                           // [16][PS]
    // row blocks x and nrb - 1 - x: every workgroup does about the same
    // causal work, so one round of workgroups covers the prompt
    const int nrb = (R + 15) / 16;
    for (int pass = 0; pass < 2; ++pass) {
    const int rb = pass == 0 ? (int)blockIdx.x : nrb - 1 - (int)blockIdx.x;
    if (pass == 1 && rb <= (int)blockIdx.x) break;
    if (pass == 1) __syncthreads();  // the first block's merge has read the LDS
    const int i0 = rb * 16;
    // A operand of Q K^T: row i0 + lr; step 4 j + e takes dimension
    // 16 j + 4 lq + e (the same order on the K side), so that a lane's K
    // values for four steps are one 16-byte LDS read
    const int qi = i0 + lr;
    float qa[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = qi < R ? *reinterpret_cast<const float4*>(q + ((size_t)b * R + qi) * d + h * 64 + 16 * j + 4 * lq)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        qa[4 * j] = v.x, qa[4 * j + 1] = v.y, qa[4 * j + 2] = v.z, qa[4 * j + 3] = v.w;
    }
    // rows 4 lq + r of the block (query positions)
    int qpos[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) qpos[r] = t0 + i0 + 4 * lq + r;
    float m[4], l[4];
    f32x4 o[4];  // output tiles: dimensions 16 n + lr
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kmax = t0 + min(i0 + 15, R - 1);  // last key any row of the block sees
    const size_t base = ((size_t)(layer * Btot + bs) * t_cap) * d + h * 64;
    // K and V rows of a block go through registers: the next block of this
    // wave is requested before the current one is multiplied.  Every load is
    // issued (key clamped to kmax) and keys past kmax are zeroed afterwards,
    // so the waits count exactly one block's loads.
    constexpr int NE = PKB * 16 / 64;
    float4 pk[NE], pv[NE];
    auto load_block = [&](int kb) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int idx = lane + 64 * e, t = kb + (idx >> 4), c4 = idx & 15;
            const size_t off = base + (size_t)min(t, kmax) * d + c4 * 4;
            const float4 kv = *reinterpret_cast<const float4*>(kc + off);
            const float4 vv = *reinterpret_cast<const float4*>(vc + off);
            pk[e] = t <= kmax ? kv : make_float4(0.f, 0.f, 0.f, 0.f);
            pv[e] = t <= kmax ? vv : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    load_block(PKB * wave);
    for (int kb = PKB * wave; kb <= kmax; kb += 4 * PKB) {
        // this wave's K and V block (its own tiles: no workgroup barrier)
#pragma unroll
        for (int e = 0; e < NE; ++e) {
            const int idx = lane + 64 * e, kk = idx >> 4, c4 = idx & 15;
            *reinterpret_cast<float4*>(Kw + kk * PS + c4 * 4) = pk[e];
            *reinterpret_cast<float4*>(Vw + kk * PS + c4 * 4) = pv[e];
        }
        // (LDS operations of one wave complete in order: the tiles written
        // above are what the reads below see, with no barrier)
        load_block(kb + 4 * PKB);
        // S tiles n: keys kb + 16 n + lr
        f32x4 sc[2];
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            sc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 kv = *reinterpret_cast<const float4*>(Kw + (16 * n + lr) * PS + 16 * j + 4 * lq);
                sc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * j], kv.x, sc[n], 0, 0, 0);
                sc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * j + 1], kv.y, sc[n], 0, 0, 0);
                sc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * j + 2], kv.z, sc[n], 0, 0, 0);
                sc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[4 * j + 3], kv.w, sc[n], 0, 0, 0);
            }
        }
        // mask, row max over the block (in-lane over n, then the 16-lane row)
        float bm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bm[r] = -INFINITY;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const int key = kb + 16 * n + lr;
                float v = sc[n][r] * 0.125f;
                if (key > qpos[r]) v = -INFINITY;
                sc[n][r] = v;
                bm[r] = fmaxf(bm[r], v);
            }
            bm[r] = row_max16(bm[r]);
        }
        float rs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float mn = fmaxf(m[r], bm[r]);
            const float corr = mn == -INFINITY ? 1.f : expf(m[r] - mn);
            float ps = 0.f;
#pragma unroll
            for (int n = 0; n < 2; ++n) {
                const float p = mn == -INFINITY ? 0.f : expf(sc[n][r] - mn);
                P[(4 * lq + r) * PS + 16 * n + lr] = p;
                ps += p;
            }
            rs[r] = corr;
            l[r] = fmaf(l[r], corr, row_sum16(ps));
            m[r] = mn;
        }
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[n][r] *= rs[r];
        // O += P V (P rows written by this wave only).  Step 4 j + e takes key
        // 16 j + 4 lq + e: one 16-byte read of P per four steps.
#pragma unroll
        for (int j = 0; j < PKB / 16; ++j) {
            const float4 pa = *reinterpret_cast<const float4*>(P + lr * PS + 16 * j + 4 * lq);
            const float pe[4] = {pa.x, pa.y, pa.z, pa.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float* vr = Vw + (16 * j + 4 * lq + e) * PS + lr;
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    o[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(pe[e], vr[16 * n], o[n], 0, 0, 0);
            }
        }
    }
    // merge the four waves: output tiles [wave][16][64], (max, sum) [wave][16]
    __syncthreads();
    float* mo = asm_lds;
    float* ml = asm_lds + 4 * 16 * 64;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) mo[wave * 1024 + (4 * lq + r) * 64 + 16 * n + lr] = o[n][r];
    if (lr == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            ml[(wave * 16 + 4 * lq + r) * 2] = m[r];
            ml[(wave * 16 + 4 * lq + r) * 2 + 1] = l[r];
        }
    }
    __syncthreads();
    const int row = tid >> 4, c = (tid & 15) * 4;
    if (i0 + row < R) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, ml[(w * 16 + row) * 2]);
        float L = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = ml[(w * 16 + row) * 2];
            if (mw == -INFINITY) continue;
            const float e = expf(mw - M);
            L = fmaf(e, ml[(w * 16 + row) * 2 + 1], L);
            const float4 v = *reinterpret_cast<const float4*>(mo + w * 1024 + row * 64 + c);
            acc.x = fmaf(e, v.x, acc.x);
            acc.y = fmaf(e, v.y, acc.y);
            acc.z = fmaf(e, v.z, acc.z);
            acc.w = fmaf(e, v.w, acc.w);
        }
        const float inv = 1.0f / L;
        *reinterpret_cast<float4*>(out + ((size_t)b * R + i0 + row) * d + h * 64 + c) =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
    }
}

// The same attention with 64 query rows per workgroup (wave w: rows
// 16 w .. 16 w + 15) and K/V blocks of 64 keys staged once for all four
// waves.  Used when there are enough row blocks (batched prompts) to fill the
// GPU: it reads each K/V block once per 64 rows instead of once per 16.
__global__ __launch_bounds__(256) void k_attn_prefill_wide(const float* __restrict__ q,
                                                      const float* __restrict__ kc,
                                                      const float* __restrict__ vc, int layer,
                                                      int Btot, int b0, int H, int t_cap, SeqPos tp, int R,
                                                      float* __restrict__ out) {
    __shared__ float Ks[64 * PS];
    __shared__ float Vs[64 * PS];
    __shared__ float Pw[4][16 * PS];
    const int d = H * 64;
    const int i0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
    const int bs = b0 + b, t0 = tp.t[bs];  // sequence in the cache, its first new position
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lq = lane >> 4;
    float* P = Pw[wave];
    // A operand of Q K^T: row i0 + 16 w + lr, dimensions 4 s + lq
    const int qi = i0 + 16 * wave + lr;
    float qa[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) qa[s] = qi < R ? q[((size_t)b * R + qi) * d + h * 64 + 4 * s + lq] : 0.f;
    // rows 4 lq + r of this wave's 16 (query positions)
    int qpos[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) qpos[r] = t0 + i0 + 16 * wave + 4 * lq + r;
    float m[4], l[4];
    f32x4 o[4];  // output tiles: dimensions 16 n + lr
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m[r] = -INFINITY;
        l[r] = 0.f;
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kmax = t0 + min(i0 + 63, R - 1);  // last key any row of the block sees
    const size_t base = ((size_t)(layer * Btot + bs) * t_cap) * d + h * 64;
    for (int kb = 0; kb <= kmax; kb += 64) {
        __syncthreads();  // the previous block's K and V have been used
        for (int e = tid; e < 64 * 16; e += 256) {
            const int kk = e >> 4, c4 = e & 15, t = kb + kk;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (t <= kmax) {
                kv = *reinterpret_cast<const float4*>(kc + base + (size_t)t * d + c4 * 4);
                vv = *reinterpret_cast<const float4*>(vc + base + (size_t)t * d + c4 * 4);
            }
            *reinterpret_cast<float4*>(Ks + kk * PS + c4 * 4) = kv;
            *reinterpret_cast<float4*>(Vs + kk * PS + c4 * 4) = vv;
        }
        __syncthreads();
        // S tiles n: keys kb + 16 n + lr
        f32x4 sc[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
            sc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 16; ++s)
                sc[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[s], Ks[(16 * n + lr) * PS + 4 * s + lq], sc[n], 0, 0, 0);
        }
        // mask, row max over the block (in-lane over n, then the 16-lane row)
        float bm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bm[r] = -INFINITY;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int key = kb + 16 * n + lr;
                float v = sc[n][r] * 0.125f;
                if (key > qpos[r]) v = -INFINITY;
                sc[n][r] = v;
                bm[r] = fmaxf(bm[r], v);
            }
            bm[r] = row_max16(bm[r]);
        }
        float rs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float mn = fmaxf(m[r], bm[r]);
            const float corr = mn == -INFINITY ? 1.f : expf(m[r] - mn);
            float ps = 0.f;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const float p = mn == -INFINITY ? 0.f : expf(sc[n][r] - mn);
                P[(4 * lq + r) * PS + 16 * n + lr] = p;
                ps += p;
            }
            rs[r] = corr;
            l[r] = fmaf(l[r], corr, row_sum16(ps));
            m[r] = mn;
        }
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) o[n][r] *= rs[r];
        // O += P V (P rows written by this wave only: no workgroup barrier)
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll 4
        for (int s = 0; s < 16; ++s) {
            const float pa = P[lr * PS + 4 * s + lq];
#pragma unroll
            for (int n = 0; n < 4; ++n)
                o[n] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, Vs[(4 * s + lq) * PS + 16 * n + lr], o[n], 0, 0, 0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int i = i0 + 16 * wave + 4 * lq + r;
        if (i < R) {
            const float inv = 1.0f / l[r];
#pragma unroll
            for (int n = 0; n < 4; ++n) out[((size_t)b * R + i) * d + h * 64 + 16 * n + lr] = o[n][r] * inv;
        }
    }
}

// ---------------------------------------------------------------- LM head + argmax

// logits[b, v] = z[b] . W[v]; one wave per vocabulary row.
__global__ __launch_bounds__(256) void k_lm_head(const float* __restrict__ z, int B,
                                                 const float* __restrict__ W, int V, int d,
                                                 float* __restrict__ logits) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int v = blockIdx.x * 4 + wave;
    if (v >= V) return;
    const float4* w4 = reinterpret_cast<const float4*>(W + (size_t)v * d);
    const int nf4 = d / 4;
    for (int b0 = 0; b0 < B; b0 += 8) {
        float acc[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = 0.f;
        for (int c = lane; c < nf4; c += 64) {
            const float4 wv = w4[c];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (b0 + k < B) {
                    const float4 zv = reinterpret_cast<const float4*>(z + (size_t)(b0 + k) * d)[c];
                    acc[k] = fmaf(wv.x, zv.x, fmaf(wv.y, zv.y, fmaf(wv.z, zv.z, fmaf(wv.w, zv.w, acc[k]))));
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (b0 + k < B) {
                const float s = wave_sum(acc[k]);
                if (lane == 0) logits[(size_t)(b0 + k) * V + v] = s;
            }
        }
    }
}

// Greedy argmax per sequence; the lowest index wins a tie.
// Argmax over one workgroup's candidates: (best, bi) of each thread, bi =
// INT_MAX when the thread saw no element.  The larger value wins, the lower
// index on equal values; a row of no candidates gives 0.
__device__ int block_argmax256(float best, int bi, float* sv, int* si) {
    const int tid = threadIdx.x;
    sv[tid] = best;
    si[tid] = bi;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            const float ov = sv[tid + o];
            const int oi = si[tid + o];
            if (ov > sv[tid] || (ov == sv[tid] && oi < si[tid])) {
                sv[tid] = ov;
                si[tid] = oi;
            }
        }
        __syncthreads();
    }
    return si[0] == 0x7fffffff ? 0 : si[0];
}

__global__ __launch_bounds__(256) void k_argmax(const float* __restrict__ logits, int V,
                                                int64_t* __restrict__ next) {
    __shared__ float sv[256];
    __shared__ int si[256];
    const int b = blockIdx.x, tid = threadIdx.x;
    const float* lg = logits + (size_t)b * V;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int v = tid; v < V; v += 256) {
        const float x = lg[v];
        if (bi == 0x7fffffff || x > best) {
            best = x;
            bi = v;
        }
    }
    const int r = block_argmax256(best, bi, sv, si);
    if (tid == 0) next[b] = r;
}

// Classifier-free guidance over row pairs (MuScriptor model card: optional
// CFG; the rule is the usual guidance of logits): workgroup i forms
// g = c + (cfg - 1) (c - u) from conditional row i and its unconditional
// partner, row pairs + i, as a binary64 difference, product and sum rounded
// to binary32 (never fused), stores g when `guided` is given, and writes the
// argmax of g to next[i] and, when `token_pair` is given, to both rows of the
// pair there.
__global__ __launch_bounds__(256) void k_cfg_combine(const float* __restrict__ logits, int pairs, int V, float cfg,
                                                     float* __restrict__ guided, int64_t* __restrict__ next,
                                                     int64_t* __restrict__ token_pair) {
#pragma clang fp contract(off)
    __shared__ float sv[256];
    __shared__ int si[256];
    const int i = blockIdx.x, tid = threadIdx.x;
    const float* c = logits + (size_t)i * V;
    const float* u = logits + (size_t)(pairs + i) * V;
    const double w = (double)cfg - 1.0;
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int v = tid; v < V; v += 256) {
        const double cv = (double)c[v];
        const double diff = cv - (double)u[v];
        const double step = w * diff;
        const float g = (float)(cv + step);
        if (guided) guided[(size_t)i * V + v] = g;
        if (bi == 0x7fffffff || g > best) {
            best = g;
            bi = v;
        }
    }
    const int r = block_argmax256(best, bi, sv, si);
    if (tid == 0) {
        next[i] = r;
        if (token_pair) {
            token_pair[i] = r;
            token_pair[pairs + i] = r;
        }
    }
}

// ---------------------------------------------------------------- debug dequant

__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                 int N, int K, float* __restrict__ out) {
    const size_t nbytes = (size_t)N * K / 2;
    for (size_t j = blockIdx.x * (size_t)blockDim.x + threadIdx.x; j < nbytes;
         j += (size_t)gridDim.x * blockDim.x) {
        const unsigned byte = q[j];
        const size_t k0 = 2 * j;
        const size_t n = k0 / K, k = k0 % K;
        const float sc = s[n * (K / 32) + k / 32];
        out[k0] = (float)((int)(byte & 15u) - 8) * sc;
        out[k0 + 1] = (float)((int)(byte >> 4) - 8) * sc;
    }
}

// GEMV tiling of a projection (see k_gemv_w4): unit (t, g, l) for row block
// t, group g and lane l = 16 kq + r holds row 16 t + r's piece kq of group g:
// INT4 its dword kq (8 nibbles) with the scale in a [t][g][16] array, half
// its 8 values 8 kq .. 8 kq + 7 (16 B), float its 8 values as two 16-byte
// units (the first four at unit l, the rest at unit 64 + l).  Rows past N
// are zero (INT4: nibbles 8, scale 0).  One thread per 4-byte word of the
// tiled copy.
__global__ __launch_bounds__(256) void k_tile_weights(const uint8_t* __restrict__ q, const float* __restrict__ s,
                                                      int N, int K, int fmt, uint32_t* __restrict__ qt,
                                                      float* __restrict__ st, size_t nwords) {
    const int G = K / 32;
    const int wpu = fmt == WF_INT4 ? 1 : 4;             // words per 16-byte or 4-byte unit
    const int upt = fmt == WF_F32 ? 128 : 64;           // units per (row block, group)
    for (size_t j = blockIdx.x * (size_t)blockDim.x + threadIdx.x; j < nwords; j += (size_t)gridDim.x * blockDim.x) {
        const size_t unit = j / wpu;
        const int w = (int)(j % wpu);
        const size_t tg = unit / upt;
        const int u = (int)(unit % upt);
        const int l = u & 63, half = u >> 6;            // half: second 16 bytes of a float piece
        const int t = (int)(tg / G), g = (int)(tg % G);
        const int r = l & 15, kq = l >> 4;
        const int row = 16 * t + r;
        uint32_t v;
        if (fmt == WF_INT4) {
            v = row < N ? *reinterpret_cast<const uint32_t*>(q + (size_t)row * (K / 2) + (size_t)g * 16 + 4 * kq)
                        : 0x88888888u;
            if (kq == 0) st[tg * 16 + r] = row < N ? s[(size_t)row * G + g] : 0.f;
        } else {
            const int esz = fmt == WF_F16 ? 2 : 4;
            const size_t col = (size_t)g * 32 + 8 * kq + (size_t)half * 4;  // first column of the unit
            v = row < N ? *reinterpret_cast<const uint32_t*>(q + ((size_t)row * K + col) * esz + 4 * w) : 0u;
        }
        qt[j] = v;
    }
}

size_t tiled_weight_bytes(const Int4Mat& w) {
    const size_t rows = (size_t)(w.N + 15) / 16 * 16;
    return rows * w.K * (w.fmt == WF_INT4 ? 1 : w.fmt == WF_F16 ? 4 : 8) / 2;
}
size_t tiled_scale_floats(const Int4Mat& w) {
    return w.fmt == WF_INT4 ? (size_t)(w.N + 15) / 16 * 16 * (w.K / 32) : 0;
}

hipError_t launch_tile_weights(const Int4Mat& w, uint8_t* qt, float* st, hipStream_t st_) {
    if (w.K % 32) return hipErrorInvalidValue;
    const size_t nwords = tiled_weight_bytes(w) / 4;
    const int grid = (int)std::min<size_t>((nwords + 255) / 256, 65536);
    hipLaunchKernelGGL(k_tile_weights, dim3(grid), dim3(256), 0, st_, w.q, w.s, w.N, w.K, w.fmt,
                       reinterpret_cast<uint32_t*>(qt), st, nwords);
    return hipGetLastError();
}

// Dense weights as float (half widened exactly).
__global__ __launch_bounds__(256) void k_widen(const uint8_t* __restrict__ q, bool half, size_t n,
                                               float* __restrict__ out) {
    for (size_t j = blockIdx.x * (size_t)blockDim.x + threadIdx.x; j < n; j += (size_t)gridDim.x * blockDim.x)
        out[j] = half ? __half2float(reinterpret_cast<const __half*>(q)[j]) : reinterpret_cast<const float*>(q)[j];
}

// ---------------------------------------------------------------- launchers

hipError_t launch_embed(const int64_t* tokens, int S, const float* prefix, int P, const float* emb,
                        int V, int d, int B, float* x, int* err, hipStream_t st) {
    hipLaunchKernelGGL(k_embed, dim3(B * (P + S)), dim3(256), 0, st, tokens, S, prefix, P, emb, V, d,
                       x, err);
    return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, long ldx, const float* g, const float* b, float eps,
                            int d, int rows, float* y, long ldy, hipStream_t st) {
    if (d > 8 * 256) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_layernorm, dim3(rows), dim3(256), 0, st, x, ldx, g, b, eps, d, y, ldy);
    return hipGetLastError();
}

int splitk_plan(int M, const Int4Mat& w) {
    // INT4 weights, 64 x 64 tiles: split K where the unsplit grid would
    // leave CUs idle, up to 4 ways (at least 256 columns of K each)
    if (w.fmt != WF_INT4 || w.N % 4 || w.N > 8 * 256) return 1;  // k_splitk_add holds a row in 8 per thread
    const long tiles = (long)((M + 63) / 64) * ((w.N + 63) / 64);
    if (tiles >= 256) return 1;
    for (int c = 4; c >= 2; --c)
        if (tiles * c <= 1024 && w.K % (64 * c) == 0 && w.K / c >= 256) return c;
    return 1;
}

hipError_t launch_w4_gemm_splitk(const float* x, int ldx, int M, const Int4Mat& w, float* y, int ldy, float* part,
                                 int nsplit, hipStream_t st, const float* ln_g, const float* ln_b, float eps,
                                 float* a, int lda) {
    if (w.fmt != WF_INT4 || nsplit < 1 || w.K % (64 * nsplit) || w.N > 8 * 256) return hipErrorInvalidValue;
    EpiArgs ep{};
    ep.epi = EPI_RESID;
    ep.part = part;
    const dim3 grid((w.N + 63) / 64, (M + 63) / 64, nsplit);
    hipLaunchKernelGGL((k_gemm_w4_bf3<64, 64, 64>), grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y, ldy, ep,
                       w.K / nsplit);
    hipLaunchKernelGGL(k_splitk_add, dim3(M), dim3(256), 0, st, y, ldy, part, nsplit, M, w.N, ln_g, ln_b, eps, a,
                       lda);
    return hipGetLastError();
}

constexpr size_t kGemvMaxLds = 152 * 1024;  // dynamic LDS of the GEMV (static: 4.3 KB)

struct GemvArgs {
    const float* x;
    int ldx, M, K, kspan;
    const float *ln_g, *ln_b;
    float eps;
    const float* part;
    int H, ns;
    const uint8_t* q;
    const float* s;
    int N;
    float* y;
    int ldy;
    EpiArgs ep;
};

template <int WF, bool A8, int SRC>
static hipError_t gemv_set_lds_src() {
    const void* fns[4] = {(const void*)k_gemv_w4<WF, A8, 4, SRC>, (const void*)k_gemv_w4<WF, A8, 8, SRC>,
                          (const void*)k_gemv_w4<WF, A8, 12, SRC>, (const void*)k_gemv_w4<WF, A8, 16, SRC>};
    for (const void* f : fns) {
        const hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kGemvMaxLds);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int WF, bool A8>
static hipError_t gemv_set_lds() {
    hipError_t e = gemv_set_lds_src<WF, A8, GS_ROWS>();
    if (e == hipSuccess) e = gemv_set_lds_src<WF, A8, GS_LN>();
    if (e == hipSuccess) e = gemv_set_lds_src<WF, A8, GS_PARTS>();
    return e;
}

template <int WF, bool A8, int SRC>
static void gemv_launch_src(int ng, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
#define MT_GEMV(NGV)                                                                                                 \
    hipLaunchKernelGGL((k_gemv_w4<WF, A8, NGV, SRC>), grid, dim3(256), lds, st, a.x, a.ldx, a.M, a.K, a.kspan, a.ln_g, \
                       a.ln_b, a.eps, a.part, a.H, a.ns, a.q, a.s, a.N, a.y, a.ldy, a.ep)
    switch (ng) {
        case 4: MT_GEMV(4); break;
        case 8: MT_GEMV(8); break;
        case 12: MT_GEMV(12); break;
        default: MT_GEMV(16); break;
    }
#undef MT_GEMV
}

template <int WF, bool A8>
static void gemv_launch(int ng, dim3 grid, size_t lds, hipStream_t st, const GemvArgs& a) {
    if (a.part) gemv_launch_src<WF, A8, GS_PARTS>(ng, grid, lds, st, a);
    else if (a.ln_g) gemv_launch_src<WF, A8, GS_LN>(ng, grid, lds, st, a);
    else gemv_launch_src<WF, A8, GS_ROWS>(ng, grid, lds, st, a);
}

// GEMV plan: k split (grid.y) and columns per split.  The += epilogue
// splits K so that about 256 workgroups run; the other epilogues keep one
// split per output block.
static void plan_gemv(int N, int K, Epilogue epi, int granule, int* ksplit, int* kspan) {
    const int G = K / granule, nblk = (N + 15) / 16;
    int want = epi == EPI_RESID ? std::max(1, 256 / nblk) : 1;
    want = std::max(want, epi == EPI_RESID ? (K + GV_MAXSPAN - 1) / GV_MAXSPAN : 1);
    int ks = 1;
    for (int c = std::min(want, G); c >= 1; --c)
        if (G % c == 0) {
            ks = c;
            break;
        }
    *ksplit = ks;
    *kspan = K / ks;
}

hipError_t launch_w4_matmul(const float* x, int ldx, int M, const Int4Mat& w, const float* ln_g,
                            const float* ln_b, float eps, float* y, int ldy, Epilogue epi, const QkvDest* qkv,
                            bool force_gemm, hipStream_t st, const AttnParts* parts, bool a8) {
    if (a8 && w.fmt != WF_INT4) return hipErrorInvalidValue;  // A8 codes pair with nibbles only
    const AttnParts ap = parts ? *parts : AttnParts{nullptr, 0, 0};
    EpiArgs ep{};
    ep.epi = epi;
    if (qkv) ep.qkv = *qkv;
    const int per = (epi == EPI_QKV && qkv) ? qkv->rows_per_seq : 1;
    if (!force_gemm && gemv_takes_rows(M, per)) {
        if (ln_g && w.K > GV_MAXSPAN) return hipErrorInvalidValue;
        if (ap.part && (ln_g || ap.H * 64 != w.K)) return hipErrorInvalidValue;
        // rows in slices of whole sequences, at most GV_M rows each; every
        // slice is one launch (the weights it re-reads come from the caches)
        const int slice = GV_M / per * per;
        const int ms0 = std::min(M, slice);
        int ksplit, kspan;
        // merged partials: whole heads (64 columns) per k split
        plan_gemv(w.N, w.K, ln_g ? EPI_STORE : epi, ap.part ? 64 : 32, &ksplit, &kspan);
        // activation rows (stride span + 4); merged partials also need their
        // weights [rows][heads][splits]; the A8 form adds the INT8 codes
        // [GV_M][span] and their scales [span / 32][GV_M]
        const int span = std::min(kspan, GV_MAXSPAN);
        const size_t wts = ap.part ? (size_t)ms0 * (span / 64) * ap.nsplit : 0;
        if (ap.part && (span % 64 || (int)(ms0 * (span / 64)) > 256)) return hipErrorInvalidValue;
        size_t lds = sizeof(float) * ((size_t)(span + 4) * GV_M + wts);
        if (a8) lds = sizeof(float) * ((size_t)(span + 4) * GV_M + ((wts + 3) & ~(size_t)3)) + (size_t)GV_M * span +
                      sizeof(float) * (size_t)(span / 32) * GV_M;
        if (ln_g) lds = std::max(lds, sizeof(float) * ((size_t)(span + 4) * GV_M + 2 * (size_t)span));
        if (lds > kGemvMaxLds) return hipErrorInvalidValue;
        // groups per wave and chunk, rounded up to a multiple of 4
        const int ng = std::min(16, ((span / 32 + 3) / 4 + 3) / 4 * 4);
        static bool attr = false;
        if (!attr) {
            hipError_t e = gemv_set_lds<WF_INT4, false>();
            if (e == hipSuccess) e = gemv_set_lds<WF_INT4, true>();
            if (e == hipSuccess) e = gemv_set_lds<WF_F16, false>();
            if (e == hipSuccess) e = gemv_set_lds<WF_F32, false>();
            if (e != hipSuccess) return e;
            attr = true;
        }
        const dim3 grid((w.N + 15) / 16, ksplit);
        if (!w.qt || (w.fmt == WF_INT4 && !w.st)) return hipErrorInvalidValue;  // needs the GEMV tiling
        for (int r0 = 0; r0 < M; r0 += slice) {
            const int ms = std::min(slice, M - r0);
            EpiArgs es = ep;
            if (epi == EPI_QKV) {
                es.qkv.q += (size_t)r0 * es.qkv.d;
                es.qkv.b0 += r0 / per;
            }
            const float* xs = x ? x + (size_t)r0 * ldx : nullptr;
            float* ys = y ? y + (size_t)r0 * ldy : nullptr;
            const float* ps = ap.part ? ap.part + (size_t)r0 * ap.H * ap.nsplit * PART : nullptr;
            const GemvArgs ga{xs, ldx, ms, w.K, kspan, ln_g, ln_b, eps, ps, ap.H, ap.nsplit, w.qt, w.st, w.N, ys, ldy, es};
            if (w.fmt == WF_F16) gemv_launch<WF_F16, false>(ng, grid, lds, st, ga);
            else if (w.fmt == WF_F32) gemv_launch<WF_F32, false>(ng, grid, lds, st, ga);
            else if (a8) gemv_launch<WF_INT4, true>(ng, grid, lds, st, ga);
            else gemv_launch<WF_INT4, false>(ng, grid, lds, st, ga);
        }
        return hipGetLastError();
    }
    if (ln_g || ap.part) return hipErrorInvalidValue;  // the GEMM path takes plain rows
    // 32-row tiles when 64-row tiles would give fewer than two workgroups
    // per CU.  One workgroup per tile over all of K, so that results do not
    // depend on the order of atomic additions (prefill is bit-reproducible),
    // except with fewer than 128 tiles on a += epilogue (the O and FFN-down
    // projections of a decode batch): then K is split over up to 8
    // workgroups per tile and their products are added atomically, as the
    // GEMV does.
    const int ntile = (w.N + GN - 1) / GN;
    const bool small = (long)ntile * ((M + 63) / 64) < 512;
    const int TM = small ? 32 : 64, GKs = small ? 128 : 64;
    const int mtile = (M + TM - 1) / TM;
    const int stages = (w.K + GKs - 1) / GKs;
    int ksplit = 1;
    if (epi == EPI_RESID && (long)ntile * mtile < 128) {
        const int want = std::min(8, std::max(1, 256 / (ntile * mtile)));
        for (int c = std::min(want, stages); c >= 1; --c)
            if (stages % c == 0) {
                ksplit = c;
                break;
            }
    }
    const dim3 grid(ntile, mtile, ksplit);
    if (a8 && w.fmt == WF_INT4) {
        if (small)
            hipLaunchKernelGGL((k_gemm_w4a8<32, 128>), grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y, ldy,
                               ep, stages / ksplit * GKs);
        else
            hipLaunchKernelGGL((k_gemm_w4a8<64, 64>), grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y, ldy,
                               ep, stages / ksplit * GKs);
        return hipGetLastError();
    }
    const int kspan = stages / ksplit * GKs;
    if (w.fmt == WF_INT4) {
        // 32-column tiles where 64-column ones would leave fewer than two
        // workgroups per CU (the K range stays whole: no atomics)
        if (small && ksplit == 1 && (long)ntile * mtile < 512) {
            const dim3 g32((w.N + 31) / 32, mtile, 1);
            hipLaunchKernelGGL((k_gemm_w4_bf3<32, 128, 32>), g32, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y,
                               ldy, ep, kspan);
        } else if (small) {
            hipLaunchKernelGGL((k_gemm_w4_bf3<32, 128, 64>), grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y,
                               ldy, ep, kspan);
        } else {
            hipLaunchKernelGGL((k_gemm_w4_bf3<64, 64, 64>), grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y,
                               ldy, ep, kspan);
        }
        return hipGetLastError();
    }
    static bool attr = false;
    if (!attr) {
        const void* f64[3] = {(const void*)k_gemm_w4<64, 64, WF_INT4>, (const void*)k_gemm_w4<64, 64, WF_F16>,
                              (const void*)k_gemm_w4<64, 64, WF_F32>};
        const void* f32[3] = {(const void*)k_gemm_w4<32, 128, WF_INT4>, (const void*)k_gemm_w4<32, 128, WF_F16>,
                              (const void*)k_gemm_w4<32, 128, WF_F32>};
        for (int i = 0; i < 3; ++i) {
            hipError_t e = hipFuncSetAttribute(f64[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemm_lds(64, 64));
            if (e == hipSuccess)
                e = hipFuncSetAttribute(f32[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)gemm_lds(32, 128));
            if (e != hipSuccess) return e;
        }
        attr = true;
    }
#define MT_GEMM(TMV, GKV, WFV)                                                                                   \
    hipLaunchKernelGGL((k_gemm_w4<TMV, GKV, WFV>), grid, dim3(256), gemm_lds(TMV, GKV), st, x, ldx, M, w.K, w.q, \
                       w.s, w.N, y, ldy, ep, kspan)
    if (small) {
        if (w.fmt == WF_F16) MT_GEMM(32, 128, WF_F16);
        else if (w.fmt == WF_F32) MT_GEMM(32, 128, WF_F32);
        else MT_GEMM(32, 128, WF_INT4);
    } else {
        if (w.fmt == WF_F16) MT_GEMM(64, 64, WF_F16);
        else if (w.fmt == WF_F32) MT_GEMM(64, 64, WF_F32);
        else MT_GEMM(64, 64, WF_INT4);
    }
#undef MT_GEMM
    return hipGetLastError();
}

bool gemv_takes_rows(int M, int rows_per_seq) {
    return M >= 1 && M <= kGemvRowsMax && rows_per_seq >= 1 && rows_per_seq <= GV_M;
}
bool gemv_fuses_layernorm(int M, int K) { return gemv_takes_rows(M, 1) && K <= GV_MAXSPAN; }

hipError_t launch_attn_decode(const float* q, const float* kc, const float* vc, int layer, int B,
                              int H, int t_cap, const SeqPos& T, float* part, int nsplit, int chunk,
                              hipStream_t st) {
    if (B > kMaxBatch || chunk > 256) return hipErrorInvalidValue;
    for (int b = 0; b < B; ++b)
        if (T.t[b] < 1 || T.t[b] > t_cap || nsplit * chunk < T.t[b]) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_decode, dim3(nsplit, H, B), dim3(256), 0, st, q, kc, vc, layer, B, H,
                       t_cap, T, chunk, part);
    return hipGetLastError();
}

hipError_t launch_attn_prefill(const float* q, const float* kc, const float* vc, int layer, int Btot, int b0,
                               int nb, int H, int t_cap, const SeqPos& t0, int R, float* out, hipStream_t st) {
    if (b0 < 0 || nb < 1 || b0 + nb > Btot || Btot > kMaxBatch) return hipErrorInvalidValue;
    for (int b = b0; b < b0 + nb; ++b)
        if (t0.t[b] < 0 || t0.t[b] + R > t_cap) return hipErrorInvalidValue;
    if ((long)((R + 63) / 64) * H * nb >= 512) {
        hipLaunchKernelGGL(k_attn_prefill_wide, dim3((R + 63) / 64, H, nb), dim3(256), 0, st, q, kc, vc, layer, Btot,
                           b0, H, t_cap, t0, R, out);
        return hipGetLastError();
    }
    static bool attr = false;
    if (!attr) {
        hipError_t e = hipFuncSetAttribute((const void*)k_attn_prefill, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kAttnPrefillLds);
        if (e != hipSuccess) return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_attn_prefill, dim3(((R + 15) / 16 + 1) / 2, H, nb), dim3(256), kAttnPrefillLds, st, q, kc, vc,
                       layer, Btot, b0, H, t_cap, t0, R, out);
    return hipGetLastError();
}

hipError_t launch_lm_head(const float* z, int B, const float* w, int V, int d, float* logits,
                          hipStream_t st) {
    if (d % 4) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_lm_head, dim3((V + 3) / 4), dim3(256), 0, st, z, B, w, V, d, logits);
    return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int B, int V, int64_t* next, hipStream_t st) {
    hipLaunchKernelGGL(k_argmax, dim3(B), dim3(256), 0, st, logits, V, next);
    return hipGetLastError();
}

hipError_t launch_attn_merge(const float* part, int B, int H, int nsplit, float* out, hipStream_t st) {
    if (B < 1 || H < 1 || nsplit < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_attn_merge, dim3(H, B), dim3(64), 0, st, part, H, nsplit, out);
    return hipGetLastError();
}

hipError_t launch_cfg_combine(const float* logits, int pairs, int V, float cfg, float* guided, int64_t* next,
                              int64_t* token_pair, hipStream_t st) {
    hipLaunchKernelGGL(k_cfg_combine, dim3(pairs), dim3(256), 0, st, logits, pairs, V, cfg, guided, next, token_pair);
    return hipGetLastError();
}

hipError_t launch_dequant(const Int4Mat& w, float* out, hipStream_t st) {
    if (w.fmt != WF_INT4) {
        const size_t n = (size_t)w.N * w.K;
        const int grid = (int)((n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536);
        hipLaunchKernelGGL(k_widen, dim3(grid), dim3(256), 0, st, w.q, w.fmt == WF_F16, n, out);
        return hipGetLastError();
    }
    const size_t nbytes = (size_t)w.N * w.K / 2;
    const int grid = (int)((nbytes + 255) / 256 < 65536 ? (nbytes + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(256), 0, st, w.q, w.s, w.N, w.K, out);
    return hipGetLastError();
}

}  // namespace mt
