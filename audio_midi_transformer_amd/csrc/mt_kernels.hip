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
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "mt_internal.h"

namespace mt {

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752440f));
}

// Dot product of one 32-weight group with 32 activations.
// Byte j of the group holds input 2j in its low nibble and 2j+1 in its high
// nibble; the stored nibble is code + 8.  Returns sum_k (u_k - 8) * x_k,
// evaluated as sum_k u_k x_k - 8 sum_k x_k.
__device__ __forceinline__ float group_dot(uint4 w, const float* __restrict__ x) {
    const float4* x4 = reinterpret_cast<const float4*>(x);
    const unsigned wd[4] = {w.x, w.y, w.z, w.w};
    float acc = 0.f, xs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 xa = x4[2 * j], xb = x4[2 * j + 1];
        const unsigned lo = wd[j] & 0x0F0F0F0Fu;
        const unsigned hi = (wd[j] >> 4) & 0x0F0F0F0Fu;
        acc = fmaf((float)(lo & 0xFFu), xa.x, acc);
        acc = fmaf((float)(hi & 0xFFu), xa.y, acc);
        acc = fmaf((float)((lo >> 8) & 0xFFu), xa.z, acc);
        acc = fmaf((float)((hi >> 8) & 0xFFu), xa.w, acc);
        acc = fmaf((float)((lo >> 16) & 0xFFu), xb.x, acc);
        acc = fmaf((float)((hi >> 16) & 0xFFu), xb.y, acc);
        acc = fmaf((float)(lo >> 24), xb.z, acc);
        acc = fmaf((float)(hi >> 24), xb.w, acc);
        xs += ((xa.x + xa.y) + (xa.z + xa.w)) + ((xb.x + xb.y) + (xb.z + xb.w));
    }
    return fmaf(-8.f, xs, acc);
}

struct EpiArgs {
    Epilogue epi;
    QkvDest qkv;
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
                const int b = m / q.rows_per_seq, i = m % q.rows_per_seq;
                const size_t slot = ((size_t)(q.layer * q.batch + b) * q.t_cap + q.t0 + i) * q.d;
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

// ---------------------------------------------------------------- INT4 GEMV (M <= 8)

// Lane group of LPR lanes owns one output row; lane r of the group holds
// groups r, r + LPR, ... (cpl of them) of that row.  The group dot products
// are summed over the LPR lanes with cross-lane adds.
template <int LPR>
__global__ __launch_bounds__(256) void k_gemv_w4(const float* __restrict__ X, int ldx, int M, int K,
                                                 const uint8_t* __restrict__ Wq,
                                                 const float* __restrict__ Ws, int N, int cpl,
                                                 float* __restrict__ Y, int ldy, EpiArgs ep) {
    constexpr int RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int sub = lane / LPR, lr = lane % LPR;
    const int row = (blockIdx.x * 4 + wave) * RPW + sub;
    const bool valid = row < N;
    const int G = K / 32;
    uint4 w[4];
    float s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        w[j] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        s[j] = 0.f;
        const int c = lr + LPR * j;
        if (valid && j < cpl) {
            w[j] = *reinterpret_cast<const uint4*>(Wq + (size_t)row * (K / 2) + (size_t)c * 16);
            s[j] = Ws[(size_t)row * G + c];
        }
    }
    for (int m = 0; m < M; ++m) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (j < cpl) {
                const int c = lr + LPR * j;
                acc = fmaf(s[j], group_dot(w[j], X + (size_t)m * ldx + (size_t)c * 32), acc);
            }
        }
        acc = group_sum<LPR>(acc);
        if (valid && lr == 0) epilogue(ep, Y, ldy, m, row, acc);
    }
}

// ---------------------------------------------------------------- INT4 GEMM (FP32 MFMA)

// Y[M, N] = X[M, K] . W'^T with W' = (u - 8) * s dequantised exactly into LDS.
// Tile 64 x 64 per workgroup, K step 32 (one quantisation group); four waves
// as 2 x 2, each a 32 x 32 sub-tile of 2 x 2 v_mfma_f32_16x16x4f32 blocks.
// Operand layout of that instruction: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; it receives D[4 (l / 16) + r][l % 16], r = 0..3.
constexpr int GT = 64;
constexpr int GS = 34;  // LDS row stride in floats (conflict-free column reads)

__global__ __launch_bounds__(256) void k_gemm_w4(const float* __restrict__ X, int ldx, int M, int K,
                                                 const uint8_t* __restrict__ Wq,
                                                 const float* __restrict__ Ws, int N,
                                                 float* __restrict__ Y, int ldy, EpiArgs ep) {
    __shared__ float As[GT * GS];
    __shared__ float Bs[GT * GS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
    const int G = K / 32;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // A tile load: 64 rows x 32 floats = 512 float4, two per thread.
    // W tile load: 64 rows x 4 dwords of nibbles, one dword (8 weights) per thread.
    const int wr = tid >> 2, wdw = tid & 3;
    for (int g = 0; g < G; ++g) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = tid + e * 256;
            const int r = idx >> 3, c4 = idx & 7;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (m0 + r < M) v = *reinterpret_cast<const float4*>(X + (size_t)(m0 + r) * ldx + g * 32 + c4 * 4);
            float* dst = As + r * GS + c4 * 4;
            *reinterpret_cast<float2*>(dst) = make_float2(v.x, v.y);
            *reinterpret_cast<float2*>(dst + 2) = make_float2(v.z, v.w);
        }
        {
            float* dst = Bs + wr * GS + wdw * 8;
            if (n0 + wr < N) {
                const unsigned word = *reinterpret_cast<const unsigned*>(
                    Wq + (size_t)(n0 + wr) * (K / 2) + (size_t)g * 16 + wdw * 4);
                const float sc = Ws[(size_t)(n0 + wr) * G + g];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const unsigned byte = (word >> (8 * b)) & 0xFFu;
                    const float lo = (float)((int)(byte & 15u) - 8) * sc;
                    const float hi = (float)((int)(byte >> 4) - 8) * sc;
                    *reinterpret_cast<float2*>(dst + 2 * b) = make_float2(lo, hi);
                }
            } else {
#pragma unroll
                for (int b = 0; b < 4; ++b) *reinterpret_cast<float2*>(dst + 2 * b) = make_float2(0.f, 0.f);
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int k = kk * 4 + (lane >> 4);
            float a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = As[(wm * 32 + i * 16 + (lane & 15)) * GS + k];
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = Bs[(wn * 32 + j * 16 + (lane & 15)) * GS + k];
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = m0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
                const int n = n0 + wn * 32 + j * 16 + (lane & 15);
                if (m < M && n < N) epilogue(ep, Y, ldy, m, n, acc[i][j][r]);
            }
}

// ---------------------------------------------------------------- decode attention

// Split-K decode attention.  Workgroup (split, h, b) covers positions
// [split * chunk, min(T, (split + 1) * chunk)) of head h of sequence b and
// writes the unnormalised partial (max score, sum of exp, sum of exp * V).
// 16 lane groups of 16 lanes; a group handles one position at a time, each
// lane 4 of the 64 dimensions.
constexpr int PART = 68;  // floats per partial: m, l, acc[64], pad

__global__ __launch_bounds__(256) void k_attn_decode(const float* __restrict__ q,
                                                     const float* __restrict__ kc,
                                                     const float* __restrict__ vc, int layer,
                                                     int B, int H, int t_cap, int T, int chunk,
                                                     float* __restrict__ part) {
    __shared__ float sm[16], sl[16];
    __shared__ float sacc[16][64];
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int d = H * 64;
    const int tid = threadIdx.x, g = tid >> 4, ql = tid & 15;
    const float4 q4 = *reinterpret_cast<const float4*>(q + (size_t)b * d + h * 64 + ql * 4);
    const size_t base = ((size_t)(layer * B + b) * t_cap) * d + h * 64 + ql * 4;
    const int t_begin = split * chunk;
    const int t_end = min(T, t_begin + chunk);
    float m = -INFINITY, l = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int t = t_begin + g; t < t_end; t += 16) {
        const float4 k4 = *reinterpret_cast<const float4*>(kc + base + (size_t)t * d);
        const float4 v4 = *reinterpret_cast<const float4*>(vc + base + (size_t)t * d);
        float s = q4.x * k4.x + q4.y * k4.y + q4.z * k4.z + q4.w * k4.w;
        s = group_sum<16>(s) * 0.125f;
        const float mn = fmaxf(m, s);
        const float corr = expf(m - mn);
        const float p = expf(s - mn);
        l = fmaf(l, corr, p);
        acc.x = fmaf(acc.x, corr, p * v4.x);
        acc.y = fmaf(acc.y, corr, p * v4.y);
        acc.z = fmaf(acc.z, corr, p * v4.z);
        acc.w = fmaf(acc.w, corr, p * v4.w);
        m = mn;
    }
    if (ql == 0) {
        sm[g] = m;
        sl[g] = l;
    }
    sacc[g][ql * 4 + 0] = acc.x;
    sacc[g][ql * 4 + 1] = acc.y;
    sacc[g][ql * 4 + 2] = acc.z;
    sacc[g][ql * 4 + 3] = acc.w;
    __syncthreads();
    if (tid < 64) {
        float M = -INFINITY;
        for (int i = 0; i < 16; ++i) M = fmaxf(M, sm[i]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
            for (int i = 0; i < 16; ++i) {
                if (sm[i] == -INFINITY) continue;
                const float w = expf(sm[i] - M);
                L = fmaf(w, sl[i], L);
                A = fmaf(w, sacc[i][tid], A);
            }
        }
        float* out = part + ((size_t)(b * H + h) * gridDim.x + split) * PART;
        if (tid == 0) {
            out[0] = M;
            out[1] = L;
        }
        out[2 + tid] = A;
    }
}

// Merge the splits of one (b, h): out = sum_s e^(m_s - M) acc_s / sum_s e^(m_s - M) l_s.
__global__ __launch_bounds__(64) void k_attn_merge(const float* __restrict__ part, int nsplit, int H,
                                                   float* __restrict__ out) {
    const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
    const float* p = part + (size_t)(b * H + h) * nsplit * PART;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, p[s * PART]);
    float L = 0.f, A = 0.f;
    for (int s = 0; s < nsplit; ++s) {
        const float ms = p[s * PART];
        if (ms == -INFINITY) continue;
        const float w = expf(ms - M);
        L = fmaf(w, p[s * PART + 1], L);
        A = fmaf(w, p[s * PART + 2 + j], A);
    }
    out[(size_t)b * H * 64 + h * 64 + j] = A / L;
}

// ---------------------------------------------------------------- prefill attention

// Causal attention of R new rows per sequence (positions t0 .. t0+R-1) over
// the cache.  Workgroup (row block, h, b) handles 64 query rows; wave w rows
// 16w .. 16w+15; four lanes per row, each 16 of the 64 dimensions.  Keys
// and values are staged through LDS 64 positions at a time.
__global__ __launch_bounds__(256) void k_attn_prefill(const float* __restrict__ q,
                                                      const float* __restrict__ kc,
                                                      const float* __restrict__ vc, int layer,
                                                      int B, int H, int t_cap, int t0, int R,
                                                      float* __restrict__ out) {
    __shared__ float Ks[64 * 68];
    __shared__ float Vs[64 * 68];
    const int d = H * 64;
    const int i0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int r = lane >> 2, qd = lane & 3;
    const int i = i0 + wave * 16 + r;
    const bool valid = i < R;
    const int p = t0 + i;
    float qv[16], acc[16];
    const float* qrow = q + ((size_t)b * R + (valid ? i : 0)) * d + h * 64 + qd * 16;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        qv[j] = valid ? qrow[j] : 0.f;
        acc[j] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int kmax = t0 + min(i0 + 63, R - 1);
    const size_t base = ((size_t)(layer * B + b) * t_cap) * d + h * 64;
    for (int kb = 0; kb <= kmax; kb += 64) {
        __syncthreads();
        for (int e = tid; e < 64 * 16; e += 256) {
            const int kk = e >> 4, c4 = e & 15, t = kb + kk;
            float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
            if (t <= kmax) {
                kv = *reinterpret_cast<const float4*>(kc + base + (size_t)t * d + c4 * 4);
                vv = *reinterpret_cast<const float4*>(vc + base + (size_t)t * d + c4 * 4);
            }
            *reinterpret_cast<float4*>(Ks + kk * 68 + c4 * 4) = kv;
            *reinterpret_cast<float4*>(Vs + kk * 68 + c4 * 4) = vv;
        }
        __syncthreads();
        const int nk = p - kb + 1;  // keys of this block visible to row i
        for (int kk = 0; kk < 64; ++kk) {
            const float* kr = Ks + kk * 68 + qd * 16;
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) s = fmaf(qv[j], kr[j], s);
            s = group_sum<4>(s) * 0.125f;
            if (valid && kk < nk) {
                const float mn = fmaxf(m, s);
                const float corr = expf(m - mn);
                const float pe = expf(s - mn);
                l = fmaf(l, corr, pe);
                const float* vr = Vs + kk * 68 + qd * 16;
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[j] = fmaf(acc[j], corr, pe * vr[j]);
                m = mn;
            }
        }
    }
    if (valid) {
        float* o = out + ((size_t)b * R + i) * d + h * 64 + qd * 16;
        const float inv = 1.0f / l;
#pragma unroll
        for (int j = 0; j < 16; ++j) o[j] = acc[j] * inv;
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
        if (x > best || bi == 0x7fffffff) {
            if (bi == 0x7fffffff || x > best) {
                best = x;
                bi = v;
            }
        }
    }
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
    if (tid == 0) next[b] = si[0] == 0x7fffffff ? 0 : si[0];
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

static bool pick_gemv(int K, int* lpr, int* cpl) {
    const int G = K / 32;
    for (int c = 1; c <= 4; ++c) {
        if (G % c) continue;
        const int l = G / c;
        if (l > 64 || (l & (l - 1))) continue;
        *lpr = l;
        *cpl = c;
        return true;
    }
    return false;
}

hipError_t launch_w4_matmul(const float* x, int ldx, int M, const Int4Mat& w, float* y, int ldy,
                            Epilogue epi, const QkvDest* qkv, bool force_gemm, hipStream_t st) {
    EpiArgs ep{};
    ep.epi = epi;
    if (qkv) ep.qkv = *qkv;
    int lpr = 0, cpl = 0;
    if (!force_gemm && M <= 8 && pick_gemv(w.K, &lpr, &cpl)) {
        const int rows_per_block = 4 * (64 / lpr);
        const dim3 grid((w.N + rows_per_block - 1) / rows_per_block);
#define MT_GEMV(L)                                                                                  \
    case L:                                                                                         \
        hipLaunchKernelGGL(k_gemv_w4<L>, grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, cpl, \
                           y, ldy, ep);                                                             \
        break;
        switch (lpr) {
            MT_GEMV(1)
            MT_GEMV(2)
            MT_GEMV(4)
            MT_GEMV(8)
            MT_GEMV(16)
            MT_GEMV(32)
            MT_GEMV(64)
            default: return hipErrorInvalidValue;
        }
#undef MT_GEMV
        return hipGetLastError();
    }
    const dim3 grid((w.N + GT - 1) / GT, (M + GT - 1) / GT);
    hipLaunchKernelGGL(k_gemm_w4, grid, dim3(256), 0, st, x, ldx, M, w.K, w.q, w.s, w.N, y, ldy, ep);
    return hipGetLastError();
}

hipError_t launch_attn_decode(const float* q, const float* kc, const float* vc, int layer, int B,
                              int H, int t_cap, int T, float* part, int nsplit, int chunk,
                              float* out, hipStream_t st) {
    hipLaunchKernelGGL(k_attn_decode, dim3(nsplit, H, B), dim3(256), 0, st, q, kc, vc, layer, B, H,
                       t_cap, T, chunk, part);
    hipLaunchKernelGGL(k_attn_merge, dim3(H, B), dim3(64), 0, st, part, nsplit, H, out);
    return hipGetLastError();
}

hipError_t launch_attn_prefill(const float* q, const float* kc, const float* vc, int layer, int B,
                               int H, int t_cap, int t0, int R, float* out, hipStream_t st) {
    hipLaunchKernelGGL(k_attn_prefill, dim3((R + 63) / 64, H, B), dim3(256), 0, st, q, kc, vc, layer,
                       B, H, t_cap, t0, R, out);
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

hipError_t launch_dequant(const Int4Mat& w, float* out, hipStream_t st) {
    const size_t nbytes = (size_t)w.N * w.K / 2;
    const int grid = (int)((nbytes + 255) / 256 < 65536 ? (nbytes + 255) / 256 : 65536);
    hipLaunchKernelGGL(k_dequant, dim3(grid), dim3(256), 0, st, w.q, w.s, w.N, w.K, out);
    return hipGetLastError();
}

}  // namespace mt
