// decode_model.hip - the small per-token kernels of one decode step of a
// BitLinear decoder (gfx950): everything between the low-bit products.
//
// The block is the LLaMA-like recipe the b1.58 models use (M8.8 "Native
// Binary and Ternary Transformers", the b1.58 section: RMSNorm, SwiGLU,
// rotary position embeddings, bias-free linear layers); the model shape is the
// add/sub-only engine's quick-start configuration (Atomic-1Bit README: 256-d,
// 6 layers, 4 heads, 4096-entry vocabulary, 128-token context, fp32 token
// embedding).  Each kernel is a handful of workgroups: at one token these
// steps move a few KB, so they are latency-bound and sized to one launch each.
//
// Step state (device int32[4]): token, position, activation status (the
// products' LOWBIT_ACT_* bits), step status (LOWBIT_STEP_* bits).  Every
// kernel reads the position from it, so one captured HIP graph replays the
// step token after token; a position outside [0, context) makes every kernel
// return without writing (LOWBIT_STEP_POSITION).  Without a state (the
// standalone entry points) the kernels always run.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

__device__ __forceinline__ bool step_skipped(const int32_t* state, int context) {
    if (!state) return false;
    const int pos = state[1];
    return pos < 0 || pos >= context;
}

__device__ __forceinline__ float wave_sum(float v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum over a 256-thread workgroup, the same value returned to every thread.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    const float s = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return s;
}

// h = x / sqrt(mean(x^2) + eps) * g for the d values a 256-thread workgroup
// holds in xv (element tid + 256 i), with fp32 sums.
template <int NV>
__device__ __forceinline__ void rms_out(const float* xv, int d, const float* g, float eps, float* h, float* red) {
    float ss = 0.0f;
    #pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e < d) ss += xv[i] * xv[i];
    }
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    #pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = threadIdx.x + 256 * i;
        if (e < d) h[e] = xv[i] * r * g[e];
    }
}

constexpr int kMaxNV = 16;   // d <= 4096

// x = embed[token]; h = RMSNorm(x; g).  The token is clamped into the
// vocabulary (LOWBIT_STEP_TOKEN when it was not).
__global__ __launch_bounds__(256) void embed_norm_kernel(const float* __restrict__ embed, int vocab, int d,
                                                         const float* __restrict__ g, float eps,
                                                         int32_t* state, int context, float* x, float* h) {
    __shared__ float red[4];
    if (step_skipped(state, context)) {
        if (threadIdx.x == 0) atomicOr(&state[3], LOWBIT_STEP_POSITION);
        return;
    }
    int tok = state[0];
    if (tok < 0 || tok >= vocab) {
        if (threadIdx.x == 0) atomicOr(&state[3], LOWBIT_STEP_TOKEN);
        tok = tok < 0 ? 0 : vocab - 1;
    }
    const float* row = embed + (size_t)tok * d;
    float xv[kMaxNV];
    #pragma unroll
    for (int i = 0; i < kMaxNV; ++i) {
        const int e = threadIdx.x + 256 * i;
        xv[i] = e < d ? row[e] : 0.0f;
        if (e < d) x[e] = xv[i];
    }
    rms_out<kMaxNV>(xv, d, g, eps, h, red);
}

// Row blockIdx.x: v = xs + r (r nullable: v = xs); xd = v (nullable; may be
// xs); h = RMSNorm(v; g).
__global__ __launch_bounds__(256) void add_norm_kernel(const float* xs, const float* __restrict__ r, float* xd,
                                                       int d, const float* __restrict__ g, float eps,
                                                       const int32_t* state, int context, float* h) {
    __shared__ float red[4];
    if (step_skipped(state, context)) return;
    const size_t row = (size_t)blockIdx.x * d;
    xs += row;
    h += row;
    if (r) r += row;
    if (xd) xd += row;
    float xv[kMaxNV];
    #pragma unroll
    for (int i = 0; i < kMaxNV; ++i) {
        const int e = threadIdx.x + 256 * i;
        xv[i] = e < d ? (r ? xs[e] + r[e] : xs[e]) : 0.0f;
    }
    if (xd) {
        #pragma unroll
        for (int i = 0; i < kMaxNV; ++i) {
            const int e = threadIdx.x + 256 * i;
            if (e < d) xd[e] = xv[i];
        }
    }
    rms_out<kMaxNV>(xv, d, g, eps, h, red);
}

// One 256-thread workgroup per head, head_dim 64.  The head's query and key
// (qkv [3d]: q, k, v blocks) are rotated by the position (pairs (i, i + 32),
// angle pos * base^(-i / 32), evaluated in binary64 and rounded once); key and
// value go into the caches at the position.  Then softmax attention of the
// query over positions 0 .. pos in fp32: four threads per position form a
// score from 16 dimensions each (four 16-byte loads issued together), one
// wavefront takes the softmax, and four groups of 64 threads sum the weighted
// values over every fourth position, combined in LDS.  Optional trace copies
// of the rotated query and key.
__global__ __launch_bounds__(256) void rope_attn_kernel(const float* __restrict__ qkv, int d, double base,
                                                        const int32_t* state, int pos_arg, int context, float* kc,
                                                        float* vc, float* attn, float* q_trace, float* k_trace) {
    extern __shared__ float ps[];                            // [context] scores, then weights
    __shared__ __attribute__((aligned(16))) float qs[64];
    __shared__ float part[4][64];
    __shared__ float denom;
    if (step_skipped(state, context)) return;
    const int pos = state ? state[1] : pos_arg;
    const int hb = blockIdx.x * 64;                          // head's first dimension
    const int tid = threadIdx.x;
    if (tid < 32) {
        const double inv = pow(base, -(double)tid / 32.0);
        const double ang = (double)pos * inv;
        const double c = cos(ang), s = sin(ang);
        const double qa = qkv[hb + tid], qb = qkv[hb + tid + 32];
        const double ka = qkv[d + hb + tid], kb = qkv[d + hb + tid + 32];
        const float q0 = (float)(qa * c - qb * s), q1 = (float)(qa * s + qb * c);
        const float k0 = (float)(ka * c - kb * s), k1 = (float)(ka * s + kb * c);
        qs[tid] = q0;
        qs[tid + 32] = q1;
        float* kp = kc + (size_t)pos * d + hb;
        kp[tid] = k0;
        kp[tid + 32] = k1;
        if (q_trace) { q_trace[hb + tid] = q0; q_trace[hb + tid + 32] = q1; }
        if (k_trace) { k_trace[hb + tid] = k0; k_trace[hb + tid + 32] = k1; }
    } else if (tid < 96) {
        vc[(size_t)pos * d + hb + tid - 32] = qkv[2 * d + hb + tid - 32];
    }
    __syncthreads();                                         // this position's key and value, and qs

    // scores: thread 4 j + c takes dimensions 16 c .. 16 c + 15 of position j,
    // two 64-position chunks per pass with all their loads issued together
    const int c = tid & 3;
    const float4* qv = reinterpret_cast<const float4*>(qs + 16 * c);
    for (int j0 = 0; j0 <= pos; j0 += 128) {
        float4 kv[2][4];
        #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int j = j0 + 64 * h2 + (tid >> 2);
            const int jj = j <= pos ? j : pos;               // (clamped: a valid row, result unused)
            const float4* kj = reinterpret_cast<const float4*>(kc + (size_t)jj * d + hb + 16 * c);
            #pragma unroll
            for (int u = 0; u < 4; ++u) kv[h2][u] = kj[u];
        }
        #pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int j = j0 + 64 * h2 + (tid >> 2);
            float s = 0.0f;
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float4 q4 = qv[u];
                s += q4.x * kv[h2][u].x;
                s += q4.y * kv[h2][u].y;
                s += q4.z * kv[h2][u].z;
                s += q4.w * kv[h2][u].w;
            }
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if (c == 0 && j <= pos) ps[j] = s * 0.125f;      // 1 / sqrt(64), exact
        }
    }
    __syncthreads();
    if (tid < 64) {                                          // softmax weights (unnormalised) and their sum
        float m = -INFINITY;
        for (int j = tid; j <= pos; j += 64) m = ps[j] > m ? ps[j] : m;
        m = wave_max(m);
        float sum = 0.0f;
        for (int j = tid; j <= pos; j += 64) {
            const float e = expf(ps[j] - m);
            ps[j] = e;
            sum += e;
        }
        sum = wave_sum(sum);
        if (tid == 0) denom = sum;
    }
    __syncthreads();
    // weighted values: thread (grp, dim) sums positions grp, grp + 4, ... in
    // four independent chains, so that its loads run ahead of the adds
    const int dim = tid & 63, grp = tid >> 6;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* vp = vc + hb + dim;
    int j = grp;
    for (; j + 12 <= pos; j += 16) {
        float v[4];
        #pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = vp[(size_t)(j + 4 * u) * d];
        #pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += ps[j + 4 * u] * v[u];
    }
    for (; j <= pos; j += 4) acc[0] += ps[j] * vp[(size_t)j * d];
    part[grp][dim] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __syncthreads();
    if (tid < 64) attn[hb + tid] = ((part[0][tid] + part[1][tid]) + (part[2][tid] + part[3][tid])) / denom;
}

// a = SiLU(gate) * up, SiLU(z) = z / (1 + e^-z).
__global__ __launch_bounds__(256) void swiglu_kernel(const float* __restrict__ gate, const float* __restrict__ up,
                                                     float* a, int64_t n, const int32_t* state, int context) {
    if (step_skipped(state, context)) return;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float z = gate[i];
    const float s = z / (1.0f + expf(-z));
    a[i] = s * up[i];
}

// The greedy next token: argmax of the logits (the lowest index among equal
// maxima; NaN never wins; all NaN gives 0); the state advances to it and the
// next position, and tokens[pos + 1] receives it when inside the context.
// Every thread issues its 16-byte loads together (VEC: vocab % 4 == 0 and the
// logits 16-byte aligned).
template <bool VEC>
__global__ __launch_bounds__(256) void argmax_advance_kernel(const float* __restrict__ logits, int vocab,
                                                             int32_t* state, int context, int32_t* tokens) {
    __shared__ float rv[4];
    __shared__ int ri[4];
    if (step_skipped(state, context)) return;
    float best = -INFINITY;
    int idx = 0x7fffffff;
    auto take = [&](float v, int i) {
        if (v > best || (v == best && i < idx)) { best = v; idx = i; }
    };
    if constexpr (VEC) {
        const float4* l4 = reinterpret_cast<const float4*>(logits);
        const int n4 = vocab >> 2;
        for (int b = 0; b < n4; b += 256 * 4) {
            float4 v[4];
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = b + threadIdx.x + 256 * u;
                v[u] = l4[i < n4 ? i : n4 - 1];
            }
            #pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = b + threadIdx.x + 256 * u;
                if (i < n4) { take(v[u].x, 4 * i); take(v[u].y, 4 * i + 1); take(v[u].z, 4 * i + 2); take(v[u].w, 4 * i + 3); }
            }
        }
    } else {
        for (int i = threadIdx.x; i < vocab; i += 256) take(logits[i], i);
    }
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(best, off, 64);
        const int oi = __shfl_xor(idx, off, 64);
        if (ov > best || (ov == best && oi < idx)) { best = ov; idx = oi; }
    }
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) { rv[w] = best; ri[w] = idx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        best = rv[0];
        idx = ri[0];
        for (int k = 1; k < 4; ++k)
            if (rv[k] > best || (rv[k] == best && ri[k] < idx)) { best = rv[k]; idx = ri[k]; }
        const int next = idx == 0x7fffffff ? 0 : idx;
        const int pos = state[1];
        state[0] = next;
        state[1] = pos + 1;
        if (tokens && pos + 1 < context) tokens[pos + 1] = next;
    }
}

}  // namespace

hipError_t launch_embed_norm(const float* embed, int vocab, int d, const float* g, float eps, int32_t* state,
                             int context, float* x, float* h, hipStream_t st) {
    embed_norm_kernel<<<1, 256, 0, st>>>(embed, vocab, d, g, eps, state, context, x, h);
    return hipGetLastError();
}

hipError_t launch_add_norm(const float* xs, const float* r, float* xd, int rows, int d, const float* g,
                           float eps, const int32_t* state, int context, float* h, hipStream_t st) {
    add_norm_kernel<<<rows, 256, 0, st>>>(xs, r, xd, d, g, eps, state, context, h);
    return hipGetLastError();
}

hipError_t launch_rope_attn(const float* qkv, int d, int heads, double base, const int32_t* state, int pos,
                            int context, float* kc, float* vc, float* attn, float* q_trace, float* k_trace,
                            hipStream_t st) {
    rope_attn_kernel<<<heads, 256, (size_t)context * sizeof(float), st>>>(qkv, d, base, state, pos, context, kc,
                                                                           vc, attn, q_trace, k_trace);
    return hipGetLastError();
}

hipError_t launch_swiglu(const float* gate, const float* up, float* a, int64_t n, const int32_t* state,
                         int context, hipStream_t st) {
    swiglu_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(gate, up, a, n, state, context);
    return hipGetLastError();
}

hipError_t launch_argmax_advance(const float* logits, int vocab, int32_t* state, int context, int32_t* tokens,
                                 hipStream_t st) {
    if (vocab % 4 == 0 && (uintptr_t)logits % 16 == 0)
        argmax_advance_kernel<true><<<1, 256, 0, st>>>(logits, vocab, state, context, tokens);
    else
        argmax_advance_kernel<false><<<1, 256, 0, st>>>(logits, vocab, state, context, tokens);
    return hipGetLastError();
}

}  // namespace lowbit
