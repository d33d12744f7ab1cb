// lowbit_host.cpp - the C ABI of include/lowbit.h: argument checks, the host
// weight quantiser/packer, and dispatch to the HIP kernels.
//
// The packer is the export step of M8.8 "Native Binary and Ternary
// Transformers" (0x04D: export freezes the final code/scale contract): it
// runs once per weight matrix, offline, on host threads, and writes the packed
// layout the kernels stream.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <mutex>
#include <thread>
#include <vector>

#include "gemv.hpp"
#include "kernels.hpp"
#include "lowbit.h"

// The workspace of lowbit_decode_step_noalloc: one copy per GPU, held until
// the process ends.  Host code never passes this name to a kernel or a copy
// (on the host it is only a stand-in for the symbol); it uses the device
// address that hipGetSymbolAddress returns on each device (noalloc_work).
static __device__ __align__(256) uint8_t scratch[LOWBIT_NOALLOC_WORK_BYTES];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

hipError_t noalloc_work(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (uintptr_t)p % 256 != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

constexpr int32_t kAbiVersion = 5;

// Field geometry of the packed formats (the layout comment of lowbit.h).
int codes_per_word(int32_t fmt) { return fmt == LOWBIT_TERNARY2 ? 16 : (fmt == LOWBIT_INT4 ? 8 : 32); }
int block_k(int32_t fmt) { return fmt == LOWBIT_BINARY1 ? 128 : 64; }   // k of one matrix-core step

int32_t max_k_of(int32_t fmt) {
    // int32 sums of (scaled code) x (activation code): |sum| <= k * 128 * qmax
    // * scale.  128, not 127: the Q_b = 128 quantiser's codes reach -128 and
    // feed the same products.
    switch (fmt) {
        case LOWBIT_TERNARY2:
        case LOWBIT_BINARY1: return (int32_t)(2147483647LL / (128LL * 1 * 64));
        case LOWBIT_INT4:    return (int32_t)(2147483647LL / (128LL * 7 * 16));
        default:             return 0;
    }
}

lowbit_status fill_desc(int32_t format, int32_t scale, int32_t n, int32_t k, int32_t group, int32_t flags,
                        lowbit_desc* out) {
    if (!out) return LOWBIT_E_ARG;
    if (format < LOWBIT_TERNARY2 || format > LOWBIT_INT4) return LOWBIT_E_ARG;
    if (scale < LOWBIT_SCALE_TENSOR || scale > LOWBIT_SCALE_GROUP) return LOWBIT_E_ARG;
    if (n < 1 || k < 1) return LOWBIT_E_ARG;
    if ((flags & ~(LOWBIT_FLAG_TANH3 | LOWBIT_FLAG_CENTERED)) != 0) return LOWBIT_E_ARG;
    if ((flags & LOWBIT_FLAG_CENTERED) && format != LOWBIT_BINARY1) return LOWBIT_E_ARG;
    if (scale == LOWBIT_SCALE_GROUP) {
        const int32_t step = block_k(format);
        if (group < step || group % step != 0) return LOWBIT_E_ARG;
    } else if (group != 0) {
        return LOWBIT_E_ARG;
    }
    if (k > max_k_of(format)) return LOWBIT_E_RANGE;
    // k-step: the widest of 4, 2, 1 words per lane (int4: 4, 2 - one int4
    // operand is two words) that pads k no further than the narrowest does
    const int cpw = codes_per_word(format);
    const int wmin = format == LOWBIT_INT4 ? 2 : 1;
    auto padded = [&](int w) { const int64_t sk = 4LL * w * cpw; return (k + sk - 1) / sk * sk; };
    int wpl = 4;
    while (wpl > wmin && padded(wpl) != padded(wmin)) wpl /= 2;
    lowbit_desc d;
    d.format = format; d.scale = scale; d.n = n; d.k = k; d.group = group; d.flags = flags;
    d.wpl = wpl;
    d.step_k = 4 * wpl * cpw;
    d.n_steps = (k + d.step_k - 1) / d.step_k;
    d.packed_bytes = ((int64_t)n + 15) / 16 * d.n_steps * 256 * wpl;
    d.n_groups = scale == LOWBIT_SCALE_GROUP ? ((int64_t)k + group - 1) / group : 1;
    d.n_scales = scale == LOWBIT_SCALE_TENSOR ? 1
               : (scale == LOWBIT_SCALE_ROW ? n : ((int64_t)n + 15) / 16 * 16 * d.n_groups);
    *out = d;
    return LOWBIT_OK;
}

// A descriptor is accepted only if it is exactly what lowbit_describe returns.
lowbit_status check_desc(const lowbit_desc* d) {
    if (!d) return LOWBIT_E_ARG;
    lowbit_desc ref;
    lowbit_status st = fill_desc(d->format, d->scale, d->n, d->k, d->group, d->flags, &ref);
    if (st != LOWBIT_OK) return st;
    if (ref.wpl != d->wpl || ref.step_k != d->step_k || ref.n_steps != d->n_steps ||
        ref.packed_bytes != d->packed_bytes || ref.n_groups != d->n_groups || ref.n_scales != d->n_scales)
        return LOWBIT_E_ARG;
    return LOWBIT_OK;
}

// ---------------------------------------------------------------- packer

inline float premapped(float w, bool tanh3) {
    return tanh3 ? (float)(3.0 * std::tanh((double)w / 3.0)) : w;
}

// Scale of one domain of `count` values handed out by get(i), i ascending.
template <class Get>
float domain_scale(int32_t fmt, int64_t count, Get get) {
    if (fmt == LOWBIT_INT4) {
        float peak = 0.0f;
        for (int64_t i = 0; i < count; ++i) peak = std::max(peak, std::fabs(get(i)));
        return peak / 7.0f;
    }
    double total = 0.0;   // binary64, ascending order: absmean of M8.8 0x05A / 0x02B
    for (int64_t i = 0; i < count; ++i) total += (double)std::fabs(get(i));
    return (float)(total / (double)count);
}

// Mean of one domain (the centered binary rule's threshold, M8.8 0x02B):
// binary64 sum in ascending order / count, rounded once.
template <class Get>
float domain_mean(int64_t count, Get get) {
    double total = 0.0;
    for (int64_t i = 0; i < count; ++i) total += (double)get(i);
    return (float)(total / (double)count);
}

// One code from a (premapped) weight, its domain scale and, for centered
// binary codes, the domain mean (a NaN threshold otherwise).
inline int code_of(int32_t fmt, float v, float s, float centre) {
    if (fmt == LOWBIT_BINARY1) return centre == centre ? (v > centre ? 1 : -1) : (v >= 0.0f ? 1 : -1);
    if (s == 0.0f) return 0;
    const float lim = fmt == LOWBIT_INT4 ? 7.0f : 1.0f;
    float r = std::rint(v / s);
    return (int)std::min(lim, std::max(-lim, r));
}

struct RowPacker {
    const lowbit_desc& d;
    const float* w;
    uint8_t* packed;
    float* scales;
    float tensor_scale;
    float tensor_mean;   // centered binary, tensor domain; NaN when unused
    std::atomic<int>* bad;

    void operator()(int64_t r0, int64_t r1) const {
        const int64_t K = d.k;
        const bool tanh3 = (d.flags & LOWBIT_FLAG_TANH3) != 0;
        std::vector<float> row((size_t)K);
        std::vector<int8_t> codes((size_t)K);
        for (int64_t r = r0; r < r1; ++r) {
            const float* wr = w + r * K;
            for (int64_t c = 0; c < K; ++c) {
                if (!std::isfinite(wr[c])) { bad->store(1); return; }
                row[(size_t)c] = premapped(wr[c], tanh3);
            }
            // scale domains of this row
            const int64_t span = d.scale == LOWBIT_SCALE_GROUP ? d.group : K;
            const bool centered = (d.flags & LOWBIT_FLAG_CENTERED) != 0;
            for (int64_t c0 = 0, gi = 0; c0 < K; c0 += span, ++gi) {
                const int64_t c1 = std::min(K, c0 + span);
                float s = tensor_scale, centre = tensor_mean;
                if (d.scale != LOWBIT_SCALE_TENSOR) {
                    auto get = [&](int64_t i) { return row[(size_t)(c0 + i)]; };
                    s = domain_scale(d.format, c1 - c0, get);
                    if (centered) centre = domain_mean(c1 - c0, get);
                    if (d.scale == LOWBIT_SCALE_ROW) scales[r] = s;
                    else scales[((r / 16) * d.n_groups + gi) * 16 + r % 16] = s;   // [tile][group][16]
                }
                for (int64_t c = c0; c < c1; ++c)
                    codes[(size_t)c] = (int8_t)code_of(d.format, row[(size_t)c], s, centre);
            }
            emit_row(r, codes.data());
        }
    }

    // Scatter one row of codes into its words of the tiled layout (lowbit.h).
    // Each word belongs to exactly one row, so rows can be packed concurrently;
    // the buffer was zeroed beforehand (padding rows and k stay zero).
    void emit_row(int64_t row, const int8_t* c) const {
        const int64_t K = d.k;
        const int cpw = codes_per_word(d.format), kb = block_k(d.format), wb = kb / 4 / cpw;
        const int bits = d.format == LOWBIT_TERNARY2 ? 2 : (d.format == LOWBIT_INT4 ? 4 : 1);
        const uint32_t mask = (1u << bits) - 1u;
        const int64_t t = row / 16, rr = row % 16;
        for (int64_t s = 0; s < d.n_steps; ++s)
            for (int g = 0; g < 4; ++g)
                for (int w = 0; w < d.wpl; ++w) {
                    const int64_t k0 = s * d.step_k + (w / wb) * kb + g * (kb / 4) + (w % wb) * cpw;
                    if (k0 >= K) continue;
                    uint32_t word = 0;
                    for (int j = 0; j < cpw && k0 + j < K; ++j) {
                        const int8_t v = c[k0 + j];
                        if (d.format == LOWBIT_BINARY1)
                            word |= (uint32_t)(v < 0) << j;                        // byte j/8, bit j%8
                        else
                            word |= ((uint32_t)v & mask) << (8 * (j % 4) + bits * (j / 4));
                    }
                    const int64_t off = ((((t * d.n_steps + s) * 4 + g) * 16 + rr) * d.wpl + w) * 4;
                    packed[off + 0] = (uint8_t)(word);
                    packed[off + 1] = (uint8_t)(word >> 8);
                    packed[off + 2] = (uint8_t)(word >> 16);
                    packed[off + 3] = (uint8_t)(word >> 24);
                }
    }
};

thread_local hipError_t g_last_hip_error = hipSuccess;

// Launch errors are read with hipGetLastError, which also returns errors left
// behind by earlier, unrelated runtime calls of the caller; the error state is
// therefore cleared right before each launch (see clear_hip_error).
void clear_hip_error() { (void)hipGetLastError(); }

lowbit_status hip_status(hipError_t e) {
    if (e == hipSuccess) return LOWBIT_OK;
    g_last_hip_error = e;
    return LOWBIT_E_HIP;
}

lowbit_status linear_common(const lowbit_desc* d, const uint8_t* packed, const float* scales, const int8_t* q,
                            const float* sx, int32_t t, float* y, int32_t* acc, lowbit::LinearArgs* out) {
    lowbit_status st = check_desc(d);
    if (st != LOWBIT_OK) return st;
    if (!packed || !scales || !q || !sx || !y || t < 1) return LOWBIT_E_ARG;
    if ((uintptr_t)packed % 16 != 0 || (uintptr_t)scales % 4 != 0 || (uintptr_t)sx % 4 != 0 ||
        (uintptr_t)y % 4 != 0 || (uintptr_t)acc % 4 != 0)
        return LOWBIT_E_ARG;
    lowbit::LinearArgs a;
    a.fmt = d->format; a.scale = d->scale; a.group = d->group; a.n_groups = (int)d->n_groups;
    a.n = d->n; a.k = d->k; a.t = t;
    a.wpl = d->wpl; a.step_k = d->step_k; a.n_steps = (int)d->n_steps;
    a.packed = packed; a.scales = scales; a.q = q; a.sx = sx; a.y = y; a.acc = acc;
    *out = a;
    return LOWBIT_OK;
}

// The grouped entry points: every matrix validated, then 16 tokens and at
// most kGemvMaxMats matrices per launch.  x == nullptr: q / sx are inputs;
// else x is quantised into q / sx (fused).
lowbit_status grouped_common(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                             const float* const* scales, const int8_t* const* q, const float* const* sx,
                             const float* const* x, int32_t* status, int32_t t, float* const* y,
                             int32_t* const* acc, void* hip_stream) {
    if (count < 1 || !descs || !packed || !scales || !q || !sx || !y || t < 1) return LOWBIT_E_ARG;
    std::vector<lowbit::LinearArgs> args((size_t)count);
    for (int32_t i = 0; i < count; ++i) {
        const lowbit_desc& d0 = descs[0];
        const lowbit_desc& d = descs[i];
        if (d.format != d0.format || d.scale != d0.scale || d.group != d0.group || d.flags != d0.flags ||
            d.k != d0.k)
            return LOWBIT_E_ARG;
        lowbit_status st = linear_common(&d, packed[i], scales[i], q[i], sx[i], t, y[i], acc ? acc[i] : nullptr,
                                         &args[(size_t)i]);
        if (st != LOWBIT_OK) return st;
        if (x) {
            if (!x[i] || (uintptr_t)x[i] % 4 != 0) return LOWBIT_E_ARG;
            args[(size_t)i].x = x[i];
            args[(size_t)i].status = status;
        }
    }
    clear_hip_error();
    const hipStream_t stream = (hipStream_t)hip_stream;
    for (int32_t t0 = 0; t0 < t; t0 += 16) {              // 16 tokens per launch
        const int32_t tc = std::min(16, t - t0);
        std::vector<lowbit::LinearArgs> chunk(args);
        for (auto& a : chunk) {
            a.t = tc;
            a.q += (size_t)t0 * a.k;
            a.sx += t0;
            a.y += (size_t)t0 * a.n;
            if (a.acc) a.acc += (size_t)t0 * a.n * a.n_groups;
            if (a.x) a.x += (size_t)t0 * a.k;
        }
        // as few launches as the kernel-argument space allows, of near-equal size
        const int32_t launches = (count + lowbit::kGemvMaxMats - 1) / lowbit::kGemvMaxMats;
        for (int32_t li = 0, b = 0; li < launches; ++li) {
            const int32_t e = (int32_t)((int64_t)count * (li + 1) / launches);
            lowbit_status st = hip_status(lowbit::launch_gemv_group(chunk.data() + b, e - b, stream));
            if (st != LOWBIT_OK) return st;
            b = e;
        }
    }
    return LOWBIT_OK;
}

// ---- decode step of a BitLinear decoder

bool desc_is(const lowbit_desc& d, int64_t n, int64_t k) {
    return check_desc(&d) == LOWBIT_OK && d.n == n && d.k == k;
}

// Sizes valid?  (Pointers are checked by the step itself.)
bool model_sizes_ok(const lowbit_model* m) {
    if (!m) return false;
    const int64_t d = m->d_model, ff = m->d_ff;
    if (m->n_heads < 1 || d != 64LL * m->n_heads || d > 4096 || m->n_layers < 1 || ff < 1 || m->vocab < 1 ||
        m->context < 1 || m->context > 8192 || !(m->norm_eps >= 0.0f) || !(m->rope_base > 0.0f) ||
        !std::isfinite(m->norm_eps) || !std::isfinite(m->rope_base))
        return false;
    return desc_is(m->proj[LOWBIT_PROJ_QKV], 3 * d, d) && desc_is(m->proj[LOWBIT_PROJ_O], d, d) &&
           desc_is(m->proj[LOWBIT_PROJ_GATE], ff, d) && desc_is(m->proj[LOWBIT_PROJ_UP], ff, d) &&
           desc_is(m->proj[LOWBIT_PROJ_DOWN], d, ff) && desc_is(m->proj[LOWBIT_PROJ_HEAD], m->vocab, d);
}

inline int64_t up16(int64_t b) { return (b + 15) / 16 * 16; }

// Workspace: the float intermediates, then the codes and token scales the
// fused products write (gate and up get separate code buffers).
struct WorkLayout {
    int64_t x, xb, h, qkv, attn, o, gate, up, a, dn, sx, q0, q1, total;
};

WorkLayout work_layout(const lowbit_model* m) {
    const int64_t d = m->d_model, ff = m->d_ff;
    WorkLayout w;
    int64_t o = 0;
    auto take = [&](int64_t bytes) { const int64_t at = o; o += up16(bytes); return at; };
    w.x = take(4 * d); w.xb = take(4 * d); w.h = take(4 * d); w.qkv = take(12 * d); w.attn = take(4 * d); w.o = take(4 * d);
    w.gate = take(4 * ff); w.up = take(4 * ff); w.a = take(4 * ff); w.dn = take(4 * d); w.sx = take(16);
    w.q0 = take(std::max(d, ff)); w.q1 = take(ff);
    w.total = o;
    return w;
}

// The trace: the float intermediates, padded to a whole 16 bytes, then one
// code record per product (per layer qkv, o, gate, up, down; then the head):
// 16 bytes holding s_x (first float), then the product's k int8 codes padded
// to a multiple of 16 bytes.
int64_t trace_float_part(const lowbit_model* m) {
    const int64_t d = m->d_model, ff = m->d_ff;
    return (d + (int64_t)m->n_layers * (12 * d + 3 * ff) + d + 3) / 4 * 4;
}

int64_t code_record_bytes(int64_t k) { return 16 + up16(k); }

// byte offset of the code record of (layer, slot) from the start of the code part
int64_t code_record_offset(const lowbit_model* m, int layer, int slot) {
    const int64_t d = m->d_model, ff = m->d_ff;
    const int64_t per_layer = 4 * code_record_bytes(d) + code_record_bytes(ff);
    if (layer >= m->n_layers) return (int64_t)m->n_layers * per_layer;
    return layer * per_layer + (int64_t)slot * code_record_bytes(d);   // down (slot 4) follows the four k = d records
}

int64_t trace_floats(const lowbit_model* m) {
    return trace_float_part(m) + code_record_offset(m, m->n_layers, LOWBIT_PROJ_HEAD) / 4 +
           code_record_bytes(m->d_model) / 4;
}

}  // namespace

extern "C" {

lowbit_status lowbit_rmsnorm(const float* x, const float* r, float* x_out, const float* g, int32_t t, int32_t d,
                             float eps, float* h, void* hip_stream) {
    if (!x || !g || !h || t < 1 || d < 1 || d > 4096 || !(eps >= 0.0f) || !std::isfinite(eps)) return LOWBIT_E_ARG;
    if ((uintptr_t)x % 4 || (uintptr_t)r % 4 || (uintptr_t)x_out % 4 || (uintptr_t)g % 4 || (uintptr_t)h % 4)
        return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_add_norm(x, r, x_out, t, d, g, eps, nullptr, 0, h, (hipStream_t)hip_stream));
}

lowbit_status lowbit_rope_attention(const float* qkv, int32_t n_heads, int32_t pos, int32_t context, float rope_base,
                                    float* k_cache, float* v_cache, float* attn, void* hip_stream) {
    if (!qkv || !k_cache || !v_cache || !attn || n_heads < 1 || n_heads > 64 || context < 1 || context > 8192 ||
        pos < 0 || pos >= context || !(rope_base > 0.0f) || !std::isfinite(rope_base))
        return LOWBIT_E_ARG;
    if ((uintptr_t)qkv % 4 || (uintptr_t)k_cache % 16 || (uintptr_t)v_cache % 4 || (uintptr_t)attn % 4)
        return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_rope_attn(qkv, 64 * n_heads, n_heads, (double)rope_base, nullptr, pos, context,
                                               k_cache, v_cache, attn, nullptr, nullptr, (hipStream_t)hip_stream));
}

lowbit_status lowbit_swiglu(const float* gate, const float* up, int64_t n, float* a, void* hip_stream) {
    if (!gate || !up || !a || n < 1 || n > (int64_t)256 * 0x7fffffff) return LOWBIT_E_ARG;
    if ((uintptr_t)gate % 4 || (uintptr_t)up % 4 || (uintptr_t)a % 4) return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_swiglu(gate, up, a, n, nullptr, 0, (hipStream_t)hip_stream));
}

int64_t lowbit_model_work_bytes(const lowbit_model* m) { return model_sizes_ok(m) ? work_layout(m).total : -1; }

int64_t lowbit_model_trace_floats(const lowbit_model* m) { return model_sizes_ok(m) ? trace_floats(m) : -1; }

}  // extern "C"

namespace {

// Argument checks of both decode-step entry points (the workspace aside).
lowbit_status decode_step_args_ok(const lowbit_model* m, const int32_t* state, const float* logits,
                                  const int32_t* tokens, const float* trace) {
    if (!model_sizes_ok(m)) return LOWBIT_E_ARG;
    if (!m->embed || !m->norms || !m->packed || !m->scales || !m->k_cache || !m->v_cache || !state || !logits)
        return LOWBIT_E_ARG;
    if ((uintptr_t)trace % 16 != 0 || (uintptr_t)state % 4 != 0 || (uintptr_t)logits % 4 != 0 ||
        (uintptr_t)tokens % 4 != 0 || (uintptr_t)m->embed % 4 != 0 || (uintptr_t)m->norms % 4 != 0 ||
        (uintptr_t)m->k_cache % 16 != 0 || (uintptr_t)m->v_cache % 4 != 0)
        return LOWBIT_E_ARG;
    for (int i = 0; i < 5 * m->n_layers + 1; ++i)
        if (!m->packed[i] || !m->scales[i]) return LOWBIT_E_ARG;
    return LOWBIT_OK;
}

// One step with the intermediates in `work` (work_layout(m).total bytes,
// 16-byte aligned); arguments already checked.
lowbit_status decode_step_impl(const lowbit_model* m, void* work, int32_t* state, float* logits, int32_t* tokens,
                               float* trace, void* hip_stream) {
    const int L = m->n_layers;
    const int d = m->d_model, ff = m->d_ff, ctx = m->context;
    const hipStream_t st = (hipStream_t)hip_stream;
    const WorkLayout wl = work_layout(m);
    uint8_t* wb = static_cast<uint8_t*>(work);
    auto wf = [&](int64_t off) { return reinterpret_cast<float*>(wb + off); };
    float* sx = wf(wl.sx);
    int8_t* q0 = reinterpret_cast<int8_t*>(wb + wl.q0);
    int8_t* q1 = reinterpret_cast<int8_t*>(wb + wl.q1);
    int32_t* act_status = state + 2;

    // one fused BitLinear on one token; with a trace its codes and s_x go to
    // the product's own code record
    auto product = [&](int slot, int layer, const float* x, int8_t* q, float* sxp, float* y,
                       lowbit::LinearArgs* out) -> lowbit_status {
        const int i = layer < L ? 5 * layer + slot : 5 * L;
        if (trace) {
            uint8_t* rec = reinterpret_cast<uint8_t*>(trace + trace_float_part(m)) +
                           code_record_offset(m, layer, layer < L ? slot : LOWBIT_PROJ_HEAD);
            sxp = reinterpret_cast<float*>(rec);
            q = reinterpret_cast<int8_t*>(rec + 16);
        }
        lowbit_status s = linear_common(&m->proj[slot], m->packed[i], m->scales[i], q, sxp, 1, y, nullptr, out);
        out->x = x;
        out->status = act_status;
        return s;
    };
    lowbit_status s = LOWBIT_OK;
    auto run = [&](hipError_t e) { if (s == LOWBIT_OK && e != hipSuccess) s = hip_status(e); };
    auto single = [&](int slot, int layer, const float* x, float* y) {
        lowbit::LinearArgs a;
        if (s != LOWBIT_OK) return;
        s = product(slot, layer, x, q0, sx, y, &a);
        if (s == LOWBIT_OK) run(lowbit::launch_gemv(a, st));
    };

    // intermediates: trace slots, or the workspace (x updated in place)
    const int64_t ls = 12LL * d + 3LL * ff;                  // trace floats per layer
    auto tl = [&](int layer, int64_t off) { return trace + d + layer * ls + off; };
    float* x = trace ? trace : wf(wl.x);
    float* h = trace ? tl(0, 0) : wf(wl.h);
    const float eps = m->norm_eps;

    clear_hip_error();
    run(lowbit::launch_embed_norm(m->embed, m->vocab, d, m->norms, eps, state, ctx, x, h, st));

    // Fused form (k <= 3072 per product, ff % 4 == 0, aligned gains): each
    // residual add + RMSNorm runs in the next product's quantiser prologue
    // (the q/k/v of the next layer, gate and up, the head) and SwiGLU in the
    // down product's: 5 launches per layer instead of 8.  The residual stream
    // alternates between two buffers, since a launch must not overwrite the x
    // its other workgroups still read.
    const bool fused = ff % 4 == 0 && d <= 3072 && ff <= 3072 && (uintptr_t)m->norms % 16 == 0;
    if (fused) {
        const float* xs = x;                                 // x entering layer l
        const float* prev_mid = nullptr;                     // layer l-1: x after attention, down output
        const float* prev_dn = nullptr;
        float* xa = trace ? nullptr : wf(wl.x);
        float* xb = trace ? nullptr : wf(wl.xb);
        for (int l = 0; l < L && s == LOWBIT_OK; ++l) {
            float* qkv = trace ? tl(l, d) : wf(wl.qkv);
            float* qrot = trace ? tl(l, 4LL * d) : nullptr;
            float* krot = trace ? tl(l, 5LL * d) : nullptr;
            float* attn = trace ? tl(l, 6LL * d) : wf(wl.attn);
            float* o = trace ? tl(l, 7LL * d) : wf(wl.o);
            float* xmid = trace ? tl(l, 8LL * d) : xb;
            float* h2 = trace ? tl(l, 9LL * d) : nullptr;
            float* gate = trace ? tl(l, 10LL * d) : wf(wl.gate);
            float* up = trace ? tl(l, 10LL * d + ff) : wf(wl.up);
            float* a = trace ? tl(l, 10LL * d + 2LL * ff) : nullptr;
            float* dn = trace ? tl(l, 10LL * d + 3LL * ff) : wf(wl.dn);
            const size_t cache_off = (size_t)l * ctx * d;
            lowbit::LinearArgs pa;
            if (l == 0) {
                single(LOWBIT_PROJ_QKV, 0, h, qkv);         // on the embedding row's norm
            } else {                                         // x_l = mid + down of layer l-1, normed
                float* xl = trace ? tl(l - 1, 11LL * d + 3LL * ff) : xa;
                s = product(LOWBIT_PROJ_QKV, l, prev_mid, q0, sx, qkv, &pa);
                pa.pre = 1; pa.pre_r = prev_dn; pa.pre_g = m->norms + (size_t)(2 * l) * d; pa.pre_eps = eps;
                pa.pre_xo = xl; pa.pre_ho = trace ? tl(l, 0) : nullptr;
                if (s == LOWBIT_OK) run(lowbit::launch_gemv(pa, st));
                xs = xl;
            }
            if (s != LOWBIT_OK) break;
            run(lowbit::launch_rope_attn(qkv, d, m->n_heads, (double)m->rope_base, state, 0, ctx,
                                         m->k_cache + cache_off, m->v_cache + cache_off, attn, qrot, krot, st));
            single(LOWBIT_PROJ_O, l, attn, o);
            if (s != LOWBIT_OK) break;
            // gate and up on RMSNorm(x_l + o): one launch when their formats allow
            lowbit::LinearArgs gu[2];
            s = product(LOWBIT_PROJ_GATE, l, xs, q0, sx + 1, gate, &gu[0]);
            if (s == LOWBIT_OK) s = product(LOWBIT_PROJ_UP, l, xs, q1, sx + 2, up, &gu[1]);
            if (s != LOWBIT_OK) break;
            for (auto& g2 : gu) {
                g2.pre = 1; g2.pre_r = o; g2.pre_g = m->norms + (size_t)(2 * l + 1) * d; g2.pre_eps = eps;
                g2.pre_xo = xmid; g2.pre_ho = h2;
            }
            const lowbit_desc& dg = m->proj[LOWBIT_PROJ_GATE];
            const lowbit_desc& du = m->proj[LOWBIT_PROJ_UP];
            if (dg.format == du.format && dg.scale == du.scale && dg.group == du.group && dg.flags == du.flags) {
                run(lowbit::launch_gemv_group(gu, 2, st));
            } else {
                run(lowbit::launch_gemv(gu[0], st));
                run(lowbit::launch_gemv(gu[1], st));
            }
            // down on SiLU(gate) * up
            s = s == LOWBIT_OK ? product(LOWBIT_PROJ_DOWN, l, gate, q0, sx, dn, &pa) : s;
            if (s != LOWBIT_OK) break;
            pa.pre = 2; pa.pre_r = up; pa.pre_ho = a;
            run(lowbit::launch_gemv(pa, st));
            prev_mid = xmid;
            prev_dn = dn;
        }
        if (s == LOWBIT_OK) {                                // the head on RMSNorm(x_L)
            lowbit::LinearArgs ph;
            s = product(LOWBIT_PROJ_HEAD, L, prev_mid, q0, sx, logits, &ph);
            ph.pre = 1; ph.pre_r = prev_dn; ph.pre_g = m->norms + (size_t)(2 * L) * d; ph.pre_eps = eps;
            ph.pre_xo = trace ? tl(L - 1, 11LL * d + 3LL * ff) : xa;
            ph.pre_ho = trace ? trace + d + L * ls : nullptr;
            if (s == LOWBIT_OK) run(lowbit::launch_gemv(ph, st));
        }
        if (s == LOWBIT_OK) run(lowbit::launch_argmax_advance(logits, m->vocab, state, ctx, tokens, st));
        return s;
    }

    // general form: every step its own launch
    for (int l = 0; l < L && s == LOWBIT_OK; ++l) {
        float* qkv = trace ? tl(l, d) : wf(wl.qkv);
        float* qrot = trace ? tl(l, 4LL * d) : nullptr;
        float* krot = trace ? tl(l, 5LL * d) : nullptr;
        float* attn = trace ? tl(l, 6LL * d) : wf(wl.attn);
        float* o = trace ? tl(l, 7LL * d) : wf(wl.o);
        float* xmid = trace ? tl(l, 8LL * d) : x;
        float* h2 = trace ? tl(l, 9LL * d) : wf(wl.h);
        float* gate = trace ? tl(l, 10LL * d) : wf(wl.gate);
        float* up = trace ? tl(l, 10LL * d + ff) : wf(wl.up);
        float* a = trace ? tl(l, 10LL * d + 2LL * ff) : wf(wl.a);
        float* dn = trace ? tl(l, 10LL * d + 3LL * ff) : wf(wl.dn);
        float* xout = trace ? tl(l, 11LL * d + 3LL * ff) : x;
        float* hnext = trace ? (l + 1 < L ? tl(l + 1, 0) : trace + d + L * ls) : wf(wl.h);
        const size_t cache_off = (size_t)l * ctx * d;

        single(LOWBIT_PROJ_QKV, l, h, qkv);
        if (s != LOWBIT_OK) break;
        run(lowbit::launch_rope_attn(qkv, d, m->n_heads, (double)m->rope_base, state, 0, ctx,
                                     m->k_cache + cache_off, m->v_cache + cache_off, attn, qrot, krot, st));
        single(LOWBIT_PROJ_O, l, attn, o);
        if (s != LOWBIT_OK) break;
        run(lowbit::launch_add_norm(x, o, xmid, 1, d, m->norms + (size_t)(2 * l + 1) * d, eps, state, ctx, h2,
                                    st));
        // gate and up share their input: one launch when their formats allow
        lowbit::LinearArgs gu[2];
        s = product(LOWBIT_PROJ_GATE, l, h2, q0, sx + 1, gate, &gu[0]);
        if (s == LOWBIT_OK) s = product(LOWBIT_PROJ_UP, l, h2, q1, sx + 2, up, &gu[1]);
        if (s != LOWBIT_OK) break;
        const lowbit_desc& dg = m->proj[LOWBIT_PROJ_GATE];
        const lowbit_desc& du = m->proj[LOWBIT_PROJ_UP];
        if (dg.format == du.format && dg.scale == du.scale && dg.group == du.group && dg.flags == du.flags) {
            run(lowbit::launch_gemv_group(gu, 2, st));
        } else {
            run(lowbit::launch_gemv(gu[0], st));
            run(lowbit::launch_gemv(gu[1], st));
        }
        run(lowbit::launch_swiglu(gate, up, a, ff, state, ctx, st));
        single(LOWBIT_PROJ_DOWN, l, a, dn);
        if (s != LOWBIT_OK) break;
        const float* gnext = m->norms + (size_t)(2 * l + 2) * d;   // next layer's attention norm, or the final one
        run(lowbit::launch_add_norm(xmid, dn, xout, 1, d, gnext, eps, state, ctx, hnext, st));
        x = xout;
        h = hnext;
    }
    single(LOWBIT_PROJ_HEAD, L, h, logits);
    if (s == LOWBIT_OK) run(lowbit::launch_argmax_advance(logits, m->vocab, state, ctx, tokens, st));
    return s;
}

}  // namespace

extern "C" {

lowbit_status lowbit_decode_step(const lowbit_model* m, int32_t* state, float* logits, int32_t* tokens,
                                 float* trace, void* hip_stream) {
    const lowbit_status a = decode_step_args_ok(m, state, logits, tokens, trace);
    if (a != LOWBIT_OK) return a;
    if (!m->work || (uintptr_t)m->work % 16 != 0) return LOWBIT_E_ARG;
    return decode_step_impl(m, m->work, state, logits, tokens, trace, hip_stream);
}

lowbit_status lowbit_decode_step_noalloc(const lowbit_model* m, int32_t* state, float* logits, int32_t* tokens,
                                         float* trace, void* hip_stream) {
    const lowbit_status a = decode_step_args_ok(m, state, logits, tokens, trace);
    if (a != LOWBIT_OK) return a;
    if (work_layout(m).total > LOWBIT_NOALLOC_WORK_BYTES) return LOWBIT_E_RANGE;
    clear_hip_error();
    void* work = nullptr;
    const hipError_t e = noalloc_work(&work);
    if (e != hipSuccess) return hip_status(e);
    return decode_step_impl(m, work, state, logits, tokens, trace, hip_stream);
}

lowbit_status lowbit_calib_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream) {
    if (!src || !sink || bytes < 16 || bytes % 16 || (uintptr_t)src % 16 || (uintptr_t)sink % 4) return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_calib_read(src, bytes, sink, (hipStream_t)hip_stream));
}

int64_t lowbit_calib_mfma_i8_ops(int32_t iters) {
    return iters < 1 ? -1 : (int64_t)iters * lowbit::calib_mfma_i8_ops_per_iter();
}

lowbit_status lowbit_calib_mfma_i8(int32_t iters, uint32_t* sink, void* hip_stream) {
    if (iters < 1 || !sink || (uintptr_t)sink % 4) return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_calib_mfma_i8(iters, sink, (hipStream_t)hip_stream));
}

lowbit_status lowbit_describe(int32_t format, int32_t scale, int32_t n, int32_t k, int32_t group, int32_t flags,
                              lowbit_desc* out) {
    return fill_desc(format, scale, n, k, group, flags, out);
}

lowbit_status lowbit_pack(const lowbit_desc* d, const float* w, uint8_t* packed, float* scales) {
    lowbit_status st = check_desc(d);
    if (st != LOWBIT_OK) return st;
    if (!w || !packed || !scales) return LOWBIT_E_ARG;
    const int64_t N = d->n, K = d->k;
    const bool tanh3 = (d->flags & LOWBIT_FLAG_TANH3) != 0;

    float tensor_scale = 0.0f, tensor_mean = std::numeric_limits<float>::quiet_NaN();
    if (d->scale == LOWBIT_SCALE_TENSOR) {   // one sequential pass over all of W
        for (int64_t i = 0; i < N * K; ++i)
            if (!std::isfinite(w[i])) return LOWBIT_E_NONFINITE;
        auto get = [&](int64_t i) { return premapped(w[i], tanh3); };
        tensor_scale = domain_scale(d->format, N * K, get);
        if (d->flags & LOWBIT_FLAG_CENTERED) tensor_mean = domain_mean(N * K, get);
        scales[0] = tensor_scale;
    }

    std::memset(packed, 0, (size_t)d->packed_bytes);
    if (d->scale == LOWBIT_SCALE_GROUP) std::memset(scales, 0, (size_t)d->n_scales * sizeof(float));

    std::atomic<int> bad{0};
    RowPacker job{*d, w, packed, scales, tensor_scale, tensor_mean, &bad};
    const int64_t work = N * K;
    unsigned hw = std::max(1u, std::thread::hardware_concurrency());
    unsigned nthreads = (unsigned)std::min<int64_t>({(int64_t)hw, N, std::max<int64_t>(1, work / (1 << 16))});
    if (nthreads <= 1) {
        job(0, N);
    } else {
        std::vector<std::thread> pool;
        for (unsigned i = 0; i < nthreads; ++i) {
            const int64_t r0 = N * i / nthreads, r1 = N * (i + 1) / nthreads;
            pool.emplace_back([&job, r0, r1] { job(r0, r1); });
        }
        for (auto& th : pool) th.join();
    }
    return bad.load() ? LOWBIT_E_NONFINITE : LOWBIT_OK;
}

lowbit_status lowbit_act_quant(const float* x, int32_t t, int32_t k, int8_t* q, float* sx, int32_t* status,
                               void* hip_stream) {
    if (!x || !q || !sx || t < 1 || k < 1) return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_act_quant(x, t, k, q, sx, status, (hipStream_t)hip_stream));
}

lowbit_status lowbit_act_quant_v1(const float* x, int32_t t, int32_t k, float eps, int32_t per_tensor, int8_t* q,
                                  float* sx, int32_t* status, uint32_t* work, void* hip_stream) {
    if (!x || !q || !sx || t < 1 || k < 1 || !(eps >= 0.0f) || !std::isfinite(eps)) return LOWBIT_E_ARG;
    if (per_tensor != 0 && per_tensor != 1) return LOWBIT_E_ARG;
    if (per_tensor && (!work || (uintptr_t)work % 4)) return LOWBIT_E_ARG;
    if ((uintptr_t)x % 4 || (uintptr_t)sx % 4 || (uintptr_t)status % 4) return LOWBIT_E_ARG;
    if (k > 262143) return LOWBIT_E_RANGE;
    clear_hip_error();
    hipStream_t st = (hipStream_t)hip_stream;
    if (per_tensor) {
        hipError_t e = lowbit::launch_tensor_absmax(x, (int64_t)t * k, work, st);
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(lowbit::launch_act_quant_v1(x, t, k, eps, per_tensor ? work : nullptr, q, sx, status, st));
}

lowbit_status lowbit_onebit_linear(const lowbit_desc* d, const uint8_t* packed, const uint16_t* g, const uint16_t* h,
                                   const uint16_t* x, int32_t t, float* y, void* hip_stream) {
    lowbit_status st = check_desc(d);
    if (st != LOWBIT_OK) return st;
    if (d->format != LOWBIT_BINARY1 || !packed || !g || !h || !x || !y || t < 1) return LOWBIT_E_ARG;
    if ((uintptr_t)packed % 16 || (uintptr_t)g % 2 || (uintptr_t)h % 2 || (uintptr_t)x % 2 || (uintptr_t)y % 4)
        return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_onebit(packed, g, h, x, y, d->n, d->k, t, d->wpl, d->step_k, (int)d->n_steps,
                                            (hipStream_t)hip_stream));
}

lowbit_status lowbit_layernorm(const float* x, int32_t t, int32_t d, float eps, const float* g, const float* b,
                               float* out, void* hip_stream) {
    if (!x || !out || t < 1 || d < 1 || !(eps >= 0.0f) || !std::isfinite(eps)) return LOWBIT_E_ARG;
    if ((uintptr_t)x % 4 || (uintptr_t)out % 4 || (uintptr_t)g % 4 || (uintptr_t)b % 4) return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_layernorm(x, t, d, eps, g, b, out, (hipStream_t)hip_stream));
}

lowbit_status lowbit_act_quant_h4(const float* x, int32_t t, int32_t k, int8_t* q, float* sx, int32_t* status,
                                  void* hip_stream) {
    if (!x || !q || !sx || t < 1 || k < 64 || k % 64) return LOWBIT_E_ARG;
    if ((uintptr_t)x % 16 || (uintptr_t)q % 4 || (uintptr_t)sx % 4 || (uintptr_t)status % 4) return LOWBIT_E_ARG;
    if (k > lowbit::kH4MaxK) return LOWBIT_E_RANGE;
    clear_hip_error();
    return hip_status(lowbit::launch_act_quant_h4(x, t, k, q, sx, status, (hipStream_t)hip_stream));
}

lowbit_status lowbit_act_quant_a4(const float* x, int32_t t, int32_t k, int8_t* q, float* sx, int32_t* status,
                                  void* hip_stream) {
    if (!x || !q || !sx || t < 1 || k < 1) return LOWBIT_E_ARG;
    if ((uintptr_t)x % 4 || (uintptr_t)sx % 4 || (uintptr_t)status % 4) return LOWBIT_E_ARG;
    clear_hip_error();
    return hip_status(lowbit::launch_act_quant_a4(x, t, k, q, sx, status, (hipStream_t)hip_stream));
}

lowbit_status lowbit_act_quant_sparse8(const float* x, int32_t t, int32_t k, int32_t keep, int8_t* q, float* sx,
                                       int32_t* status, void* hip_stream) {
    if (!x || !q || !sx || t < 1 || k < 4 || k % 4 || keep < 1 || keep > k) return LOWBIT_E_ARG;
    if ((uintptr_t)x % 16 || (uintptr_t)q % 4 || (uintptr_t)sx % 4 || (uintptr_t)status % 4) return LOWBIT_E_ARG;
    if (k > lowbit::kSparse8MaxK) return LOWBIT_E_RANGE;
    clear_hip_error();
    return hip_status(lowbit::launch_act_quant_sparse8(x, t, k, keep, q, sx, status, (hipStream_t)hip_stream));
}

lowbit_status lowbit_linear(const lowbit_desc* d, const uint8_t* packed, const float* scales, const int8_t* q,
                            const float* sx, int32_t t, float* y, int32_t* acc, void* hip_stream) {
    lowbit::LinearArgs a;
    lowbit_status st = linear_common(d, packed, scales, q, sx, t, y, acc, &a);
    if (st != LOWBIT_OK) return st;
    clear_hip_error();
    return hip_status(lowbit::launch_gemv(a, (hipStream_t)hip_stream));
}

lowbit_status lowbit_linear_batched(const lowbit_desc* d, const uint8_t* packed, const float* scales,
                                    const int8_t* q, const float* sx, int32_t t, float* y, int32_t* acc,
                                    void* hip_stream) {
    lowbit::LinearArgs a;
    lowbit_status st = linear_common(d, packed, scales, q, sx, t, y, acc, &a);
    if (st != LOWBIT_OK) return st;
    clear_hip_error();
    return hip_status(lowbit::launch_gemm(a, (hipStream_t)hip_stream));
}

lowbit_status lowbit_linear_fused(const lowbit_desc* d, const uint8_t* packed, const float* scales, const float* x,
                                  int32_t t, int8_t* q, float* sx, float* y, int32_t* status, void* hip_stream) {
    lowbit::LinearArgs a;
    lowbit_status st = linear_common(d, packed, scales, q, sx, t, y, nullptr, &a);
    if (st != LOWBIT_OK) return st;
    if (!x || (uintptr_t)x % 4 != 0 || (uintptr_t)status % 4 != 0) return LOWBIT_E_ARG;
    a.x = x;
    a.status = status;
    clear_hip_error();
    return hip_status(lowbit::launch_gemv(a, (hipStream_t)hip_stream));
}

lowbit_status lowbit_linear_batched_grouped(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                                            const float* const* scales, const int8_t* const* q,
                                            const float* const* sx, int32_t t, float* const* y,
                                            int32_t* const* acc, void* hip_stream) {
    if (count < 1 || !descs || !packed || !scales || !q || !sx || !y || t < 1) return LOWBIT_E_ARG;
    std::vector<lowbit::LinearArgs> args((size_t)count);
    for (int32_t i = 0; i < count; ++i) {
        const lowbit_desc& d0 = descs[0];
        const lowbit_desc& d = descs[i];
        if (d.format != d0.format || d.scale != d0.scale || d.group != d0.group || d.flags != d0.flags ||
            d.k != d0.k)
            return LOWBIT_E_ARG;
        lowbit_status st = linear_common(&d, packed[i], scales[i], q[i], sx[i], t, y[i], acc ? acc[i] : nullptr,
                                         &args[(size_t)i]);
        if (st != LOWBIT_OK) return st;
    }
    clear_hip_error();
    return hip_status(lowbit::launch_gemm_group(args.data(), count, (hipStream_t)hip_stream));
}

lowbit_status lowbit_linear_grouped(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                                    const float* const* scales, const int8_t* const* q, const float* const* sx,
                                    int32_t t, float* const* y, int32_t* const* acc, void* hip_stream) {
    return grouped_common(count, descs, packed, scales, q, sx, nullptr, nullptr, t, y, acc, hip_stream);
}

lowbit_status lowbit_linear_grouped_fused(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                                          const float* const* scales, const float* const* x, int8_t* const* q,
                                          float* const* sx, int32_t t, float* const* y, int32_t* status,
                                          void* hip_stream) {
    if (!x || (uintptr_t)status % 4 != 0) return LOWBIT_E_ARG;
    return grouped_common(count, descs, packed, scales, reinterpret_cast<const int8_t* const*>(q),
                          reinterpret_cast<const float* const*>(sx), x, status, t, y, nullptr, hip_stream);
}

int32_t lowbit_max_k(int32_t format) { return max_k_of(format); }

const char* lowbit_status_string(lowbit_status s) {
    switch (s) {
        case LOWBIT_OK: return "ok";
        case LOWBIT_E_ARG: return "invalid argument";
        case LOWBIT_E_RANGE: return "k exceeds the int32 accumulator bound";
        case LOWBIT_E_NONFINITE: return "non-finite latent weight";
        case LOWBIT_E_FORMAT: return "invalid packed data";
        case LOWBIT_E_HIP: return "HIP launch failed";
        default: return "unknown status";
    }
}

int32_t lowbit_abi_version(void) { return kAbiVersion; }

const char* lowbit_last_hip_error(void) { return hipGetErrorString(g_last_hip_error); }

}  // extern "C"
