// device_common.hpp - gfx950 device helpers shared by the low-bit kernels.
//
// Code decode.  Every packed format is turned into int8 matrix-core operands
// whose bytes are the code times a power of two, by moving each field to the
// top of its byte with one shift and one mask (the sign bit of the field lands
// on the sign bit of the byte):
//   ternary 2-bit two's complement -> 64 * q   (q in {-1, 0, +1})
//   int4    4-bit two's complement -> 16 * q   (q in -7..+7)
//   binary  bit b (s = 1 - 2b)     -> 64 * s   (0x40 | 0x80 * b)
// so an i8 MFMA over them yields 64 (16) times the exact integer product, which
// an arithmetic shift turns back into the product (it is always a multiple).
// This is the sign-controlled accumulation of the add/sub form (M8.8
// "Native Binary and Ternary Transformers", 0x05D; Atomic-1Bit README), carried
// out by the matrix cores instead of scalar adds.
//
// Operand k-order.  An MFMA sums over whatever 16 k values each lane group
// supplies, as long as its A and B bytes name the same k.  For ternary and int4
// the decode yields k in natural order (16 consecutive codes per operand), so
// the activation operand is 16 consecutive bytes of q.  Binary keeps the
// page's packbits order, where register j of a decoded word holds codes
// 8b + j (b = byte); its activation operand is permuted to match
// (perm_binary_a).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { FMT_TERNARY = 0, FMT_BINARY = 1, FMT_INT4 = 2 };

// Codes per 32-bit packed word and the power of two the decode scales by.
template <int FMT> struct Fmt;
template <> struct Fmt<FMT_TERNARY> { static constexpr int kCodesPerWord = 16; static constexpr int kShift = 6; };
template <> struct Fmt<FMT_BINARY>  { static constexpr int kCodesPerWord = 32; static constexpr int kShift = 6; };
template <> struct Fmt<FMT_INT4>    { static constexpr int kCodesPerWord = 8;  static constexpr int kShift = 4; };

__device__ __forceinline__ i32x4 mfma16(const i32x4& a, const i32x4& b, const i32x4& c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ternary word (16 codes) -> one operand, byte 4r + b = 64 * code(4r + b)
__device__ __forceinline__ i32x4 decode_ternary(uint32_t w) {
    i32x4 o;
    o[0] = (int32_t)((w << 6) & 0xC0C0C0C0u);
    o[1] = (int32_t)((w << 4) & 0xC0C0C0C0u);
    o[2] = (int32_t)((w << 2) & 0xC0C0C0C0u);
    o[3] = (int32_t)(w & 0xC0C0C0C0u);
    return o;
}

// two int4 words (16 codes) -> one operand, byte i = 16 * code(i)
__device__ __forceinline__ i32x4 decode_int4(uint32_t w0, uint32_t w1) {
    i32x4 o;
    o[0] = (int32_t)((w0 << 4) & 0xF0F0F0F0u);
    o[1] = (int32_t)(w0 & 0xF0F0F0F0u);
    o[2] = (int32_t)((w1 << 4) & 0xF0F0F0F0u);
    o[3] = (int32_t)(w1 & 0xF0F0F0F0u);
    return o;
}

// binary word (32 codes) -> two operands; register j (0..7) byte b holds
// 64 * s(8b + j); operand 0 = registers 0..3, operand 1 = registers 4..7.
__device__ __forceinline__ void decode_binary(uint32_t w, i32x4& o0, i32x4& o1) {
    o0[0] = (int32_t)(((w << 7) & 0x80808080u) | 0x40404040u);
    o0[1] = (int32_t)(((w << 6) & 0x80808080u) | 0x40404040u);
    o0[2] = (int32_t)(((w << 5) & 0x80808080u) | 0x40404040u);
    o0[3] = (int32_t)(((w << 4) & 0x80808080u) | 0x40404040u);
    o1[0] = (int32_t)(((w << 3) & 0x80808080u) | 0x40404040u);
    o1[1] = (int32_t)(((w << 2) & 0x80808080u) | 0x40404040u);
    o1[2] = (int32_t)(((w << 1) & 0x80808080u) | 0x40404040u);
    o1[3] = (int32_t)((w & 0x80808080u) | 0x40404040u);
}

// one of the two operands of decode_binary (op 0: registers 0..3, op 1: 4..7)
__device__ __forceinline__ i32x4 decode_binary_half(uint32_t w, int op) {
    const int sh = op == 0 ? 7 : 3;
    i32x4 o;
    o[0] = (int32_t)(((w << sh) & 0x80808080u) | 0x40404040u);
    o[1] = (int32_t)(((w << (sh - 1)) & 0x80808080u) | 0x40404040u);
    o[2] = (int32_t)(((w << (sh - 2)) & 0x80808080u) | 0x40404040u);
    o[3] = (int32_t)(((w << (sh - 3)) & 0x80808080u) | 0x40404040u);
    return o;
}

// 4x4 byte transpose: out[j] byte i = in[i] byte j  (8 v_perm_b32)
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d, i32x4& o) {
    // v_perm_b32(s0, s1, sel): byte i of the result = byte sel[i] of {s0:s1},
    // where bytes 0-3 are s1 and 4-7 are s0.
    uint32_t ab_lo = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    uint32_t ab_hi = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    uint32_t cd_lo = __builtin_amdgcn_perm(d, c, 0x05010400u);   // c0 d0 c1 d1
    uint32_t cd_hi = __builtin_amdgcn_perm(d, c, 0x07030602u);   // c2 d2 c3 d3
    o[0] = (int32_t)__builtin_amdgcn_perm(cd_lo, ab_lo, 0x05040100u);   // a0 b0 c0 d0
    o[1] = (int32_t)__builtin_amdgcn_perm(cd_lo, ab_lo, 0x07060302u);   // a1 b1 c1 d1
    o[2] = (int32_t)__builtin_amdgcn_perm(cd_hi, ab_hi, 0x05040100u);   // a2 b2 c2 d2
    o[3] = (int32_t)__builtin_amdgcn_perm(cd_hi, ab_hi, 0x07060302u);   // a3 b3 c3 d3
}

// 32 activation bytes X[0..7] (X[d] byte e = x[4d + e]) -> the two operands
// matching decode_binary: operand a, register j, byte b = x[8b + 4a + j].
__device__ __forceinline__ void perm_binary_a(const uint32_t* X, i32x4& a0, i32x4& a1) {
    transpose4x4(X[0], X[2], X[4], X[6], a0);
    transpose4x4(X[1], X[3], X[5], X[7], a1);
}

// Byte-safe loads.  `valid` = number of leading bytes that exist (<= n);
// the rest read as zero.  Used for ragged tails and unaligned rows only.
__device__ __forceinline__ uint32_t load_u32_partial(const uint8_t* p, int valid) {
    uint32_t v = 0;
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < valid) v |= (uint32_t)p[i] << (8 * i);
    return v;
}

template <int NWORDS>
__device__ __forceinline__ void load_words(const uint8_t* p, int valid, bool aligned_full, uint32_t* out) {
    if (aligned_full) {
        if constexpr (NWORDS == 4) {
            u32x4 v = *reinterpret_cast<const u32x4*>(p);
            out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
        } else if constexpr (NWORDS == 2) {
            u32x2 v = *reinterpret_cast<const u32x2*>(p);
            out[0] = v[0]; out[1] = v[1];
        } else {
            #pragma unroll
            for (int i = 0; i < NWORDS; ++i) out[i] = reinterpret_cast<const uint32_t*>(p)[i];
        }
    } else {
        #pragma unroll
        for (int i = 0; i < NWORDS; ++i) {
            int vi = valid - 4 * i;
            out[i] = vi <= 0 ? 0u : load_u32_partial(p + 4 * i, vi < 4 ? vi : 4);
        }
    }
}

// NWORDS aligned words read with the non-temporal hint: data that is read
// exactly once (the decode GEMV's weight stream) should not displace reused
// lines in the caches.
template <int NWORDS>
__device__ __forceinline__ void load_words_stream(const uint8_t* p, uint32_t* out) {
    if constexpr (NWORDS == 4) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (NWORDS == 2) {
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    }
}

// The same stream through a buffer resource: NWORDS words at byte offset
// voff (per lane) + soff (uniform) of the resource, non-temporal.
template <int NWORDS>
__device__ __forceinline__ void load_words_stream_buf(__amdgpu_buffer_rsrc_t r, int voff, int soff, uint32_t* out) {
    constexpr int kNT = 2;                                   // the non-temporal cache policy
    if constexpr (NWORDS == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNT);
        out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
    } else if constexpr (NWORDS == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNT);
        out[0] = v[0]; out[1] = v[1];
    } else {
        out[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNT);
    }
}

// One activation code (M8.8 0x02C, 0x05C): clip(rint(v * r), -127, 127) with
// r = 127 / max|x| of the token row; one fp32 multiply (files are built without
// contraction), rintf rounds half to even.
__device__ __forceinline__ int8_t quant1(float v, float r) {
    float p = v * r;
    float c = rintf(p);
    c = c < -127.0f ? -127.0f : (c > 127.0f ? 127.0f : c);
    return (int8_t)(int)c;
}

__device__ __forceinline__ float wave_max(float v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        float o = __shfl_xor(v, off, 64);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_or(int v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v |= __shfl_xor(v, off, 64);
    return v;
}

}  // namespace lowbit
