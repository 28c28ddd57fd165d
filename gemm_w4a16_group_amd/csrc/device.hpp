// Device helpers shared by the W4A16 kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 128;          // weights per (scale, zero) pair
constexpr uint32_t kBias = 0x64006400u;  // fp16 1024.0 in both halves

__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// (1024 + z) in both fp16 halves of a word, for a 4-bit zero code z.
__device__ __forceinline__ uint32_t zero_bias(uint32_t z) { return kBias | z | (z << 16); }

// One packed word (8 codes, nibble j = k offset j) -> 8 fp16 values (q - z),
// exact.  Each nibble is OR-ed into the mantissa of fp16 1024 (ulp 1 there),
// which gives 1024 + q; subtracting 1024 + z leaves the integer q - z.
// Element order of the result: k offsets 0, 4, 1, 5, 2, 6, 3, 7 (each fp16
// pair holds nibbles p and p + 4 of the word).  The activation operand of the
// matrix instruction is stored in the same order.
__device__ __forceinline__ half8 dequant_word(uint32_t w, uint32_t zb) {
    const half2v z2 = as_h2(zb);
    half2v p0 = as_h2((w & 0x000F000Fu) | kBias) - z2;
    half2v p1 = as_h2(((w >> 4) & 0x000F000Fu) | kBias) - z2;
    half2v p2 = as_h2(((w >> 8) & 0x000F000Fu) | kBias) - z2;
    half2v p3 = as_h2(((w >> 12) & 0x000F000Fu) | kBias) - z2;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Same, then multiplied by the group scale (result rounded to fp16).
__device__ __forceinline__ half8 dequant_word_scaled(uint32_t w, uint32_t zb, half2v s2) {
    const half2v z2 = as_h2(zb);
    half2v p0 = (as_h2((w & 0x000F000Fu) | kBias) - z2) * s2;
    half2v p1 = (as_h2(((w >> 4) & 0x000F000Fu) | kBias) - z2) * s2;
    half2v p2 = (as_h2(((w >> 8) & 0x000F000Fu) | kBias) - z2) * s2;
    half2v p3 = (as_h2(((w >> 12) & 0x000F000Fu) | kBias) - z2) * s2;
    half8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// 8 consecutive activations x[k0 .. k0+7] (as four fp16 pairs) reordered to
// the dequant order 0, 4, 1, 5, 2, 6, 3, 7.
__device__ __forceinline__ u32x4 permute_k8(u32x4 v) {
    // v.x = (x0, x1), v.y = (x2, x3), v.z = (x4, x5), v.w = (x6, x7)
    u32x4 r;
    r.x = __builtin_amdgcn_perm(v.z, v.x, 0x05040100u);  // (x0, x4)
    r.y = __builtin_amdgcn_perm(v.z, v.x, 0x07060302u);  // (x1, x5)
    r.z = __builtin_amdgcn_perm(v.w, v.y, 0x05040100u);  // (x2, x6)
    r.w = __builtin_amdgcn_perm(v.w, v.y, 0x07060302u);  // (x3, x7)
    return r;
}

// Low halves of two words -> (lo(a), lo(b)); high halves -> (hi(a), hi(b)).
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ uint32_t f32_to_h16_bits(float v) {
    _Float16 h = (_Float16)v;   // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

}  // namespace w4a16
