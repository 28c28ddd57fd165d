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

// Raw buffer resource over [base, base + bytes): loads through it take a
// 32-bit per-lane byte offset plus a scalar offset, and read 0 past the end.
// bytes is clamped to the 32-bit record count.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// 16 bytes per lane from a buffer straight into LDS: lane i's bytes land at
// lds + 16 i (lds must be the same for the whole wave).  Written as inline
// assembly on purpose: the compiler then does not track the LDS write, so it
// does not drain the load counter before every later LDS read (it cannot
// tell which LDS bytes the load writes); the caller orders the write with
// its own s_waitcnt vmcnt and barrier before any wave reads those bytes.
// The resource is a raw buffer descriptor {base, base_hi, bytes, flags}.
// m0 carries the LDS address; no other instruction of the kernels that use
// this helper reads m0.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 raw_rsrc(const void* base, int64_t bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return i32x4{(int)(uint32_t)b, (int)((b >> 32) & 0xFFFF), n, 0x00020000};
}

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, void* lds, int voffset, int soffset) {
#if defined(__HIP_DEVICE_COMPILE__)
    const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)lds;
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(la), "v"(voffset), "s"(rsrc), "s"(soffset)
                 : "memory", "m0");
#endif
}
#pragma clang diagnostic pop

}  // namespace w4a16
