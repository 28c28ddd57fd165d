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
__device__ __forceinline__ half2v as_h2(uint32_t v) { return __builtin_bit_cast(half2v, v); }
__device__ __forceinline__ uint32_t as_u32(half2v v) { return __builtin_bit_cast(uint32_t, v); }

// (w & mask) | bias in one instruction (the bias lives in a vector register
// so that the instruction needs only one scalar operand).
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t bias) {
    uint32_t d;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(w), "s"(mask), "v"(bias));
    return d;
}

// Eight fp16 weights (q - z) * s of one packed word, in the k order
// 0, 4, 1, 5, 2, 6, 3, 7 (the order the activation chunks use).  Nibbles
// at bits 0-3 of a half are OR-ed into fp16 1024 (ulp 1), nibbles at bits
// 4-7 into fp16 64 (ulp 1/16); the differences with 1024 + z and 64 + z are
// the exact integers q - z, and the product with s is the one rounding.
struct Dequant {
    uint32_t b1024, b64;     // fp16 1024 / 64 in both halves (vector registers)
    half2v z1024, z64, s2;   // per row and group
    __device__ __forceinline__ void init() {
        b1024 = 0x64006400u;
        b64 = 0x54005400u;
    }
    __device__ __forceinline__ half8 operator()(uint32_t w) const {
        const uint32_t w8 = w >> 8;
        const half2v p0 = (as_h2(and_or(w, 0x000F000Fu, b1024)) - z1024) * s2;
        const half2v p1 = (as_h2(and_or(w, 0x00F000F0u, b64)) - z64) * s2;
        const half2v p2 = (as_h2(and_or(w8, 0x000F000Fu, b1024)) - z1024) * s2;
        const half2v p3 = (as_h2(and_or(w8, 0x00F000F0u, b64)) - z64) * s2;
        half8 r;
        r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
        r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
        return r;
    }
    // z: 4-bit zero code; sbits: fp16 bits of the scale
    __device__ __forceinline__ void set(uint32_t z, uint32_t sbits) {
        z1024 = as_h2(0x64006400u | z | (z << 16));
        z64 = as_h2(0x54005400u | (z << 4) | (z << 20));
        s2 = as_h2(sbits | (sbits << 16));
    }
};

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

// Bits of a float, taken from a value (a __builtin_bit_cast applied directly
// to an element of an ext_vector_type yields element 0 whatever the index
// with this compiler, so vector elements pass through here by value).
__device__ __forceinline__ uint32_t f32_bits(float v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
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
