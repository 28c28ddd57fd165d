// Round-to-nearest asymmetric group quantizer: fp16 W [M, K] -> packed
// 4-bit codes, fp16 scales and packed 4-bit zeros, one (scale, zero) per 128
// consecutive k of a row.  This is the step that produces the layer's
// weights on the PerfXLLM page on Snapdragon 8 Gen2, §3.1 (weights only, to
// int4, group size 128, a scale and a zero per group); the plain min/max
// form, without AWQ's activation-aware scale search:
//
//   lo, hi = min(group min, 0), max(group max, 0)     (float32)
//   s      = fp16(max(hi - lo, 1e-5) / 15)             (float32 divide)
//   z      = clamp(rint(-lo / s), 0, 15)               (float32 divide)
//   q      = clamp(rint(w / s) + z, 0, 15)             (float32 divide)
//
// with correctly rounded float32 divides and round-half-to-even, so that the
// integer codes are the same on any IEEE implementation of these steps.
//
// One wave takes eight consecutive groups of one row (2 KB of fp16): lane l
// holds values 16 l .. 16 l + 15 of the eight groups (group l / 8), the eight
// lanes of a group reduce its minimum and maximum with lane shuffles, each
// lane writes the two packed words of its sixteen codes (the wave writes
// 512 contiguous bytes), the first lane of a group its scale, and lane 0 the
// zero word of the eight groups.  HBM-bound: 2 bytes read and 0.5 + 2.5/128
// bytes written per weight.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

__global__ void __launch_bounds__(256) quantize_kernel(const uint16_t* __restrict__ w, uint32_t* __restrict__ qpk,
                                                       uint16_t* __restrict__ scales, uint32_t* __restrict__ zpk,
                                                       int64_t M, int64_t K, int32_t G, int32_t ZW) {
    const int lane = threadIdx.x & 63;
    const int64_t chunk = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (row, zero word)
    const int64_t nchunks = M * ZW;
    if (chunk >= nchunks) return;                                          // whole waves only
    const int64_t row = chunk / ZW;
    const int zw = (int)(chunk % ZW);
    const int g = zw * 8 + (lane >> 3);                                   // this lane's group
    const bool live = g < G;

    // sixteen values: k = 128 g + 16 (lane % 8) .. + 15
    float v[16];
    {
        const int gg = live ? g : G - 1;                                  // spare lanes re-read a real group
        const u32x4* src = reinterpret_cast<const u32x4*>(w + row * K + (int64_t)gg * kGroup + 16 * (lane & 7));
        const u32x4 a = src[0], b = src[1];
        const uint32_t words[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const half2v h = as_h2(words[i]);
            v[2 * i] = (float)h[0];
            v[2 * i + 1] = (float)h[1];
        }
    }
    float lo = 0.f, hi = 0.f;     // the range always holds 0
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        lo = fminf(lo, v[i]);
        hi = fmaxf(hi, v[i]);
    }
    // the eight lanes of a group: butterfly over lane bits 0-2
#pragma unroll
    for (int m = 1; m < 8; m <<= 1) {
        lo = fminf(lo, __shfl_xor(lo, m));
        hi = fmaxf(hi, __shfl_xor(hi, m));
    }
    const float rng = fmaxf(hi - lo, 1e-5f);
    const _Float16 s16 = (_Float16)(rng / 15.0f);
    const float s = (float)s16;
    const float z = fminf(fmaxf(rintf(-lo / s), 0.f), 15.f);

    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float q = fminf(fmaxf(rintf(v[i] / s) + z, 0.f), 15.f);
        packed[i >> 3] |= (uint32_t)q << (4 * (i & 7));
    }
    if (live) {
        uint2* dst = reinterpret_cast<uint2*>(qpk + row * (K / 8) + (int64_t)g * 16 + 2 * (lane & 7));
        *dst = uint2{packed[0], packed[1]};
        if ((lane & 7) == 0) scales[row * G + g] = __builtin_bit_cast(uint16_t, s16);
    }
    // zero word: nibble j from the first lane of group j (0 past G)
    uint32_t zword = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float zj = __shfl(z, 8 * j);
        const uint32_t code = (zw * 8 + j < G) ? (uint32_t)zj : 0u;
        zword |= code << (4 * j);
    }
    if (lane == 0) zpk[row * ZW + zw] = zword;
}

}  // namespace

hipError_t launch_quantize(const uint16_t* w, uint32_t* qpk, uint16_t* scales, uint32_t* zpk, int64_t M, int64_t K,
                           hipStream_t stream) {
    const int32_t G = (int32_t)(K / kGroup), ZW = (G + 7) / 8;
    const int64_t nchunks = M * ZW;
    const unsigned blocks = (unsigned)((nchunks + 3) / 4);
    hipLaunchKernelGGL(quantize_kernel, dim3(blocks), dim3(256), 0, stream, w, qpk, scales, zpk, M, K, G, ZW);
    return hipGetLastError();
}

}  // namespace w4a16
