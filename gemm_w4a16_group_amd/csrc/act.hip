// Gated activation of the decoder layer's MLP on the fused gate/up
// projection's token-major output gu [N, 2 I] (gate in columns 0 .. I - 1,
// up in I .. 2 I - 1):  act[n, i] = fp16(silu(g) * u), silu(g) = g / (1 +
// exp(-g)), in float32.  One thread per 8 outputs: two 16-byte loads, one
// 16-byte store.  HBM-bound: 6 bytes per output.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

__device__ __forceinline__ float silu_times(float g, float u) { return g / (1.0f + expf(-g)) * u; }

__global__ void __launch_bounds__(256) silu_mul_kernel(const uint16_t* __restrict__ gu, uint16_t* __restrict__ act,
                                                       int64_t N, int64_t I) {
    const int64_t IC = I / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= N * IC) return;
    const int64_t n = t / IC, c = t % IC;
    const u32x4 g = reinterpret_cast<const u32x4*>(gu + n * 2 * I)[c];
    const u32x4 u = reinterpret_cast<const u32x4*>(gu + n * 2 * I + I)[c];
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2v gh = as_h2(gw[i]), uh = as_h2(uw[i]);
        const _Float16 lo = (_Float16)silu_times((float)gh[0], (float)uh[0]);
        const _Float16 hi = (_Float16)silu_times((float)gh[1], (float)uh[1]);
        o[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    reinterpret_cast<u32x4*>(act + n * I)[c] = u32x4{o[0], o[1], o[2], o[3]};
}

}  // namespace

hipError_t launch_silu_mul(const uint16_t* gu, uint16_t* act, int64_t N, int64_t I, hipStream_t stream) {
    const int64_t chunks = N * (I / 8);
    hipLaunchKernelGGL(silu_mul_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, gu, act, N, I);
    return hipGetLastError();
}

}  // namespace w4a16
