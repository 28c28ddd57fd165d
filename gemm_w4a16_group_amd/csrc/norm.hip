// Residual add + RMS normalization, token-major (the first fusion of §3.2 of
// the PerfXLLM page: the residual network's addition and the normalization
// as one operator; the normalization read as LLaMA's RMSNorm):
//
//   h = fp16(x + r)                                 the stored residual stream
//   y = fp16(h * rsqrt(mean_k h^2 + eps) * gamma)   the next projection's input
//
// x, r, h: [N, K] fp16 row-major; gamma: [K] fp16.  One workgroup of 256
// threads per token.  A thread owns the 16-byte chunks c = tid + 256 i of its
// token: it reads x and r once, writes h, keeps h in registers for the first
// kNormRegChunks chunks (K <= 16384 never re-reads anything) and squares the
// stored fp16 values into a float32 sum.  Wave sums meet in LDS; every thread
// then scales its chunks.  y goes either to a row-major [N, K] buffer or,
// for the chunk-staging GEMM kernels, straight into their activation layout
// (chunk (ko, n) = the eight k of octet ko of token n in the order 0, 4, 1,
// 5, 2, 6, 3, 7), so the normalized activations never exist in any other
// form.  HBM-bound: 2 + 2 bytes read and 2 + 2 written per element.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int kNormThreads = 256;
constexpr int kNormRegChunks = 8;

// fp16 sum of two fp16 pairs, rounded once: float32 holds x + r with at most
// one rounding that cannot change the fp16 result (24 >= 2 * 11 + 2 bits).
__device__ __forceinline__ uint32_t add_pair(uint32_t a, uint32_t b, float& ss) {
    const half2v ha = as_h2(a), hb = as_h2(b);
    const _Float16 lo = (_Float16)((float)ha[0] + (float)hb[0]);
    const _Float16 hi = (_Float16)((float)ha[1] + (float)hb[1]);
    const float flo = (float)lo, fhi = (float)hi;
    ss = fmaf(flo, flo, ss);
    ss = fmaf(fhi, fhi, ss);
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__device__ __forceinline__ uint32_t scale_pair(uint32_t h, uint32_t g, float rs) {
    const half2v hh = as_h2(h), gg = as_h2(g);
    const _Float16 lo = (_Float16)((float)hh[0] * rs * (float)gg[0]);
    const _Float16 hi = (_Float16)((float)hh[1] * rs * (float)gg[1]);
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <bool CHUNKS>
__global__ void __launch_bounds__(kNormThreads) add_rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                                   const uint16_t* r, const uint16_t* __restrict__ gamma,
                                                                   float eps, uint16_t* h, uint16_t* __restrict__ y,
                                                                   int64_t N, int64_t K) {
    // r and h may be the same buffer (in-place update of the stream): every
    // chunk is read before the same thread writes it
    __shared__ float wsum[kNormThreads / 64];
    const int64_t n = blockIdx.x;
    const int tid = threadIdx.x;
    const int64_t KC = K / 8;
    const u32x4* xr = reinterpret_cast<const u32x4*>(x + n * K);
    const u32x4* rr = reinterpret_cast<const u32x4*>(r + n * K);
    u32x4* hr = reinterpret_cast<u32x4*>(h + n * K);
    const u32x4* gr = reinterpret_cast<const u32x4*>(gamma);

    // the gains of the register window are loaded with x and r, so the
    // second pass waits on no memory
    u32x4 hv[kNormRegChunks], gv[kNormRegChunks];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kNormRegChunks; ++i) {
        const int64_t c = tid + (int64_t)kNormThreads * i;
        if (c < KC) {
            const u32x4 a = xr[c], b = rr[c];
            gv[i] = gr[c];
            u32x4 s;
            s.x = add_pair(a.x, b.x, ss);
            s.y = add_pair(a.y, b.y, ss);
            s.z = add_pair(a.z, b.z, ss);
            s.w = add_pair(a.w, b.w, ss);
            hr[c] = s;
            hv[i] = s;
        }
    }
    for (int64_t c = tid + (int64_t)kNormThreads * kNormRegChunks; c < KC; c += kNormThreads) {
        const u32x4 a = xr[c], b = rr[c];
        u32x4 s;
        s.x = add_pair(a.x, b.x, ss);
        s.y = add_pair(a.y, b.y, ss);
        s.z = add_pair(a.z, b.z, ss);
        s.w = add_pair(a.w, b.w, ss);
        hr[c] = s;
    }
    // wave sum (butterfly over the 64 lanes), then the four waves in LDS
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m);
    if ((tid & 63) == 0) wsum[tid >> 6] = ss;
    __syncthreads();
    const float total = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
    const float rs = 1.0f / sqrtf(total / (float)K + eps);

    auto emit = [&](int64_t c, const u32x4& hc, const u32x4& g) {
        u32x4 o;
        o.x = scale_pair(hc.x, g.x, rs);
        o.y = scale_pair(hc.y, g.y, rs);
        o.z = scale_pair(hc.z, g.z, rs);
        o.w = scale_pair(hc.w, g.w, rs);
        if (CHUNKS)
            reinterpret_cast<u32x4*>(y)[c * N + n] = permute_k8(o);
        else
            reinterpret_cast<u32x4*>(y + n * K)[c] = o;
    };
#pragma unroll
    for (int i = 0; i < kNormRegChunks; ++i) {
        const int64_t c = tid + (int64_t)kNormThreads * i;
        if (c < KC) emit(c, hv[i], gv[i]);
    }
    // chunks past the register window: read back this thread's own h
    for (int64_t c = tid + (int64_t)kNormThreads * kNormRegChunks; c < KC; c += kNormThreads) emit(c, hr[c], gr[c]);
}

}  // namespace

hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* gamma, float eps, uint16_t* h,
                              uint16_t* y, int64_t N, int64_t K, bool chunks, hipStream_t stream) {
    if (chunks)
        hipLaunchKernelGGL(add_rmsnorm_kernel<true>, dim3((unsigned)N), dim3(kNormThreads), 0, stream, x, r, gamma,
                           eps, h, y, N, K);
    else
        hipLaunchKernelGGL(add_rmsnorm_kernel<false>, dim3((unsigned)N), dim3(kNormThreads), 0, stream, x, r,
                           gamma, eps, h, y, N, K);
    return hipGetLastError();
}

}  // namespace w4a16
