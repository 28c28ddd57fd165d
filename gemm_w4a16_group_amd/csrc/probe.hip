// Streaming-read probe: the attainable HBM rate of one launch that reads a
// buffer once, in the decode GEMV's own launch shape.  It is the floor the
// memory-bound kernels of the PerfXLLM page on Snapdragon 8 Gen2 (§3.3
// item 2: the GEMV is memory-bound, its efficiency is that of its memory
// accesses) are measured against, not part of the layer.
//
// A workgroup of `waves` waves reads a contiguous L KB per wave (L
// non-temporal 16-byte loads per lane, each instruction one 1 KB run; the
// GEMV's shape is L = 4), all loads issued before any is used, XORs what it
// read and stores one word per wave, so that no load can be dropped and the
// kernel ends with a store, as the GEMV does.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

template <int kProbeLoads>
__global__ void __launch_bounds__(1024) stream_read_kernel(const u32x4* __restrict__ src, uint32_t* __restrict__ sink,
                                                           int64_t n16) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t wave_id = (int64_t)blockIdx.x * (blockDim.x >> 6) + wave;
    const int64_t base = wave_id * 64 * kProbeLoads + lane;
    u32x4 v[kProbeLoads];
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) {
        int64_t i = base + (int64_t)j * 64;
        i = i < n16 ? i : n16 - 1;
        v[j] = __builtin_nontemporal_load(src + i);
    }
    uint32_t x = 0;
#pragma unroll
    for (int j = 0; j < kProbeLoads; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x ^= __shfl_xor(x, m);
    if (lane == 0) sink[wave_id] = x;
}

template <int L>
hipError_t launch_l(const void* buf, int64_t n16, uint32_t* sink, int waves, hipStream_t stream) {
    const int64_t nw = (n16 + 64 * L - 1) / (64 * L);
    const int64_t blocks = (nw + waves - 1) / waves;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_read_kernel<L>, dim3((unsigned)blocks), dim3(64 * waves), 0, stream,
                       static_cast<const u32x4*>(buf), sink, n16);
    return hipGetLastError();
}

}  // namespace

int64_t stream_read_waves(int64_t bytes, int loads) { return (bytes / 16 + 64 * loads - 1) / (64 * loads); }

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int waves, int loads,
                              hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    if (n16 < 1) return hipErrorInvalidValue;
    switch (loads) {
        case 1: return launch_l<1>(buf, n16, sink, waves, stream);
        case 2: return launch_l<2>(buf, n16, sink, waves, stream);
        case 4: return launch_l<4>(buf, n16, sink, waves, stream);
        case 8: return launch_l<8>(buf, n16, sink, waves, stream);
        case 16: return launch_l<16>(buf, n16, sink, waves, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
