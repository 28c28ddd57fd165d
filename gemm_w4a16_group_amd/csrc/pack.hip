// Packing of 4-bit codes into 32-bit words (storage of PerfXLLM §3.1: int4
// weights, one zero per group of 128).  Eight codes per word along the row,
// code j of a word in bits 4j..4j+3; padding nibbles past the row end are 0.
#include "launch.hpp"

namespace w4a16 {

// One thread per output word.  `codes` is uint8 [rows, len]; `words` is
// uint32 [rows, ceil(len / 8)].
__global__ void __launch_bounds__(256) pack_rows_kernel(const uint8_t* __restrict__ codes,
                                                        uint32_t* __restrict__ words,
                                                        int64_t rows, int64_t len, int64_t nwords) {
    const int64_t total = rows * nwords;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = t / nwords;
        const int64_t w = t - r * nwords;
        const uint8_t* src = codes + r * len + w * 8;
        const int64_t left = len - w * 8;
        uint32_t v = 0;
        if (left >= 8 && (((uintptr_t)src) & 7) == 0) {
            uint2 b = *reinterpret_cast<const uint2*>(src);
            // gather the low nibble of each byte: byte j -> bits 4j..4j+3
            uint32_t lo = b.x & 0x0F0F0F0Fu;   // bytes 0..3
            uint32_t hi = b.y & 0x0F0F0F0Fu;   // bytes 4..7
            lo = (lo | (lo >> 4)) & 0x00FF00FFu;
            lo = (lo | (lo >> 8)) & 0x0000FFFFu;
            hi = (hi | (hi >> 4)) & 0x00FF00FFu;
            hi = (hi | (hi >> 8)) & 0x0000FFFFu;
            v = lo | (hi << 16);
        } else {
            const int n = left < 8 ? (int)left : 8;
            for (int j = 0; j < n; ++j) v |= (uint32_t)(src[j] & 0xF) << (4 * j);
        }
        words[t] = v;
    }
}

hipError_t launch_pack_rows(const uint8_t* codes, uint32_t* words, int64_t rows, int64_t len,
                            hipStream_t stream) {
    const int64_t nwords = (len + 7) / 8;
    const int64_t total = rows * nwords;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(pack_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, codes, words,
                       rows, len, nwords);
    return hipGetLastError();
}

}  // namespace w4a16
