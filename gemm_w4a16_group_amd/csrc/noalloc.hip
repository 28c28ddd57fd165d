// w4a16_gemm without a caller workspace, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The split-K partial sums, arrival counters and activation
// chunks that w4a16_gemm keeps in the caller's workspace live here in one
// file-scope device array of fixed size, `scratch`; each GPU the library
// runs on holds its own copy until the process ends.
//
// Host code never passes `scratch` itself (its host-side name is not a
// device address): the first call on a device, with that device current,
// looks up the array's device address with hipGetSymbolAddress and keeps
// it per device, clears the arrival counters there once with a fill kernel
// on the caller's stream (every kernel leaves them at zero again), and
// every call hands that address to w4a16_gemm as its workspace.  Nothing
// here calls hipMalloc, hipFree or any allocating routine.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/w4a16.h"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // 16 MiB per GPU
constexpr size_t kCounterBytesNa = 64 << 10;         // arrival counters at the start of a workspace
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ void __launch_bounds__(256) zero_words_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;       // device address of this device's `scratch`
    hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

}  // namespace

}  // namespace w4a16

using namespace w4a16;

extern "C" size_t w4a16_gemm_noalloc_max_bytes(void) { return kScratchBytes; }

extern "C" int w4a16_gemm_noalloc(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed,
                                  const void* x, void* c, int64_t M, int64_t N, int64_t K, int32_t group_size,
                                  void* stream) {
    // shape checks first (w4a16_gemm_workspace_size is 0 for a bad shape,
    // which w4a16_gemm then rejects with its own message)
    const size_t need = w4a16_gemm_workspace_size(M, N, K, group_size);
    if (need > kScratchBytes)
        return set_last_error(W4A16_ERR_WORKSPACE,
                              "this shape needs %zu bytes of scratch, above the %zu bytes w4a16_gemm_noalloc holds "
                              "per GPU; call w4a16_gemm with a workspace",
                              need, kScratchBytes);
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return set_last_error(W4A16_ERR_HIP, "no current device (%s)", hipGetErrorString(e));
    DeviceScratch& d = g_scratch[dev];
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::call_once(d.once, [&] {
        void* p = nullptr;
        d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (d.err != hipSuccess) return;
        const int64_t words = (int64_t)(kCounterBytesNa / 4);
        hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, s,
                           static_cast<uint32_t*>(p), words);
        d.err = hipGetLastError();
        if (d.err == hipSuccess) d.ptr = p;
    });
    if (!d.ptr)
        return set_last_error(W4A16_ERR_HIP, "device scratch unavailable on device %d: %s", dev,
                              hipGetErrorString(d.err));
    return w4a16_gemm(q_packed, scales, z_packed, x, c, M, N, K, group_size, d.ptr, kScratchBytes, stream);
}
