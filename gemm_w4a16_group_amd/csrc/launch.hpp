// Internal launchers of the W4A16 kernels (called by the C ABI in abi.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

struct GemmArgs {
    const uint32_t* qpk;      // [M, K/8]
    const uint16_t* scales;   // fp16 bits [M, G]
    const uint32_t* zpk;      // [M, ZW]
    const uint16_t* x;        // fp16 bits [K, N]
    uint16_t* xp;             // tiled kernel: X as 16-byte chunks [K/8][N] (workspace)
    uint16_t* c;              // fp16 bits [M, N]
    float* part;              // fp32 partial sums (splitk > 1): [splitk, M, N]; the tiled kernel keeps
                              //    [splitk, tiles, waves, its register layout]
    uint32_t* counters;       // one arrival counter per output tile (splitk > 1)
    int64_t M, N, K;
    int32_t G, ZW;
    int32_t tm;               // 1: token-major x [N, K] and c [N, M]
    int32_t xp_ready;         // 1: a.xp already holds the activation chunks (no rewrite before the GEMM)
    int32_t act;              // 1: x is a gate/up output [N, 2K] (token-major); the activations are
                              //    silu(gate) * up, formed while staging or rewriting them
    // residual add + RMSNorm while staging (skinny kernel, token-major, splitk 1): the
    // activations are rmsnorm(x + res) * gamma and h = fp16(x + res) is written to hout
    int32_t norm;
    float eps;
    const uint16_t* res;      // [N, K]
    const uint16_t* gamma;    // [K]
    uint16_t* hout;           // [N, K], must not alias x or res
};

// One decode step of multi-head attention (head dimension 128).
struct AttnArgs {
    const uint16_t* qkv;      // [B, 3 H D]: q | k | v of each sequence's new token
    uint16_t* k_cache;        // [B, H, S, D]
    uint16_t* v_cache;        // [B, H, S, D]
    const int32_t* pos;       // [B] position of the new token
    uint16_t* out;            // [B, H D]
    float* part;              // [B H, splits, D + 2] partial (o, max, sum) per split
    uint32_t* counters;       // one arrival counter per (sequence, head)
    int64_t S, max_len;       // cache capacity; bound on pos + 1 (<= S)
    int32_t B, H;
    double theta1;            // base^(-2 / D)
    float scale;              // softmax scale (1 / sqrt(D) in LLaMA)
};

struct SkinnyShape {
    int ncol, rb, wm, wk, splitk;
};

struct TiledShape {
    int bm, bn, splitk;
    int wm;    // waves along M: 4 (4 x 1), 2 (2 x 2) or 8 (8 x 1, bm = 512)
    int wpf;   // stages of weights loaded ahead: 1 or 2 (up to 4 with xpf > 1)
    int xpf;   // stages of activation chunks staged ahead: 1, or 2 or 3 (four-wave tiles up to 256 x 64)
    int wk;    // K slices: 1, or 2 (four-wave 128 x 64 / 128 x 128 tiles, xpf = 1, wpf <= 2)
};

struct NarrowShape {
    int ncol;     // staged columns: 16, 32 or 64 (>= N)
    int pf;       // groups of weights in flight per wave: 8 or 16
    int splitk;
    int rb;       // 16-row blocks per wave: 1 or 2
    int wk;       // waves along K per row block: 1, 2 or 4
    int wm;       // waves along M: 4, or 3 with wk = 1 (16 wm rb rows, 64 wm wk threads per workgroup)
};

bool skinny_supported(const SkinnyShape& s);
// nullptr if the skinny kernel can run this shape and plan, else the reason.
const char* skinny_check(const GemmArgs& a, const SkinnyShape& s);
int64_t skinny_row_tiles(const GemmArgs& a, const SkinnyShape& s);
int skinny_pf(const GemmArgs& a, const SkinnyShape& s);   // the kernel's PF template argument
hipError_t launch_skinny(const GemmArgs& a, const SkinnyShape& s, hipStream_t stream);

bool tiled_supported(const TiledShape& t);
// nullptr if the tiled kernel can run this shape, else the reason.
const char* tiled_check(const GemmArgs& a, const TiledShape& t);
int64_t tiled_tiles(const GemmArgs& a, const TiledShape& t);
// fp32 partial tiles of a split plan (whole tiles, in the waves' register layout)
size_t tiled_partial_bytes(const GemmArgs& a, const TiledShape& t);
size_t xpack_bytes(const GemmArgs& a);   // workspace the tiled kernel's activation chunks take
hipError_t launch_tiled(const GemmArgs& a, const TiledShape& t, hipStream_t stream);

bool narrow_supported(const NarrowShape& s);
// nullptr if the narrow kernel can run this shape and plan, else the reason.
const char* narrow_check(const GemmArgs& a, const NarrowShape& s);
int64_t narrow_row_tiles(const GemmArgs& a, const NarrowShape& s);
// fp32 partial tiles of a split plan (whole row tiles, ncol columns, register layout)
size_t narrow_partial_bytes(const GemmArgs& a, const NarrowShape& s);
size_t narrow_lds_bytes(const GemmArgs& a, const NarrowShape& s);
// true when the narrow kernel stages the activations straight from x ([K, N],
// N a multiple of 8), with no re-layout launch before it
bool narrow_direct_x(const GemmArgs& a);
// the tiled plan reads X [K, N] in place (no xpack_col launch)
bool tiled_direct_x(const GemmArgs& a, const TiledShape& t);
hipError_t launch_narrow(const GemmArgs& a, const NarrowShape& s, hipStream_t stream);

// X [K, N] -> 16-byte chunks [K/8][N] in a.xp (the tiled and narrow kernels' B/A operand layout)
hipError_t launch_xpack(const GemmArgs& a, hipStream_t stream);

// h = fp16(x + r), y = fp16(h * rsqrt(mean h^2 + eps) * gamma), token-major [N, K]; with chunks, y is
// written in the activation-chunk layout [K/8][N] of the tiled and narrow kernels
hipError_t launch_add_rmsnorm(const uint16_t* x, const uint16_t* r, const uint16_t* gamma, float eps, uint16_t* h,
                              uint16_t* y, int64_t N, int64_t K, bool chunks, hipStream_t stream);

// decode attention: a workgroup of `waves` waves (4 or 8; 16 with kpw 16) takes waves * kpw
// consecutive keys (kpw = 16, 32 or 64 keys per wave); splits along the keys at most kAttnMaxSplits
struct AttnShape {
    int kpw, waves;
};
constexpr int kAttnMaxSplits = 1024;
bool attn_shape_supported(const AttnShape& sh);
AttnShape attn_default_shape(const AttnArgs& a);
int64_t attn_splits(const AttnArgs& a, const AttnShape& sh);
hipError_t launch_decode_attn(const AttnArgs& a, const AttnShape& sh, hipStream_t stream);

// act [N, I] = fp16(silu(gate) * up) from gu [N, 2 I] (gate columns first); I % 8 == 0
hipError_t launch_silu_mul(const uint16_t* gu, uint16_t* act, int64_t N, int64_t I, hipStream_t stream);

// fp16 W [M, K] -> q_packed, fp16 scales, z_packed (round to nearest per group)
hipError_t launch_quantize(const uint16_t* w, uint32_t* qpk, uint16_t* scales, uint32_t* zpk, int64_t M, int64_t K,
                           hipStream_t stream);

// records `fmt` as the calling thread's w4a16_last_error() and returns status
int set_last_error(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// streaming-read probe: waves per workgroup `waves`, `loads` KB read per wave, one
// word stored per wave into sink[stream_read_waves(bytes, loads) rounded up to whole workgroups]
int64_t stream_read_waves(int64_t bytes, int loads);
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int waves, int loads,
                              hipStream_t stream);

hipError_t launch_pack_rows(const uint8_t* codes, uint32_t* words, int64_t rows, int64_t len,
                            hipStream_t stream);

}  // namespace w4a16
