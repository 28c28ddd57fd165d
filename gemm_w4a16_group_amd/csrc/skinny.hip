// Skinny W4A16 kernel: few activation columns (N <= 64), the bandwidth-bound
// regime of the PerfXLLM page on Snapdragon 8 Gen2, §3.3 (item 1 for few
// tokens, item 2 for one token).
//
// Every packed weight word is read from HBM exactly once, with 16-byte
// loads: eight lanes read one row's 128 bytes of a group pair, so one load
// instruction brings in eight rows x 128 bytes (whole lines); a per-wave LDS
// transpose then gives lane (r, kb) words 4kb .. 4kb+3 of row r's group,
// the MFMA layout (16-row x 64-byte loads straight into that layout stream
// about a fifth slower).
// The B operand of a 16x16x32 fp16 MFMA is made from each word with two
// masks and a shift and nothing else: a nibble q at bits 0-3 of a half is
// the fp16 subnormal q * 2^-24, a nibble at bits 4-7 is 16 q * 2^-24 (the
// matrix cores take subnormal inputs exactly).  The A operand is a 16-token
// block of the activations (tokens x k), staged per wave in LDS in the
// matching k order, with the k positions of the bits-4-7 nibbles divided by
// 16.  So one group's MFMAs give T = 2^-24 * sum_k q x exactly rounded in
// fp32, the group sums S = sum_k x come from the same staged activations
// (an MFMA with a constant operand), and the group adds
//     s * (q - z) . x = (s * 2^24) * T - (s * z) * S
// to the fp32 accumulator.  The product is C^T, so a lane's four
// accumulators are four tokens of the very row it loaded, and its scale and
// zero are per lane.  Scale and zero are staged in LDS, as §3.3 item 2 does.
//
// Work split (§3.3 item 2 tiles both dimensions of the weight matrix): a
// workgroup owns 16 * rb * wm rows and a run of groups; its wk waves along K
// each take a contiguous part of that run and are summed through LDS;
// `splitk` workgroups may share one row tile, their fp32 partials summed in
// a fixed order by the last one to arrive.
//
// Latency: all small loads (scales, zeros, activations) are issued before
// the weight loads, so that staging them never waits for the weight stream;
// up to PF groups of weights per wave are in flight at any time.
//
// Prologues (token-major activations, N <= 8), each its own kernel name so
// that the plain kernel's code is untouched: skinny_silu_kernel stages
// silu(gate) * up of a gate/up output; skinny_norm_kernel stages
// (x + res) * gamma and applies the RMS factor of each token to its sums in
// the epilogue, where the workgroup's sums of squares have met.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int kMaxThreads = 1024;
constexpr size_t kMaxLds = 160 * 1024;   // LDS per workgroup on gfx950
// One group pair of one wave's 16 rows (16 x 128 B), rows 8..15 placed one
// half bank-row later so that both the load-order writes and the MFMA-order
// reads touch all 64 banks: 17 slots of 128 B (row r at slot r + r / 8).
// Exactly that and no more, since LDS per wave decides how many workgroups
// a CU holds (eight waves at N = 4 fit three to a CU with it).
constexpr int kPairBytes = 17 * 128;
constexpr uint32_t kNormSumBytes = 16 * 8 * 4;   // [waves][8 columns] float sums of squares

// Activation columns the kernel is built for: any N <= 8, or 16 or 32.
__host__ __device__ constexpr bool ncol_ok(int n) {
    return (n >= 1 && n <= 8) || n == 16 || n == 32;
}

// Activation blocks (and scale slots) a lane stages per load: a wave of 64
// lanes stages PF groups = 16 PF octets of NB8 column-octets each, and four
// groups of scales per load.
__host__ __device__ constexpr int skinny_staging_loads(int NT, int PF) {
    const int v = (PF * (NT <= 8 ? 1 : NT / 8) + 3) / 4;
    return v > 0 ? v : 1;
}
// Largest PF per column count: staged activation registers F * min(NT, 8) * 4
// stay within 64 VGPRs and weight buffers within 64.
__host__ __device__ constexpr int skinny_max_pf(int NT) {
    return NT <= 4 ? 16 : NT <= 8 ? 8 : NT == 16 ? 4 : 2;
}

// Everything the kernel needs about a plan, computed on the host so that the
// kernel's prologue has no integer divisions ahead of its first loads.
struct SkinnyParams {
    int wm;                   // waves along M per workgroup
    int wk;                   // waves along K per workgroup
    int splitk;               // workgroups along K
    int rows;                 // rows per workgroup
    int sg_base, sg_rem;      // groups of split s: sg_base + (s < sg_rem)
    int wq0, wr0, wq1, wr1;   // per-wave share of sg_base / sg_base + 1 groups
    int ngw_max;              // groups per wave (upper bound)
    int zwt_max;              // zero words per row a wave stages (upper bound)
    int PF;                   // weight loads per lane = groups per wave (upper bound)
    int F;                    // staging loads per lane (scales, activations)
    uint32_t wave_bytes;      // one wave's LDS region
    uint32_t s_off, z_off;    // scale / zero-word offsets inside it
    uint32_t t_off;           // group-sum table offset inside it
    uint32_t q_off;           // the weight-transpose buffer inside it
    uint32_t flag_off, total; // arrival flag, total dynamic LDS
    uint32_t norm_off;        // per-wave column sums of squares (normalizing prologue), after the rest
};

// Every wave stages, in its own LDS region, what its groups need: the
// activations (NT columns; a 16-byte chunk holds eight k of one column,
// chunks ordered [k-octet][column]), the scales ([group][row] halves) and
// the zero words ([row][word]).  No wave waits for another before its main
// loop.  Returns false for a shape the kernel cannot run.
inline bool skinny_params(int NT, int G, int splitk, int rb, int wm, int wk, SkinnyParams& P) {
    if (wm < 1 || wk < 1 || splitk < 1 || splitk > G) return false;
    const int TB = (NT + 15) / 16;
    P.wm = wm;
    P.wk = wk;
    P.splitk = splitk;
    P.rows = 16 * rb * wm;
    P.sg_base = G / splitk;
    P.sg_rem = G % splitk;
    P.wq0 = P.sg_base / wk;
    P.wr0 = P.sg_base % wk;
    P.wq1 = (P.sg_base + 1) / wk;
    P.wr1 = (P.sg_base + 1) % wk;
    const int ngs_max = P.sg_base + (P.sg_rem > 0);
    P.ngw_max = (ngs_max + wk - 1) / wk;
    P.zwt_max = (P.ngw_max + 7) / 8 + 1;
    if (rb != 1 || P.zwt_max > 4) return false;
    // PF = groups of weights a wave keeps in flight = all of its groups
    P.PF = 2;
    while (P.PF < P.ngw_max) P.PF *= 2;
    P.F = skinny_staging_loads(NT, P.PF);
    if (P.PF > skinny_max_pf(NT)) return false;
    const size_t xb = (size_t)P.ngw_max * 16 * NT * 16;
    const size_t sb = (size_t)P.PF * 16 * 2;
    const size_t zb = (size_t)16 * 4 * 4;
    const size_t tb = (size_t)P.PF * NT * 4;
    P.s_off = (uint32_t)xb;
    P.z_off = (uint32_t)(P.s_off + ((sb + 15) & ~(size_t)15));
    P.t_off = (uint32_t)(P.z_off + ((zb + 15) & ~(size_t)15));
    P.q_off = (uint32_t)(P.t_off + ((tb + 15) & ~(size_t)15));
    const size_t wave_bytes = P.q_off + (size_t)kPairBytes;
    size_t main_bytes = wave_bytes * wm * wk;
    // partial sums of waves 1 .. wk-1, written after the staged data is dead
    const size_t red = (size_t)(wk - 1) * wm * rb * TB * 4 * 64 * 4;
    if (red > main_bytes) main_bytes = red;
    if (main_bytes + 16 > kMaxLds) return false;
    P.wave_bytes = (uint32_t)wave_bytes;
    P.flag_off = (uint32_t)main_bytes;
    P.total = (uint32_t)(main_bytes + 16);
    return true;
}

__device__ __forceinline__ uint32_t load_u16(const uint16_t* p) { return (uint32_t)*p; }

// The eight codes of one packed word as fp16 subnormals, in the k order
// 0, 4, 1, 5, 2, 6, 3, 7: k 0, 4, 2, 6 carry q * 2^-24, k 1, 5, 3, 7 carry
// 16 q * 2^-24 (the staged activations at those k are divided by 16).
__device__ __forceinline__ half8 codes8(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return __builtin_bit_cast(half8, u32x4{w & 0x000F000Fu, w & 0x00F000F0u,
                                           w8 & 0x000F000Fu, w8 & 0x00F000F0u});
}

// Constant B operand that sums the staged activations of each A row over a
// 32-k step: 1 at the k that were kept, 16 at the k that were divided by 16.
__device__ __forceinline__ half8 unscale_ones() {
    return __builtin_bit_cast(half8, u32x4{0x3C003C00u, 0x4C004C00u, 0x3C003C00u, 0x4C004C00u});
}

// Activation block: eight consecutive k (one octet) of T8 = min(NT, 8)
// columns, loaded with 16-byte loads.  With N == NT every block is 16-byte
// aligned: for NT <= 8 the block is 16 * NT contiguous bytes, otherwise
// eight rows of 16 bytes.  Token-major activations (x^T [N, K], NT <= 8):
// one 16-byte load per column, which is already that column's octet.  It becomes T8 LDS chunks, one per column, each
// holding the octet in the order 0, 4, 1, 5, 2, 6, 3, 7, with k 1, 5, 3, 7
// divided by 16 (exact unless the quotient is subnormal: then rounded once).
// silu(g) * u of two fp16 pairs, float32, rounded once to fp16 (the
// decoder layer's gated activation, computed while staging)
__device__ __forceinline__ uint32_t silu_mul_pair(uint32_t g, uint32_t u) {
    const half2v gh = as_h2(g), uh = as_h2(u);
    const float g0 = (float)gh[0], g1 = (float)gh[1];
    const _Float16 lo = (_Float16)(g0 / (1.0f + expf(-g0)) * (float)uh[0]);
    const _Float16 hi = (_Float16)(g1 / (1.0f + expf(-g1)) * (float)uh[1]);
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

template <int NT>
struct XStage {
    static constexpr int T8 = NT < 8 ? NT : 8;
    static constexpr int NB8 = NT <= 8 ? 1 : NT / 8;   // column octets
    u32x4 v[T8];
    u32x4 r[T8];   // normalizing prologue: the residual's octets
    u32x4 g;       //   and the gains of the octet

    // normalizing prologue (token-major, NT <= 8): x, the residual and the gains
    __device__ __forceinline__ void load_norm(const uint16_t* x, const uint16_t* res, const uint16_t* gamma,
                                              int64_t k0, int64_t K) {
#pragma unroll
        for (int t = 0; t < T8; ++t) {
            v[t] = *reinterpret_cast<const u32x4*>(x + (int64_t)t * K + k0);
            r[t] = *reinterpret_cast<const u32x4*>(res + (int64_t)t * K + k0);
        }
        g = *reinterpret_cast<const u32x4*>(gamma + k0);
    }

    template <bool ACT>
    __device__ __forceinline__ void load(const uint16_t* x, int64_t k0, int nb8, bool tm, int64_t K) {
        if (ACT && NT <= 8) {
            // x is the gate/up output [NT, 2K]: the octet is silu(gate) * up,
            // in float32, rounded once to fp16
#pragma unroll
            for (int t = 0; t < T8; ++t) {
                const u32x4 g = *reinterpret_cast<const u32x4*>(x + (int64_t)t * 2 * K + k0);
                const u32x4 u = *reinterpret_cast<const u32x4*>(x + (int64_t)t * 2 * K + K + k0);
                v[t] = u32x4{silu_mul_pair(g.x, u.x), silu_mul_pair(g.y, u.y), silu_mul_pair(g.z, u.z),
                             silu_mul_pair(g.w, u.w)};
            }
        } else if (NT <= 8) {
#pragma unroll
            for (int t = 0; t < T8; ++t) {
                const uint16_t* src = tm ? x + (int64_t)t * K + k0 : x + k0 * NT + 8 * t;
                v[t] = *reinterpret_cast<const u32x4*>(src);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 8; ++r)
                v[r] = *reinterpret_cast<const u32x4*>(x + (k0 + r) * NT + nb8 * 8);
        }
    }

    // 32-bit word e2 of the block image, row-major [8 rows][T8 columns] halves
    __device__ __forceinline__ uint32_t word(int e2) const {
        const int t = e2 >> 2, j = e2 & 3;
        return j == 0 ? v[t].x : j == 1 ? v[t].y : j == 2 ? v[t].z : v[t].w;
    }

    __device__ __forceinline__ void store(unsigned char* xs, int o, int nb8, bool tm) const {
        const half2v sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
        if (T8 == 1 || (NT <= 8 && tm)) {
#pragma unroll
            for (int c = 0; c < T8; ++c) {
                u32x4 r = permute_k8(v[c]);
                r.y = as_u32(as_h2(r.y) * sixteenth);
                r.w = as_u32(as_h2(r.w) * sixteenth);
                *reinterpret_cast<u32x4*>(xs + ((size_t)o * NT + c) * 16) = r;
            }
            return;
        }
#pragma unroll
        for (int c = 0; c < T8; ++c) {
            // pair (k r, k r+4) of column c: halves r*T8 + c and (r+4)*T8 + c
            uint32_t pr[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int e_lo = r * T8 + c, e_hi = (r + 4) * T8 + c;
                const uint32_t wl = word(e_lo >> 1), wh = word(e_hi >> 1);
                const uint32_t sel = ((e_lo & 1) ? 0x0302u : 0x0100u) | ((e_hi & 1) ? 0x07060000u : 0x05040000u);
                pr[r] = __builtin_amdgcn_perm(wh, wl, sel);
            }
            pr[1] = as_u32(as_h2(pr[1]) * sixteenth);
            pr[3] = as_u32(as_h2(pr[3]) * sixteenth);
            const int col = nb8 * 8 + c;
            *reinterpret_cast<u32x4*>(xs + ((size_t)o * NT + col) * 16) = u32x4{pr[0], pr[1], pr[2], pr[3]};
        }
    }
};

// Group sums of the staged activations for one column (NT == 1): lane b
// holds octet b of the wave's run; the sixteen octets of a group are sixteen
// consecutive lanes.  Sums in fp32, written to stab[group].
__device__ __forceinline__ void group_sums_one_column(const u32x4& v, int b, int nxb, float* stab) {
    // k 1, 5, 3, 7 of the staged chunk are divided by 16; sum the raw values
    const half2v one = {(_Float16)1.0f, (_Float16)1.0f};
    float t = 0.f;
    t = __builtin_amdgcn_fdot2(as_h2(v.x), one, t, false);
    t = __builtin_amdgcn_fdot2(as_h2(v.y), one, t, false);
    t = __builtin_amdgcn_fdot2(as_h2(v.z), one, t, false);
    t = __builtin_amdgcn_fdot2(as_h2(v.w), one, t, false);
    if (b >= nxb) t = 0.f;
    t += __shfl_xor(t, 1);
    t += __shfl_xor(t, 2);
    t += __shfl_xor(t, 4);
    t += __shfl_xor(t, 8);
    if ((b & 15) == 0 && b < nxb) stab[b >> 4] = t;
}

// MODE 1: the activations are silu(gate) * up of a gate/up output, formed
// while staging; MODE 2: they are rmsnorm(x + res) * gamma, the sum of
// squares of each column reduced over the workgroup (which covers all of K)
// while the weights are in flight.  Both token-major, NT <= 8.
template <int NT, int PF, int MODE>
__device__ __forceinline__ void skinny_body(const GemmArgs& a, const SkinnyParams& P) {
    constexpr bool ACT = MODE == 1, NORM = MODE == 2;
    constexpr int F = skinny_staging_loads(NT, PF); // activation loads per lane
    constexpr int TB = (NT + 15) / 16;              // 16-column MFMA blocks
    constexpr int NB8 = XStage<NT>::NB8;
    // only the first min(NT, 4) accumulators of a block can hold a real
    // column when NT < 4 (columns 4 kb + r with kb > 0 are past NT)
    constexpr int RMAX = NT < 4 ? NT : 4;
    constexpr int SZL = (PF + 3) / 4;               // scale loads per lane
    constexpr int NP = PF / 2;                      // group pairs per wave
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int M = (int)a.M, G = a.G;
    const int lane = threadIdx.x & 63;
    // wave-uniform (scalar) index, so that every per-wave loop bound and
    // branch below is uniform
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wave_k = wave / P.wm;               // scalar division, once
    const int wave_m = wave - wave_k * P.wm;
    const int nthreads = blockDim.x;
    const int li = lane & 15;     // weight row (B column) / column of x (A row)
    const int kb = lane >> 4;     // which quarter of the 32-k MFMA step

    unsigned char* wbase = smem + (size_t)wave * P.wave_bytes;
    unsigned char* xs = wbase;
    uint16_t* ss = reinterpret_cast<uint16_t*>(wbase + P.s_off);
    uint32_t* zsw = reinterpret_cast<uint32_t*>(wbase + P.z_off);
    float* stab = reinterpret_cast<float*>(wbase + P.t_off);
    unsigned char* qbuf = wbase + P.q_off;

    const int64_t row0 = (int64_t)blockIdx.x * P.rows + wave_m * 16;
    const int sidx = blockIdx.y;
    const int gs0 = sidx * P.sg_base + (sidx < P.sg_rem ? sidx : P.sg_rem);
    const bool big = sidx < P.sg_rem;
    const int wq = big ? P.wq1 : P.wq0, wr = big ? P.wr1 : P.wr0;
    const int gw0 = gs0 + wave_k * wq + (wave_k < wr ? wave_k : wr);
    const int ng = wq + (wave_k < wr ? 1 : 0);
    const int gw1 = gw0 + ng;
    const int glast = ng > 0 ? gw1 - 1 : (gw0 < G ? gw0 : G - 1);   // clamp target
    const int zw0 = gw0 >> 3;                     // first zero word of the wave
    const int zwt = ng > 0 ? ((gw1 - 1) >> 3) - zw0 + 1 : 1;
    int64_t lrow = row0 + li;                     // weight row of this lane (MFMA layout)
    lrow = lrow < M ? lrow : M - 1;

    // Loads are issued in the order their data is needed, and return in that
    // order: activations, scales and zeros first, then every group's
    // weights.  All loads are unconditional (indices clamped into range) so
    // that they issue back to back; stores to LDS are masked.
    // ---- 1. activations of the wave's groups: block b = lane + 64 j
    const int nxb = ng * 16 * NB8;
    XStage<NT> xst[F];
    int64_t k0s[F];   // normalizing prologue: where each block sits along K
#pragma unroll
    for (int j = 0; j < F; ++j) {
        int b = lane + j * 64;
        b = b < nxb ? b : (nxb > 0 ? nxb - 1 : 0);
        const int o = b / NB8, nb8 = b % NB8;     // NB8 is a power of two
        int64_t k0 = (int64_t)gw0 * kGroup + (int64_t)o * 8;
        k0 = k0 < a.K - 8 ? k0 : a.K - 8;
        k0s[j] = k0;
        if constexpr (NORM)
            xst[j].load_norm(a.x, a.res, a.gamma, k0, a.K);
        else
            xst[j].template load<ACT>(a.x, k0, nb8, a.tm != 0, a.K);
    }
    // ---- 2. scales: lane (row li, group 4 j + kb); zero words: lane (row
    // li, word kb)
    uint32_t sreg[SZL];
#pragma unroll
    for (int j = 0; j < SZL; ++j) {
        const int gl = 4 * j + kb;
        const int g = gw0 + gl < glast ? gw0 + gl : glast;
        sreg[j] = load_u16(a.scales + lrow * G + g);
    }
    uint32_t zreg;
    {
        const int w = zw0 + kb < a.ZW ? zw0 + kb : a.ZW - 1;
        zreg = a.zpk[lrow * a.ZW + w];
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- 3. weights, two groups (128 bytes of a row) per load: lane
    // (r = lane / 8, c = lane % 8) of half h reads 16 bytes c of the pair's
    // 128 bytes of row 8 h + r.  Eight lanes cover a whole 128-byte line.
    // Groups past the wave's run read a line every lane shares instead.
    const int lr = lane >> 3, lc = lane & 7;
    const u32x4* spare = reinterpret_cast<const u32x4*>(a.x);
    u32x4 buf[NP][2];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            int64_t row = row0 + 8 * h + lr;
            row = row < M ? row : M - 1;
            const int gl = 2 * pp + (lc >> 2);
            const u32x4* src = gl < ng ? reinterpret_cast<const u32x4*>(a.qpk + row * (a.K / 8) + (int64_t)(gw0 + gl) * 16 + (lc & 3) * 4)
                                       : spare;
            buf[pp][h] = __builtin_nontemporal_load(src);
        }
    __builtin_amdgcn_sched_barrier(0);

    // ---- 3b. normalizing prologue, while the weights are in flight: h =
    // fp16(x + res) per block (written out by the first row tile) and the
    // squares of h summed per column over the wave's blocks.  The factor
    // rsqrt(mean h^2 + eps) is one scalar per column, so it moves out of the
    // sum: the wave stages fp16(h * gamma * 2^e) and the epilogue multiplies
    // the column's sum by 2^-e (exact) and by the factor, once the sums of
    // squares of the waves along K have met behind the epilogue's barrier.
    // No wave waits for another before its main loop.  The power of two e
    // (per wave and column) brings the staged values of the wave's blocks
    // to unit mean square, so that their fp16 rounding is relative, as that
    // of the normalized activations is.
    float nscale[XStage<NT>::T8];   // 2^-e per column
    float nssq[XStage<NT>::T8];     // the wave's sums of squares, every lane
    if constexpr (NORM) {
        constexpr int T8 = XStage<NT>::T8;
        float ssq[T8];
#pragma unroll
        for (int t = 0; t < T8; ++t) ssq[t] = 0.f;
        const bool write_h = blockIdx.x == 0 && wave_m == 0;
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const bool live = lane + j * 64 < nxb;   // clamped duplicates count once
#pragma unroll
            for (int t = 0; t < T8; ++t) {
                const uint32_t xw[4] = {xst[j].v[t].x, xst[j].v[t].y, xst[j].v[t].z, xst[j].v[t].w};
                const uint32_t rw[4] = {xst[j].r[t].x, xst[j].r[t].y, xst[j].r[t].z, xst[j].r[t].w};
                uint32_t hw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const half2v xh = as_h2(xw[i]), rh = as_h2(rw[i]);
                    const _Float16 lo = (_Float16)((float)xh[0] + (float)rh[0]);
                    const _Float16 hi = (_Float16)((float)xh[1] + (float)rh[1]);
                    if (live) {
                        ssq[t] = fmaf((float)lo, (float)lo, ssq[t]);
                        ssq[t] = fmaf((float)hi, (float)hi, ssq[t]);
                    }
                    hw[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                xst[j].v[t] = u32x4{hw[0], hw[1], hw[2], hw[3]};
                if (write_h && live)
                    *reinterpret_cast<u32x4*>(a.hout + (int64_t)t * a.K + k0s[j]) = xst[j].v[t];
            }
        }
        float* nsum = reinterpret_cast<float*>(smem + P.norm_off);
        int ex[T8];
#pragma unroll
        for (int t = 0; t < T8; ++t) {
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) ssq[t] += __shfl_xor(ssq[t], m);
            if (lane == 0) nsum[wave * 8 + t] = ssq[t];
            nssq[t] = ssq[t];
            // mean square of the wave's values in [2^(E-1), 2^E): e = -floor(E / 2)
            const float ms = ssq[t] / (float)(ng > 0 ? ng * kGroup : 1);
            int e = ms > 0.f ? -(__builtin_amdgcn_frexp_expf(ms) >> 1) : 0;
            e = e < 60 ? (e > -60 ? e : -60) : 60;
            ex[t] = e;
            nscale[t] = __builtin_ldexpf(1.0f, -e);
        }
#pragma unroll
        for (int j = 0; j < F; ++j) {
            const uint32_t gw[4] = {xst[j].g.x, xst[j].g.y, xst[j].g.z, xst[j].g.w};
#pragma unroll
            for (int t = 0; t < T8; ++t) {
                const uint32_t hw[4] = {xst[j].v[t].x, xst[j].v[t].y, xst[j].v[t].z, xst[j].v[t].w};
                uint32_t yw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const half2v hh = as_h2(hw[i]), gg = as_h2(gw[i]);
                    // h * gamma is exact in float32; the power of two too
                    const _Float16 lo = (_Float16)__builtin_ldexpf((float)hh[0] * (float)gg[0], ex[t]);
                    const _Float16 hi = (_Float16)__builtin_ldexpf((float)hh[1] * (float)gg[1], ex[t]);
                    yw[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
                }
                xst[j].v[t] = u32x4{yw[0], yw[1], yw[2], yw[3]};
            }
        }
    }

    // ---- 4. stage activations, scales and zeros; group sums
    // S[g][t] = sum of the group's 128 activations of column t
#pragma unroll
    for (int j = 0; j < F; ++j) {
        const int b = lane + j * 64;
        if (b < nxb) xst[j].store(xs, b / NB8, b % NB8, a.tm != 0);
    }
#pragma unroll
    for (int j = 0; j < SZL; ++j) {
        const int gl = 4 * j + kb;
        if (gl < ng) ss[gl * 16 + li] = (uint16_t)sreg[j];
    }
    if (kb < zwt) zsw[li * 4 + kb] = zreg;
    if (NT == 1) {
#pragma unroll
        for (int j = 0; j < F; ++j) group_sums_one_column(xst[j].v[0], lane + j * 64, nxb, stab);
    }
    // LDS accesses of one wave complete in order; the fences keep the
    // compiler from moving later reads above these writes
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (NT > 1) {
        // rows of A are (group, column) pairs q = g * NT + t, sixteen per
        // MFMA, times a constant operand
        const half8 ones = unscale_ones();
        const int nq = ng * NT;
        for (int q0 = 0; q0 < nq; q0 += 16) {
            int q = q0 + li;
            q = q < nq ? q : nq - 1;
            const int gq = q / NT, tq = q - gq * NT;
            floatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const half8 xa = *reinterpret_cast<const half8*>(xs + ((size_t)(gq * 16 + kb * 4 + i) * NT + tq) * 16);
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, ones, d, 0, 0, 0);
            }
            if (li == 0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (q0 + kb * 4 + r < nq) stab[q0 + kb * 4 + r] = d[r];
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // ---- 5. per group pair, as its weights arrive: through LDS into the
    // MFMA layout (lane (j = row, kb) takes 16 bytes kb of the group), then
    // per group T = 2^-24 sum_k q x on the matrix cores and
    //   acc += s * (q - z) . x = (s * 2^24) * T - (s * z) * S
    int tok[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        const int t = tb * 16 + li;
        tok[tb] = t < NT ? t : NT - 1;          // rows of A past NT repeat a staged one
    }
    floatx4 acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // slot of 16-byte chunk c of pair row r: (r + r / 8) * 128 + (c ^ (r % 8)) * 16
    const int wslot0 = (lr + 0) * 128 + ((lc ^ lr) * 16);          // half 0: rows 0..7
    const int wslot1 = (8 + lr + 1) * 128 + ((lc ^ lr) * 16);      // half 1: rows 8..15
    const int rbase = (li + (li >> 3)) * 128;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
        if (2 * pp < ng) {
            // one transpose buffer: a wave's LDS accesses complete in
            // order, so these writes cannot overtake the previous pair's
            // reads; the fences keep the compiler from moving them up
            unsigned char* qb = qbuf;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            *reinterpret_cast<u32x4*>(qb + wslot0) = buf[pp][0];
            *reinterpret_cast<u32x4*>(qb + wslot1) = buf[pp][1];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int p = 2 * pp + e;
                if (p < ng) {
                    const u32x4 wv = *reinterpret_cast<const u32x4*>(qb + rbase + (((4 * e + kb) ^ (li & 7)) * 16));
                    const int g = gw0 + p;
                    const uint32_t zw = zsw[li * 4 + (g >> 3) - zw0];
                    const float z = (float)((zw >> (4 * (g & 7))) & 0xFu);
                    const float sc = (float)__builtin_bit_cast(_Float16, ss[p * 16 + li]);
                    const float sa = sc * 16777216.0f;   // undoes the 2^-24 of the subnormal codes
                    const float sz = sc * z;
                    floatx4 part[TB];
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) part[tb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t word = i == 0 ? wv.x : i == 1 ? wv.y : i == 2 ? wv.z : wv.w;
                        const half8 wb = codes8(word);
                        const size_t obase = (size_t)(p * 16 + kb * 4 + i) * NT;
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) {
                            const half8 xa = *reinterpret_cast<const half8*>(xs + (obase + tok[tb]) * 16);
                            part[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa, wb, part[tb], 0, 0, 0);
                        }
                    }
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                        for (int r = 0; r < RMAX; ++r) {
                            int t = tb * 16 + kb * 4 + r;
                            t = t < NT ? t : NT - 1;
                            const float v = __builtin_fmaf(sa, part[tb][r], acc[tb][r]);
                            acc[tb][r] = __builtin_fmaf(-sz, stab[p * NT + t], v);
                        }
                }
            }
        }
    }

    // ---- 6. sum the wk waves of a row block through LDS
    const int wm = P.wm, wk = P.wk, splitk = P.splitk;
    if constexpr (NORM) {
        // undo the wave's power of two (exact) before the waves meet
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                int t = tb * 16 + kb * 4 + r;
                t = t < NT ? t : NT - 1;
                acc[tb][r] *= nscale[t < XStage<NT>::T8 ? t : 0];
            }
    }
    if (wk > 1) {
        __syncthreads();   // every wave is done with its staged data
        float* red = reinterpret_cast<float*>(smem);
        if (wave_k > 0) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int r = 0; r < RMAX; ++r) {
                    const size_t idx = (((((size_t)(wave_k - 1) * wm + wave_m) * TB + tb) * 4 + r) * 64) + lane;
                    red[idx] = acc[tb][r];
                }
        }
        __syncthreads();
        if (wave_k == 0) {
            for (int kk = 1; kk < wk; ++kk) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int r = 0; r < RMAX; ++r) {
                        const size_t idx = (((((size_t)(kk - 1) * wm + wave_m) * TB + tb) * 4 + r) * 64) + lane;
                        acc[tb][r] += red[idx];
                    }
            }
        }
    }

    // ---- 7. epilogue: lane holds columns 16 tb + 4 kb + r of row row0 + li
    const int N = NT;
    const int64_t row = row0 + li;
    if constexpr (NORM) {
        // the normalization factor of each column, from the sums of squares
        // of the waves along K in K order (after the barriers above; a wave
        // alone along K has its own)
        constexpr int T8 = XStage<NT>::T8;
        const float* nsum = reinterpret_cast<const float*>(smem + P.norm_off);
        float rs[T8];
#pragma unroll
        for (int t = 0; t < T8; ++t) {
            float tot = nssq[t];
            if (wk > 1) {
                tot = 0.f;
                for (int k = 0; k < wk; ++k) tot += nsum[(k * wm + wave_m) * 8 + t];
            }
            rs[t] = 1.0f / sqrtf(tot / (float)a.K + a.eps);
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < RMAX; ++r) {
                int t = tb * 16 + kb * 4 + r;
                t = t < NT ? t : NT - 1;
                acc[tb][r] *= rs[t < T8 ? t : 0];
            }
    }
    if (wave_k == 0 && row < M) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t0 = tb * 16 + kb * 4;
            if (splitk == 1 && a.tm) {
                // token-major output: consecutive lanes hold consecutive rows
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (t0 + r < N) a.c[(t0 + r) * M + row] = (uint16_t)f32_to_h16_bits(acc[tb][r]);
            } else if (splitk == 1) {
                if ((N & 3) == 0 && t0 + 3 < N) {
                    const uint32_t lo = f32_to_h16_bits(acc[tb][0]) | (f32_to_h16_bits(acc[tb][1]) << 16);
                    const uint32_t hi = f32_to_h16_bits(acc[tb][2]) | (f32_to_h16_bits(acc[tb][3]) << 16);
                    *reinterpret_cast<uint2*>(a.c + row * N + t0) = uint2{lo, hi};
                } else {
#pragma unroll
                    for (int r = 0; r < RMAX; ++r)
                        if (t0 + r < N) a.c[row * N + t0 + r] = (uint16_t)f32_to_h16_bits(acc[tb][r]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    if (t0 + r < N)
                        __hip_atomic_store(a.part + ((int64_t)sidx * M + row) * N + t0 + r, acc[tb][r],
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (splitk == 1) return;

    // ---- 8. split-K: the last workgroup of a row tile sums the partials in
    // order.  Partials are written and read with agent-scope relaxed atomics.
    // Every thread waits until its partial stores have completed, the
    // workgroup meets, and one thread adds one to the tile's counter
    // (relaxed, agent scope); the barrier after it puts the last arriver's
    // loads after that add.  This ordering holds without an agent-scope
    // release or acquire: the partials are written and read only with
    // agent-coherent accesses (sc1, the instructions of agent-scope
    // atomics), an sc1 store has reached agent coherence once the load
    // counter shows it complete, and the barriers' fences keep the compiler
    // from moving the stores after the add or the loads before it.  A
    // release or acquire at agent scope would add a write-back (release) or
    // an invalidation (acquire) of the whole L2 of the workgroup's XCD;
    // the write-backs, one per workgroup, made plans with two to eight
    // splits up to five times slower.
    int* flag = reinterpret_cast<int*>(smem + P.flag_off);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == (unsigned)(splitk - 1);
        if (last) {
            __hip_atomic_store(a.counters + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *flag = last;
    }
    __syncthreads();
    if (!*flag) return;
    const int64_t tile0 = (int64_t)blockIdx.x * P.rows;
    const int64_t rows_here = (M - tile0) < P.rows ? (M - tile0) : P.rows;
    const int64_t total = rows_here * N;
    for (int64_t e = threadIdx.x; e < total; e += nthreads) {
        const int64_t rr = tile0 + e / N;
        const int64_t col = e - (e / N) * N;
        float v = 0.f;
        for (int s = 0; s < splitk; ++s)
            v += __hip_atomic_load(a.part + ((int64_t)s * M + rr) * N + col, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        a.c[a.tm ? col * M + rr : rr * N + col] = (uint16_t)f32_to_h16_bits(v);
    }
}

template <int NT, int PF>
__global__ void __launch_bounds__(kMaxThreads) skinny_kernel(GemmArgs a, SkinnyParams P) {
    skinny_body<NT, PF, 0>(a, P);
}

template <int NT, int PF>
__global__ void __launch_bounds__(kMaxThreads) skinny_silu_kernel(GemmArgs a, SkinnyParams P) {
    skinny_body<NT, PF, 1>(a, P);
}

template <int NT, int PF>
__global__ void __launch_bounds__(kMaxThreads) skinny_norm_kernel(GemmArgs a, SkinnyParams P) {
    skinny_body<NT, PF, 2>(a, P);
}

template <int NT, int PF, int MODE>
hipError_t launch_kernel(const GemmArgs& a, const SkinnyShape& s, const SkinnyParams& P, hipStream_t stream) {
    const void* fn;
    if constexpr (MODE == 1)
        fn = reinterpret_cast<const void*>(&skinny_silu_kernel<NT, PF>);
    else if constexpr (MODE == 2)
        fn = reinterpret_cast<const void*>(&skinny_norm_kernel<NT, PF>);
    else
        fn = reinterpret_cast<const void*>(&skinny_kernel<NT, PF>);
    dim3 grid((unsigned)((a.M + P.rows - 1) / P.rows), (unsigned)s.splitk);
    dim3 block((unsigned)(64 * s.wm * s.wk));
    // dynamic LDS above 64 KB must be allowed per kernel, once
    static const hipError_t lds_ok = [fn] {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
        if (e != hipSuccess) (void)hipGetLastError();   // keep a refusal out of later launches' status
        return e;
    }();
    if (lds_ok != hipSuccess && P.total > 65536) return lds_ok;
    if constexpr (MODE == 1)
        hipLaunchKernelGGL((skinny_silu_kernel<NT, PF>), grid, block, P.total, stream, a, P);
    else if constexpr (MODE == 2)
        hipLaunchKernelGGL((skinny_norm_kernel<NT, PF>), grid, block, P.total, stream, a, P);
    else
        hipLaunchKernelGGL((skinny_kernel<NT, PF>), grid, block, P.total, stream, a, P);
    return hipGetLastError();
}

template <int NT, int PF>
hipError_t launch_one(const GemmArgs& a, const SkinnyShape& s, const SkinnyParams& P, hipStream_t stream) {
    if constexpr (NT <= 8) {
        if (a.act) return launch_kernel<NT, PF, 1>(a, s, P, stream);
        if (a.norm) {
            SkinnyParams Q = P;
            Q.norm_off = (P.total + 15u) & ~15u;
            Q.total = Q.norm_off + kNormSumBytes;
            return launch_kernel<NT, PF, 2>(a, s, Q, stream);
        }
    }
    return launch_kernel<NT, PF, 0>(a, s, P, stream);
}

template <int NT>
hipError_t launch_nt(const GemmArgs& a, const SkinnyShape& s, hipStream_t stream) {
    SkinnyParams P;
    if (!skinny_params(NT, a.G, s.splitk, s.rb, s.wm, s.wk, P)) return hipErrorInvalidValue;
    constexpr int cap = skinny_max_pf(NT);
    switch (P.PF) {
        case 2: return launch_one<NT, 2>(a, s, P, stream);
        case 4: return launch_one<NT, (cap >= 4 ? 4 : 2)>(a, s, P, stream);
        case 8: return launch_one<NT, (cap >= 8 ? 8 : 2)>(a, s, P, stream);
        case 16: return launch_one<NT, (cap >= 16 ? 16 : 2)>(a, s, P, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool skinny_supported(const SkinnyShape& s) {
    return ncol_ok(s.ncol) && s.rb == 1 && s.wm >= 1 &&
           s.wk >= 1 && s.wm * s.wk <= kMaxThreads / 64 && s.splitk >= 1;
}

int64_t skinny_row_tiles(const GemmArgs& a, const SkinnyShape& s) {
    const int64_t rows = 16LL * s.rb * s.wm;
    return (a.M + rows - 1) / rows;
}

const char* skinny_check(const GemmArgs& a, const SkinnyShape& s) {
    if (!skinny_supported(s))
        return "ncol must be 1..8, 16, 32 or 64, rb 1, wm * wk <= 16";
    if (s.splitk > a.G) return "splitk exceeds the number of groups";
    if (a.tm && a.N > 8) return "token-major activations only for N <= 8";
    if (a.act && !a.tm) return "the gated activation prologue needs token-major activations";
    if (a.norm) {
        if (!a.tm || a.N > 8) return "the normalizing prologue needs token-major activations and N <= 8";
        if (s.splitk != 1) return "the normalizing prologue needs splitk 1 (a workgroup covers all of K)";
    }
    SkinnyParams P;
    if (!skinny_params(s.ncol, a.G, s.splitk, s.rb, s.wm, s.wk, P))
        return "a wave's groups exceed its load registers, or the staged data the workgroup's LDS; "
               "add waves along K or splits";
    if (a.norm && ((P.total + 15u) & ~15u) + kNormSumBytes > (uint32_t)kMaxLds)
        return "the normalizing prologue's sums do not fit in LDS";
    return nullptr;
}

int skinny_pf(const GemmArgs& a, const SkinnyShape& s) {
    SkinnyParams P;
    if (!skinny_params(s.ncol, a.G, s.splitk, s.rb, s.wm, s.wk, P)) return 0;
    return P.PF;
}

hipError_t launch_skinny(const GemmArgs& a, const SkinnyShape& s, hipStream_t stream) {
    if (a.N != s.ncol) return hipErrorInvalidValue;
    switch (s.ncol) {
        case 1: return launch_nt<1>(a, s, stream);
        case 2: return launch_nt<2>(a, s, stream);
        case 3: return launch_nt<3>(a, s, stream);
        case 4: return launch_nt<4>(a, s, stream);
        case 5: return launch_nt<5>(a, s, stream);
        case 6: return launch_nt<6>(a, s, stream);
        case 7: return launch_nt<7>(a, s, stream);
        case 8: return launch_nt<8>(a, s, stream);
        case 16: return launch_nt<16>(a, s, stream);
        case 32: return launch_nt<32>(a, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
