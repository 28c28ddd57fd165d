// Tiled W4A16 kernel for many activation columns: the compute-bound regime
// of the PerfXLLM page on Snapdragon 8 Gen2, §3.3 item 1 (many tokens),
// which blocks the product into tiles held in shared memory.
//
// Two launches.  xpack_col_kernel rewrites the activations X [K, N] (N
// contiguous) once into 16-byte chunks, chunk (ko, n) holding the eight k of
// octet ko of column n in the order 0, 4, 1, 5, 2, 6, 3, 7 that the
// dequantized weight words use (xpack_tm_kernel for token-major X^T [N, K],
// xpack_silu_kernel for a gate/up output; the normalizing prologue writes
// the chunks itself).  The chunks are exactly the B operand of
// v_mfma_f32_32x32x16_f16, so the GEMM stages them into LDS with
// buffer-to-LDS loads (no registers, no shuffles, contiguous LDS writes) and
// reads them back conflict-free.  The default tiles (96 x 64, 128 x 64,
// 128 x 128, 256 x 128, 512 x 128) read [K, N] activations in place instead
// when N is a multiple of 8 (tiled_dx_kernel, tiled_k2_dx_kernel): each k-octet's
// eight rows are copied into LDS in the dequant order (16-byte pieces
// permuted per row against bank conflicts) and two transposing LDS reads
// give a lane its B fragment, with no second launch.
//
// tiled_kernel: a workgroup of NWV waves (four, eight for 512-row tiles,
// three for 96-row ones) owns a BM x BN tile of C and walks K one group
// (128 k) per stage.  The
// waves form a WGM x (NWV / WGM) grid.  tiled_k2_kernel doubles the
// workgroup into two such grids along K: at stage p the first takes group
// 2p, the second group 2p + 1 of the split's run, both behind the same
// barrier, and the second's sums join the first's through LDS at the end,
// so that few-column tiles (one workgroup per CU) keep two waves on every
// SIMD with no dequantization done twice.  Each wave loads the packed weight
// words of its rows straight into registers (32 bytes per lane per 32-row
// block and stage, one or two stages ahead) and dequantizes them there, one
// MFMA step ahead, to fp16 (q - z) * s: one fp16 rounding per weight, q - z
// being exact before the scale is applied.  fp32 accumulation throughout.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int kStageRows = kGroup / 8;   // k-octets per stage

typedef short short4v __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// X [K, N] -> chunks [K/8][N] of 16 bytes: one thread per chunk (ko, n),
// eight 2-byte loads down column n (consecutive threads take consecutive
// columns, so each load instruction reads a contiguous run of a row) and
// one 16-byte store (consecutive threads write consecutive chunks).  At
// N = 4096 this moved the 67 MB faster than one thread per 8 x 8 block with
// register transposes (16-byte loads, but each store instruction strided
// 128 bytes across lanes), and at N <= 32 it keeps the chip busy.
__global__ void __launch_bounds__(256) xpack_col_kernel(const uint16_t* __restrict__ x, u32x4* __restrict__ xp,
                                                        int64_t K, int64_t N) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (K / 8) * N) return;
    const int64_t ko = t / N, n = t % N;
    const uint16_t* src = x + ko * 8 * N + n;
    uint32_t h[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) h[r] = src[r * N];
    // k order 0, 4, 1, 5, 2, 6, 3, 7
    xp[t] = u32x4{h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16), h[3] | (h[7] << 16)};
}

// Token-major X^T [N, K] -> the same chunks.  Chunk (ko, n) is the 16 bytes
// X^T[n][8 ko .. 8 ko + 7], reordered, so this is a transpose of a [N][K/8]
// matrix of 16-byte elements.  A workgroup moves a 16 x 16 block through LDS
// so that both its reads (16 chunks of one token, 256 contiguous bytes) and
// its writes (16 tokens of one k-octet) are 256-byte runs; rows of 17
// elements keep the LDS stores of consecutive threads on distinct banks.
// K / 8 is a multiple of 16; tokens past N are skipped.
__global__ void __launch_bounds__(256) xpack_tm_kernel(const uint16_t* __restrict__ xt, u32x4* __restrict__ xp,
                                                       int64_t K, int64_t N) {
    __shared__ u32x4 tile[16 * 17];
    const int64_t KO = K / 8;
    const int64_t kob = KO / 16;
    const int64_t ko0 = ((int64_t)blockIdx.x % kob) * 16, n0 = ((int64_t)blockIdx.x / kob) * 16;
    const int t = threadIdx.x, lo = t & 15, hi = t >> 4;
    if (n0 + hi < N)
        tile[lo * 17 + hi] = permute_k8(*reinterpret_cast<const u32x4*>(xt + (n0 + hi) * K + (ko0 + lo) * 8));
    __syncthreads();
    if (n0 + lo < N) xp[(ko0 + hi) * N + n0 + lo] = tile[hi * 17 + lo];
}

// The same transpose from a gate/up output gu [N, 2K] (token-major): the
// chunks hold silu(gate) * up, formed in float32 and rounded once to fp16.
__device__ __forceinline__ uint32_t silu_mul_h2(uint32_t g, uint32_t u) {
    const half2v gh = as_h2(g), uh = as_h2(u);
    const float g0 = (float)gh[0], g1 = (float)gh[1];
    const _Float16 lo = (_Float16)(g0 / (1.0f + expf(-g0)) * (float)uh[0]);
    const _Float16 hi = (_Float16)(g1 / (1.0f + expf(-g1)) * (float)uh[1]);
    return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

__global__ void __launch_bounds__(256) xpack_silu_kernel(const uint16_t* __restrict__ gu, u32x4* __restrict__ xp,
                                                         int64_t K, int64_t N) {
    __shared__ u32x4 tile[16 * 17];
    const int64_t KO = K / 8;
    const int64_t kob = KO / 16;
    const int64_t ko0 = ((int64_t)blockIdx.x % kob) * 16, n0 = ((int64_t)blockIdx.x / kob) * 16;
    const int t = threadIdx.x, lo = t & 15, hi = t >> 4;
    if (n0 + hi < N) {
        const uint16_t* row = gu + (n0 + hi) * 2 * K + (ko0 + lo) * 8;
        const u32x4 g = *reinterpret_cast<const u32x4*>(row);
        const u32x4 u = *reinterpret_cast<const u32x4*>(row + K);
        tile[lo * 17 + hi] = permute_k8(u32x4{silu_mul_h2(g.x, u.x), silu_mul_h2(g.y, u.y), silu_mul_h2(g.z, u.z),
                                              silu_mul_h2(g.w, u.w)});
    }
    __syncthreads();
    if (n0 + lo < N) xp[(ko0 + hi) * N + n0 + lo] = tile[hi * 17 + lo];
}

// ---------------------------------------------------------------------------
// NWV waves per workgroup (4, 8, or 3 for 96 x 64 tiles, whose 16 activation
// copies per stage fall six to a wave with the last two repeated) in a
// WGM x (NWV / WGM) grid.  Weights are
// loaded WPF stages ahead into WPF + 1 register sets; activation chunks XPF
// stages ahead into a ring of XPF + 1 LDS buffers.  Every stage issues its
// activation loads, then its weight loads, and ends by waiting for exactly
// what the next stage reads (loads return in issue order, so the wait
// leaves the later stages' loads in flight), then one barrier.  Deep
// pipelines matter where a workgroup's stage is short (few columns): its
// MFMA work then covers only a fraction of the memory latency.
// Waves per SIMD the register budget is held to: two when a wave's
// accumulators take at most 128 registers (so two waves fit in the 512),
// else one.
__host__ __device__ constexpr int tiled_waves_per_simd(int BM, int BN, int WGM, int NWV) {
    return (BM / WGM / 32) * (BN / (NWV / WGM) / 32) * 16 <= 128 ? 2 : 1;
}

// Loads that may stay outstanding at the end of a stage: those issued after
// the later of the next stage's activation chunks and weights.
__host__ __device__ constexpr int tiled_vmcnt(int WPF, int XPF, int XL, int WL) {
    return XPF >= WPF ? (WPF - 1) * (XL + WL) : WL + (XPF - 1) * (XL + WL);
}

__host__ __device__ constexpr int tiled_lds_bytes(int BN, int XPF, int WKS = 1) {
    return (XPF + 1) * WKS * kStageRows * BN * 16;
}

// Prefetch distances built for a tile: (1, 1) and (2, 1) everywhere; deeper
// pipelines for four waves along M and tiles of at most 256 x 64 outputs,
// as long as a wave never has more than 63 loads outstanding (the load
// counter's range).
__host__ __device__ constexpr bool tiled_pipe_ok(int BM, int BN, int WGM, int NWV, int WPF, int XPF) {
    const int xl = kStageRows * BN / 64 / NWV, wl = 4 * (BM / WGM / 32);
    if (XPF == 1) return WPF == 1 || WPF == 2;
    const bool pair = (XPF == 2 && WPF >= 2 && WPF <= 4) || (XPF == 3 && (WPF == 3 || WPF == 4));
    return pair && NWV == 4 && WGM == 4 && BN <= 128 && BM * BN <= 256 * 64 && (XPF + WPF) * (xl + wl) < 64;
}

// Two K slices are built for four-wave grids of tiles up to 128 x 128 with
// one or two stages of weights and one of activations.
__host__ __device__ constexpr bool tiled_k2_ok(int BM, int BN, int WGM, int NWV, int WPF, int XPF) {
    return NWV == 4 && WGM == 4 && BM == 128 && BN <= 128 && XPF == 1 && WPF <= 2;
}

template <int BM, int BN, int WGM, int NWV, int WPF, int XPF, int WKS, bool DX = false>
__device__ __forceinline__ void tiled_body(const GemmArgs& a, int splitk) {
    constexpr int WGN = NWV / WGM;          // waves along N
    constexpr int WM = BM / WGM;            // rows per wave
    constexpr int WN = BN / WGN;            // columns per wave
    constexpr int RBW = WM / 32;            // 32-row MFMA blocks per wave
    constexpr int CBW = WN / 32;            // 32-column MFMA blocks per wave
    constexpr int XBYTES = kStageRows * BN * 16;        // one stage of activation chunks
    constexpr int XTOT = kStageRows * BN / 64;          // 1 KB buffer-to-LDS loads per stage
    constexpr int XLOADS = (XTOT + NWV - 1) / NWV;      // per wave (three waves: two copies repeat the last)
    constexpr int NSET = WPF + 1;                       // weight register sets
    constexpr int NXB = XPF + 1;                        // activation buffers
    constexpr int WLOADS = 4 * RBW;                     // weight, zero and scale loads per wave and stage
    constexpr int VMW = tiled_vmcnt(WPF, XPF, XLOADS, WLOADS);
    constexpr int SLOT = RBW * CBW * 16 * 64;           // accumulator floats per wave
    // MFMA steps the B fragments are read ahead: as many as 32 more
    // registers allow with the wave's accumulators at 32 or 64 per lane
    constexpr int BD = RBW * CBW <= 2 ? 4 : RBW * CBW <= 4 ? 2 : 1;
    static_assert(BN % 64 == 0 && XLOADS >= 1 && XLOADS % (BN / 64) == 0, "tile");
    static_assert(XLOADS * NWV == XTOT || BN == 64, "uneven copies only with one column base");
    static_assert(WKS == 1 || WKS == 2, "waves along K");
    static_assert((WKS - 1) * NWV * SLOT * 4 <= tiled_lds_bytes(BN, XPF, WKS), "K-slice sums fit the ring");
    static_assert(WPF >= 1 && WPF <= 4 && XPF >= 1 && XPF <= 3, "prefetch distances");
    static_assert(VMW < 64, "vmcnt");
    // dynamic LDS: NXB x WKS activation buffers ([stage slot][K slice])
    extern __shared__ __attribute__((aligned(16))) unsigned char xs[];
    __shared__ int flag;

    const int64_t M = a.M, N = a.N, K = a.K;
    const int G = a.G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_k = wave_all / NWV;   // K slice
    const int wave = wave_all - wave_k * NWV;
    const int wave_m = wave / WGN, wave_n = wave % WGN;
    const int l32 = lane & 31;     // A row / B column / C column inside a 32-block
    const int hh = lane >> 5;      // which half of the 16-k MFMA step

    // ---- tile of this workgroup: XCD-contiguous, then grouped along M
    const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
    const int64_t T = ntm * ntn;
    int64_t L = blockIdx.x;
    if (T % 8 == 0) L = (L % 8) * (T / 8) + L / 8;
    constexpr int64_t GM = 8;
    const int64_t group = L / (GM * ntn);
    const int64_t first_m = group * GM;
    const int64_t gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
    const int64_t tm = first_m + (L % (GM * ntn)) % gsz;
    const int64_t tn = (L % (GM * ntn)) / gsz;
    const int64_t row0 = tm * BM, col0 = tn * BN;
    const int64_t tile_id = tm * ntn + tn;

    // groups [st0, st1) of 128 k; stage p (0 .. P - 1) takes group
    // st0 + WKS p + wave_k in K slice wave_k
    const int sidx = blockIdx.y;
    const int st0 = (int)((int64_t)G * sidx / splitk);
    const int st1 = (int)((int64_t)G * (sidx + 1) / splitk);
    const int P = (st1 - st0 + WKS - 1) / WKS;
    auto group_of = [&](int p) { return st0 + WKS * p + wave_k; };
    const int64_t KW = K / 8;

    // ---- weights of this lane: row row0 + WM wave_m + 32 rb + l32, words
    // 8 hh .. 8 hh + 7 of each group's sixteen.  Buffer resources start at the
    // tile's first row so that per-lane offsets stay small; the stage moves
    // the scalar offset only.
    const int64_t rows_left = M - row0;
    const int64_t tile_rows = rows_left < BM ? rows_left : BM;
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(a.qpk + row0 * KW, tile_rows * KW * 4);
    const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(a.scales + row0 * G, tile_rows * G * 2);
    const __amdgpu_buffer_rsrc_t zres = buffer_rsrc(a.zpk + row0 * a.ZW, tile_rows * a.ZW * 4);
    int woff[RBW], soff[RBW], zoff[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
        int r = WM * wave_m + 32 * rb + l32;
        r = r < tile_rows ? r : (int)tile_rows - 1;
        woff[rb] = (int)((r * KW + 8 * hh) * 4);
        soff[rb] = (int)(r * G * 2);
        zoff[rb] = (int)(r * a.ZW * 4);
    }

    // ---- activation chunks: load i of wave w fills LDS chunks
    // [64 (w XLOADS + i), +64) of the stage, i.e. chunk row
    // (64 (w XLOADS + i)) / BN, columns (64 (w XLOADS + i)) % BN + lane.
    // Columns past N re-read column N - 1 (they reach only output columns
    // that are never stored).
    constexpr int NCB = BN / 64;    // distinct column bases
    int xcoff[NCB];
#pragma unroll
    for (int c = 0; c < NCB; ++c) {
        int64_t n = col0 + 64 * c + lane;
        n = n < N ? n : N - 1;
        xcoff[c] = (int)(n * 16);
    }
    const int xrow = (int)(N * 16);   // bytes per chunk row

    // weight words, zero word and scale of a stage, in NSET register sets
    // used in turn (the stage loop is unrolled NSET times, so no copies)
    u32x4 wS[NSET][RBW][2];
    uint32_t zS[NSET][RBW], sS[NSET][RBW];

    auto load_w = [&](int g, int set) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb) {
            wS[set][rb][0] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rb], g * 64, 0);
            wS[set][rb][1] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rb] + 16, g * 64, 0);
            zS[set][rb] = __builtin_amdgcn_raw_buffer_load_b32(zres, zoff[rb], (g >> 3) * 4, 0);
            sS[set][rb] = __builtin_amdgcn_raw_buffer_load_b16(sres, soff[rb], g * 2, 0);
        }
    };
    // X read in place ([K, N] rows, N a multiple of 8; DX): the stage's
    // octet o (k rows 8 o .. 8 o + 7 of the group) holds its eight rows of
    // the tile's BN columns in dequant order (k offsets 0, 4, 1, 5, 2, 6, 3,
    // 7), so that two transposing reads of four rows give a lane one
    // column's eight k in the order the chunks hold them.  Row p keeps its
    // 16-byte pieces (8 columns each) in slots permuted by an XOR with
    // 4 dx_swz(p), so that the four rows a transposing read takes fall on
    // distinct banks (without it their starts coincide: BN x 2 bytes apart).
    // Copy i of an octet fills its bytes [1024 i, 1024 i + 1024): lane l
    // fills slot q = 64 i + l, row q / (BN / 8), with the row's piece
    // (q % (BN / 8)) ^ 4 dx_swz(row) (pieces past N re-read the row's last).
    constexpr int XPO = BN / 64;    // copies per octet
    auto dx_swz = [](int p) { return BN == 64 ? (p >> 1) & 1 : p & 3; };
    int dxoff[XPO];
    if constexpr (DX) {
        const int n8 = (int)(N >> 3);
#pragma unroll
        for (int i = 0; i < XPO; ++i) {
            const int q = 64 * i + lane;
            const int pr = q / (BN / 8), cc = (q % (BN / 8)) ^ (4 * dx_swz(pr));
            const int r = (pr >> 1) + 4 * (pr & 1);
            int c8 = (int)(col0 >> 3) + cc;
            c8 = c8 < n8 ? c8 : n8 - 1;
            dxoff[i] = (int)((r * N + 8 * (int64_t)c8) * 2);
        }
    }
    // stage p's chunks go to buffer p % NXB of the wave's K slice
    auto load_x = [&](int g, int slot) {
        unsigned char* buf = xs + (slot * WKS + wave_k) * XBYTES;
        if constexpr (DX) {
            const i32x4 xres = raw_rsrc(a.x + (int64_t)g * 128 * N, (int64_t)128 * N * 2);
#pragma unroll
            for (int i = 0; i < XLOADS; ++i) {
                int idx = wave * XLOADS + i;
                if constexpr (XLOADS * NWV != XTOT) idx = idx < XTOT ? idx : XTOT - 1;
                // copy idx: octet idx / XPO, part idx % XPO (XLOADS is a
                // multiple of XPO, so the part depends on i only)
                buffer_load_lds16(xres, buf + idx * 1024, dxoff[i % XPO], (idx / XPO) * 8 * (int)N * 2);
            }
            return;
        }
        const i32x4 xres = raw_rsrc(a.xp + (int64_t)g * kStageRows * N * 8, (int64_t)kStageRows * N * 16);
#pragma unroll
        for (int i = 0; i < XLOADS; ++i) {
            // XLOADS is a multiple of NCB, so the column base depends on i only
            int idx = wave * XLOADS + i;
            if constexpr (XLOADS * NWV != XTOT) idx = idx < XTOT ? idx : XTOT - 1;
            const int chunk = 64 * idx;
            const int row = chunk / BN, cb = i % NCB;
            buffer_load_lds16(xres, buf + chunk * 16, xcoff[cb], row * xrow);
        }
    };

    floatx16 acc[RBW][CBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rb][cb][e] = 0.f;

    Dequant dq[RBW];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) dq[rb].init();
    // B fragment of lane (l32, hh), block cb, MFMA step t: chunk row 8 hh + t,
    // column WN wave_n + 32 cb + l32 -> one base plus an immediate offset
    const int bbase = ((8 * hh) * BN + WN * wave_n + l32) * 16;
    // DX: lanes 4 j .. 4 j + 3 of a 16-lane group read row 4 h + j of the
    // octet, columns base + 4 (lane % 4) ..; the transpose hands lane i of
    // the group column base + i of the four rows (the second 16 lanes of a
    // half-wave take the block's columns 16 .. 31).  Rows j and 4 + j share
    // their piece permutation, so one column offset per block serves both
    // reads.
    const int dxj = (lane & 15) >> 2;
    const int dxbase = ((8 * hh) * 8 * BN + dxj * BN) * 2;
    int dxcol[CBW];
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) {
        const int col = WN * wave_n + 32 * cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        dxcol[cb] = (((col >> 3) ^ (4 * dx_swz(dxj))) * 8 + (col & 7)) * 2;
    }
    const int last = st1 - 1;
    auto clamp_g = [&](int g) { return g < st1 ? g : last; };

    // One stage p (weights in register set `set`): prefetch the chunks of
    // stage p + XPF into the buffer stage p - 1 used and the weights of stage
    // p + WPF into the set stage p - 1 used (groups past the run clamped to
    // the last group, which then loads itself again into a buffer or set
    // nobody reads any more), then 8 MFMA steps on stage p's group (none
    // past the run: the second K slice of an odd run's last stage), then
    // wait for what the next stage reads and meet.
    auto stage = [&](int p, int set) {
        const int g = group_of(p);
        load_x(clamp_g(group_of(p + XPF)), (p + XPF) % NXB);
        __builtin_amdgcn_sched_barrier(0);
        load_w(clamp_g(group_of(p + WPF)), (set + WPF) % NSET);
        // keep every load of the next stage at the top of this one
        __builtin_amdgcn_sched_barrier(0);
        if (WKS == 1 || g < st1) {   // (the second slice of an odd run's last stage has no group)
            // scale and zero of this group
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb) dq[rb].set((zS[set][rb] >> (4 * (g & 7))) & 0xFu, sS[set][rb]);

            const unsigned char* xb = xs + ((p % NXB) * WKS + wave_k) * XBYTES + (DX ? dxbase : bbase);
            // A operand of MFMA step t: word t of the lane's eight (k-octet
            // 8 hh + t), dequantized one step ahead.  B fragments are read
            // BD steps ahead: one step of MFMA work is shorter than an LDS
            // read's latency, so reading one step ahead left every step
            // waiting on LDS.
            half8 afrag[2][RBW], bfrag[BD + 1][CBW];
            auto read_b = [&](int t, half8* bf) {
#pragma unroll
                for (int cb = 0; cb < CBW; ++cb) {
                    if constexpr (DX) {
                        const unsigned char* b = xb + dxcol[cb] + t * 8 * BN * 2;
                        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) short4v*)(b));
                        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (__attribute__((address_space(3))) short4v*)(b + 4 * BN * 2));
                        bf[cb] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                    } else {
                        bf[cb] = *reinterpret_cast<const half8*>(xb + (t * BN + cb * 32) * 16);
                    }
                }
            };
            auto make_a = [&](int t, half8* af) {
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb) af[rb] = dq[rb](wS[set][rb][t >> 2][t & 3]);
            };
#pragma unroll
            for (int t = 0; t < BD; ++t) read_b(t, bfrag[t]);
            make_a(0, afrag[0]);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t + BD < 8) read_b(t + BD, bfrag[(t + BD) % (BD + 1)]);
                if (t < 7) make_a(t + 1, afrag[(t + 1) & 1]);
#pragma unroll
                for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                    for (int cb = 0; cb < CBW; ++cb)
                        acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            afrag[t & 1][rb], bfrag[t % (BD + 1)][cb], acc[rb][cb], 0, 0, 0);
            }
        }
        // the next stage's chunks have landed in LDS (and its weights in
        // registers) and every wave is done with this stage's buffer;
        // vmcnt(VMW), expcnt and lgkmcnt left alone
        __builtin_amdgcn_s_waitcnt((VMW & 15) | ((VMW >> 4) << 14) | (7 << 4) | (15 << 8));
        __syncthreads();
        // each stage is its own scheduling region (no stage's registers
        // live into the next)
        __builtin_amdgcn_sched_barrier(0);
    };

    // every split has at least one group (splitk <= G).  The prologue issues
    // what the stages before the first would have: for j = -D .. -1, the
    // chunks of stage j + XPF and the weights of stage j + WPF (those at or
    // after stage 0), so that the waits below count the same loads as in the
    // loop
    constexpr int D = XPF > WPF ? XPF : WPF;
#pragma unroll
    for (int j = -D; j < 0; ++j) {
        if (j + XPF >= 0) {
            load_x(clamp_g(group_of(j + XPF)), (j + XPF) % NXB);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (j + WPF >= 0) {
            load_w(clamp_g(group_of(j + WPF)), (j + WPF) % NSET);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __builtin_amdgcn_s_waitcnt((VMW & 15) | ((VMW >> 4) << 14) | (7 << 4) | (15 << 8));
    __syncthreads();
    // whole rounds of NSET stages, then the rest (so that every path back
    // to the loop head has the same loads in flight)
    int p0 = 0;
    for (; p0 + NSET <= P; p0 += NSET) {
#pragma unroll
        for (int j = 0; j < NSET; ++j) stage(p0 + j, j);
    }
#pragma unroll
    for (int j = 0; j < NSET - 1; ++j)
        if (p0 + j < P) stage(p0 + j, j);
    // the last stages' own reloads may still be in flight
    __builtin_amdgcn_s_waitcnt(0);

    // ---- the second K slice's sums join the first's, in LDS over the
    // activation ring: every wave is past its last read of it (each stage
    // ends with a barrier), and after this barrier past its last reload
    // into it (each has waited for its own loads above)
    if constexpr (WKS > 1) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(xs);
        if (wave_k == 1) {
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        red[(size_t)wave * SLOT + ((rb * CBW + cb) * 16 + e) * 64 + lane] = acc[rb][cb][e];
        }
        __syncthreads();
        if (wave_k == 0) {
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                for (int cb = 0; cb < CBW; ++cb)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        acc[rb][cb][e] += red[(size_t)wave * SLOT + ((rb * CBW + cb) * 16 + e) * 64 + lane];
        }
    }
    // from here on only the first slice's waves hold sums; the second's
    // still meet at every barrier below
    const bool holder = wave_k == 0;

    // ---- epilogue: lane holds rows (e / 4) * 8 + 4 hh + e % 4, column l32
    // (token-major output: the four consecutive rows e = 4 j .. 4 j + 3 of a
    // column are one 8-byte store).  [M, N] output: each store instruction
    // writes two 64-byte row runs, which non-temporal stores handle well
    // (1.3 % faster at N = 4096); the token-major stores are 8 bytes each,
    // M apart between lanes, and need the L2 to merge them (non-temporal
    // ones made that path 36 % slower), so they stay ordinary.
    auto store_c = [&](int rb, int cb, const floatx16& v) {
        const int64_t col = col0 + WN * wave_n + cb * 32 + l32;
        if (col >= N) return;
        if (a.tm) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t row = row0 + WM * wave_m + 32 * rb + j * 8 + 4 * hh;
                if ((M & 3) == 0 && row + 3 < M) {
                    uint2 u;
                    u.x = f32_to_h16_bits(v[4 * j]) | (f32_to_h16_bits(v[4 * j + 1]) << 16);
                    u.y = f32_to_h16_bits(v[4 * j + 2]) | (f32_to_h16_bits(v[4 * j + 3]) << 16);
                    *reinterpret_cast<uint2*>(a.c + col * M + row) = u;
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (row + i < M) a.c[col * M + row + i] = (uint16_t)f32_to_h16_bits(v[4 * j + i]);
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = row0 + WM * wave_m + 32 * rb + (e >> 2) * 8 + 4 * hh + (e & 3);
                if (row < M) __builtin_nontemporal_store((uint16_t)f32_to_h16_bits(v[e]), &a.c[row * N + col]);
            }
        }
    };
    if (splitk == 1) {
        if (holder) {
#pragma unroll
            for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
                for (int cb = 0; cb < CBW; ++cb) store_c(rb, cb, acc[rb][cb]);
        }
        return;
    }

    // ---- split-K: every split stores its fp32 partial tile; the last
    // workgroup of a tile to arrive adds them in split order, its own from
    // its registers, and stores C.  A partial tile is kept in the waves'
    // register layout ([wave][block][element quad][lane], 1 KB contiguous
    // per quad and wave, a private slot per split and tile), so that every
    // access is one coalesced 16-byte-per-lane store or load and no lane
    // needs a mask (4-byte accesses, four times as many, made the merge
    // of a 4-way split take 10 us).
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
    constexpr int kAgent = 16;                      // cache policy sc1
    const __amdgpu_buffer_rsrc_t pres = buffer_rsrc(a.part, (int64_t)splitk * T * NWV * SLOT * 4);
    auto slot_off = [&](int s, int rb, int cb) {     // uniform byte offset of a block
        return (int)(((((int64_t)s * T + tile_id) * NWV + wave) * SLOT + (rb * CBW + cb) * 16 * 64) * 4);
    };
    // within a block, elements 4 j .. 4 j + 3 of lane l at byte 1024 j + 16 l
    const int lo = lane * 16;
    if (holder) {
#pragma unroll
        for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int cb = 0; cb < CBW; ++cb) {
                const int so = slot_off(sidx, rb, cb);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        u32x4{f32_bits(acc[rb][cb][4 * j]), f32_bits(acc[rb][cb][4 * j + 1]),
                              f32_bits(acc[rb][cb][4 * j + 2]), f32_bits(acc[rb][cb][4 * j + 3])},
                        pres, lo + j * 1024, so, kAgent);
            }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + tile_id, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const int is_last = prev == (unsigned)(splitk - 1);
        if (is_last) {
            __hip_atomic_store(a.counters + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        flag = is_last;
    }
    __syncthreads();
    if (!flag || !holder) return;
    // the sum runs in split order, (p_0 + ... + p_(sidx-1)) + own +
    // p_(sidx+1) + ..., the order of a plain left-to-right sum whichever
    // split arrives last.  The partials of KQ splits for BG blocks are
    // loaded together before any is added (one round trip to memory per
    // split and block, taken one after another, made the merge slow).
    auto load_part = [&](int s, int rb, int cb) {
        const int so = slot_off(s, rb, cb);
        floatx16 p;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // (the whole vector is reinterpreted: this compiler turns a
            // bit_cast of one element of a loaded vector into a load of
            // element 0 alone)
            const floatx4 f =
                __builtin_bit_cast(floatx4, __builtin_amdgcn_raw_buffer_load_b128(pres, lo + j * 1024, so, kAgent));
            p[4 * j] = f[0];
            p[4 * j + 1] = f[1];
            p[4 * j + 2] = f[2];
            p[4 * j + 3] = f[3];
        }
        return p;
    };
    constexpr int NB = RBW * CBW;                   // blocks per wave
    // blocks merged together and the most splits loaded together: eight
    // loads in flight for up to two blocks per wave, four for four; tiles
    // with more blocks keep one at a time (their sums fill the registers)
    constexpr int BG = NB <= 4 && NB % 2 == 0 ? 2 : 1;
    constexpr int KQ = NB >= 8 ? 1 : NB >= 4 ? 2 : 4;
    // the other splits, o = 0 .. splitk - 2, in order: split o, or o + 1
    // from this split's own index on
    const int n_other = splitk - 1;
#pragma unroll
    for (int b0 = 0; b0 < NB; b0 += BG) {
        floatx16 pre[BG];
        auto add = [&](int s, int g, const floatx16& v) {
            floatx16& ac = acc[(b0 + g) / CBW][(b0 + g) % CBW];
            if (s < sidx) {
                pre[g] = s == 0 ? v : pre[g] + v;
                if (s == sidx - 1) ac = pre[g] + ac;
            } else {
                ac += v;
            }
        };
        // C consecutive other splits from o0 on: all loads, then the adds
        auto piece = [&](auto count, int o0) {
            constexpr int C = decltype(count)::value;
            floatx16 buf[C][BG];
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const int s = o0 + i < sidx ? o0 + i : o0 + i + 1;
#pragma unroll
                for (int g = 0; g < BG; ++g) buf[i][g] = load_part(s, (b0 + g) / CBW, (b0 + g) % CBW);
            }
#pragma unroll
            for (int i = 0; i < C; ++i) {
                const int s = o0 + i < sidx ? o0 + i : o0 + i + 1;
#pragma unroll
                for (int g = 0; g < BG; ++g) add(s, g, buf[i][g]);
            }
        };
        int o = 0;
        if constexpr (KQ >= 4) {
            for (; o + 4 <= n_other; o += 4) piece(std::integral_constant<int, 4>{}, o);
            if (o + 3 == n_other) piece(std::integral_constant<int, 3>{}, o), o += 3;
        }
        if constexpr (KQ >= 2)
            for (; o + 2 <= n_other; o += 2) piece(std::integral_constant<int, 2>{}, o);
        for (; o < n_other; ++o) piece(std::integral_constant<int, 1>{}, o);
#pragma unroll
        for (int g = 0; g < BG; ++g) store_c((b0 + g) / CBW, (b0 + g) % CBW, acc[(b0 + g) / CBW][(b0 + g) % CBW]);
    }
}

template <int BM, int BN, int WGM, int NWV, int WPF, int XPF>
__global__ void __launch_bounds__(64 * NWV)
__attribute__((amdgpu_waves_per_eu(tiled_waves_per_simd(BM, BN, WGM, NWV))))
tiled_kernel(GemmArgs a, int splitk) {
    tiled_body<BM, BN, WGM, NWV, WPF, XPF, 1>(a, splitk);
}

// two K slices of NWV waves each (two waves per SIMD for four-wave grids)
template <int BM, int BN, int WGM, int NWV, int WPF, int XPF>
__global__ void __launch_bounds__(128 * NWV) __attribute__((amdgpu_waves_per_eu(2)))
tiled_k2_kernel(GemmArgs a, int splitk) {
    tiled_body<BM, BN, WGM, NWV, WPF, XPF, 2>(a, splitk);
}

// The same two kernels reading X [K, N] in place (no xpack_col launch),
// built for the default tiles (waves along M only, one stage of
// activations ahead): 96 x 64 of three waves, 128 x 64, 128 x 128 and
// 256 x 128 of four, 512 x 128 of eight.  Each B fragment then takes two
// transposing LDS reads instead of one, which costs less than the launch
// and the 2 K N bytes of re-layout it saves once the rows' pieces are
// permuted against bank conflicts (12288x4096 N = 64 / 256 / 4096: 20.3 /
// 41.9 / 372.5 -> 17.6 / 37.6 / 364.8 us; without the permutation the
// 128 x 128 tiles lost: N = 512 65.6 -> 75.4 us).
__host__ __device__ constexpr bool tiled_dx_built(int BM, int BN, int WGM, int NWV, int WPF, int XPF) {
    return XPF == 1 && WPF <= 2 && WGM == NWV &&
           ((BM == 96 && NWV == 3 && BN == 64) || (BM == 128 && NWV == 4 && (BN == 64 || BN == 128)) ||
            (BM == 256 && NWV == 4 && BN == 128) || (BM == 512 && NWV == 8 && BN == 128));
}

template <int BM, int BN, int WGM, int NWV, int WPF, int XPF>
__global__ void __launch_bounds__(64 * NWV)
__attribute__((amdgpu_waves_per_eu(tiled_waves_per_simd(BM, BN, WGM, NWV))))
tiled_dx_kernel(GemmArgs a, int splitk) {
    tiled_body<BM, BN, WGM, NWV, WPF, XPF, 1, true>(a, splitk);
}

template <int BM, int BN, int WGM, int NWV, int WPF, int XPF>
__global__ void __launch_bounds__(128 * NWV) __attribute__((amdgpu_waves_per_eu(2)))
tiled_k2_dx_kernel(GemmArgs a, int splitk) {
    tiled_body<BM, BN, WGM, NWV, WPF, XPF, 2, true>(a, splitk);
}

template <int BM, int BN, int WGM, int NWV, int WPF, int XPF, int WKS, bool DX>
hipError_t launch_one(const GemmArgs& a, const TiledShape& t, hipStream_t stream) {
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    const dim3 grid((unsigned)tiles, (unsigned)t.splitk);
    constexpr int lds = tiled_lds_bytes(BN, XPF, WKS);
    if constexpr (lds > 65536) {
        const void* fn;
        if constexpr (WKS == 1 && DX)
            fn = reinterpret_cast<const void*>(&tiled_dx_kernel<BM, BN, WGM, NWV, WPF, XPF>);
        else if constexpr (WKS == 1)
            fn = reinterpret_cast<const void*>(&tiled_kernel<BM, BN, WGM, NWV, WPF, XPF>);
        else if constexpr (DX)
            fn = reinterpret_cast<const void*>(&tiled_k2_dx_kernel<BM, BN, WGM, NWV, WPF, XPF>);
        else
            fn = reinterpret_cast<const void*>(&tiled_k2_kernel<BM, BN, WGM, NWV, WPF, XPF>);
        // dynamic LDS above 64 KB must be allowed per kernel, once
        static const hipError_t ok = [fn] {
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (e != hipSuccess) (void)hipGetLastError();
            return e;
        }();
        if (ok != hipSuccess) return ok;
    }
    if constexpr (WKS == 1 && DX)
        hipLaunchKernelGGL((tiled_dx_kernel<BM, BN, WGM, NWV, WPF, XPF>), grid, dim3(64 * NWV), lds, stream, a,
                           t.splitk);
    else if constexpr (WKS == 1)
        hipLaunchKernelGGL((tiled_kernel<BM, BN, WGM, NWV, WPF, XPF>), grid, dim3(64 * NWV), lds, stream, a,
                           t.splitk);
    else if constexpr (DX)
        hipLaunchKernelGGL((tiled_k2_dx_kernel<BM, BN, WGM, NWV, WPF, XPF>), grid, dim3(128 * NWV), lds, stream,
                           a, t.splitk);
    else
        hipLaunchKernelGGL((tiled_k2_kernel<BM, BN, WGM, NWV, WPF, XPF>), grid, dim3(128 * NWV), lds, stream, a,
                           t.splitk);
    return hipGetLastError();
}

// The weight / activation prefetch distances built for a tile shape: one or
// two stages of weights and one of activations for every tile, deeper
// pipelines for the tiles of four waves that the few-column calls use.
template <int BM, int BN, int WGM, int NWV, int WPF, int XPF>
hipError_t launch_if(const GemmArgs& a, const TiledShape& t, bool dx, hipStream_t stream) {
    if constexpr (tiled_pipe_ok(BM, BN, WGM, NWV, WPF, XPF)) {
        if constexpr (tiled_dx_built(BM, BN, WGM, NWV, WPF, XPF)) {
            if (dx) {
                if constexpr (tiled_k2_ok(BM, BN, WGM, NWV, WPF, XPF))
                    if (t.wk == 2) return launch_one<BM, BN, WGM, NWV, WPF, XPF, 2, true>(a, t, stream);
                if (t.wk == 1) return launch_one<BM, BN, WGM, NWV, WPF, XPF, 1, true>(a, t, stream);
                return hipErrorInvalidValue;
            }
        }
        if (dx) return hipErrorInvalidValue;
        if constexpr (tiled_k2_ok(BM, BN, WGM, NWV, WPF, XPF))
            if (t.wk == 2) return launch_one<BM, BN, WGM, NWV, WPF, XPF, 2, false>(a, t, stream);
        if (t.wk == 1) return launch_one<BM, BN, WGM, NWV, WPF, XPF, 1, false>(a, t, stream);
    }
    return hipErrorInvalidValue;
}

template <int BM, int BN, int WGM = 4, int NWV = 4>
hipError_t launch_bmbn(const GemmArgs& a, const TiledShape& t, bool dx, hipStream_t stream) {
    switch (t.wpf * 10 + t.xpf) {
        case 11: return launch_if<BM, BN, WGM, NWV, 1, 1>(a, t, dx, stream);
        case 21: return launch_if<BM, BN, WGM, NWV, 2, 1>(a, t, dx, stream);
        case 22: return launch_if<BM, BN, WGM, NWV, 2, 2>(a, t, dx, stream);
        case 32: return launch_if<BM, BN, WGM, NWV, 3, 2>(a, t, dx, stream);
        case 42: return launch_if<BM, BN, WGM, NWV, 4, 2>(a, t, dx, stream);
        case 33: return launch_if<BM, BN, WGM, NWV, 3, 3>(a, t, dx, stream);
        case 43: return launch_if<BM, BN, WGM, NWV, 4, 3>(a, t, dx, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool tiled_supported(const TiledShape& t) {
    // three waves of 32 rows: 96 x 64 tiles, weights one or two stages ahead
    if (t.wm == 3) return t.bm == 96 && t.bn == 64 && t.wk == 1 && (t.wpf == 1 || t.wpf == 2) && t.xpf == 1 && t.splitk >= 1;
    if (t.wm != 2 && t.wm != 4 && t.wm != 8) return false;
    if (t.wk != 1 && !(t.wk == 2 && tiled_k2_ok(t.bm, t.bn, t.wm, t.wm == 8 ? 8 : 4, t.wpf, t.xpf))) return false;
    if (!tiled_pipe_ok(t.bm, t.bn, t.wm, t.wm == 8 ? 8 : 4, t.wpf, t.xpf)) return false;
    // a third weight register set spills with the 2 x 2 wave grid
    if (t.wpf == 2 && t.wm == 2) return false;
    if (t.wm == 8) return t.bm == 512 && t.bn == 128 && t.splitk >= 1;
    const bool bm_ok = t.bm == 128 || t.bm == 256;
    const bool bn_ok = t.bn == 64 || t.bn == 128 || t.bn == 256;
    const bool wm_ok = t.wm == 4 || (t.wm == 2 && t.bn >= 128);
    return bm_ok && bn_ok && wm_ok && t.splitk >= 1;
}

const char* tiled_check(const GemmArgs& a, const TiledShape& t) {
    // 32-bit buffer offsets and record counts: a tile's weight rows and a
    // 16-row chunk slab
    if ((int64_t)t.bm * (a.K / 2) > 0x7FFFFFFF) return "bm * K / 2 above 2^31 - 1 bytes";
    if (a.N > ((int64_t)1 << 23)) return "N above 2^23";
    // 32-bit buffer offsets over the split partials
    if (t.splitk > 1 && (int64_t)tiled_partial_bytes(a, t) > 0x7FFFFFFF)
        return "the split partial tiles exceed 2^31 - 1 bytes";
    return nullptr;
}

int64_t tiled_tiles(const GemmArgs& a, const TiledShape& t) {
    return ((a.M + t.bm - 1) / t.bm) * ((a.N + t.bn - 1) / t.bn);
}

size_t tiled_partial_bytes(const GemmArgs& a, const TiledShape& t) {
    return t.splitk <= 1 ? 0 : (size_t)t.splitk * (size_t)tiled_tiles(a, t) * t.bm * t.bn * 4;
}

size_t xpack_bytes(const GemmArgs& a) { return (size_t)a.K * (size_t)a.N * 2; }

hipError_t launch_xpack(const GemmArgs& a, hipStream_t stream) {
    if (a.xp_ready) return hipSuccess;
    if (a.tm) {
        const int64_t blocks = (a.K / 128) * ((a.N + 15) / 16);
        if (a.act)
            hipLaunchKernelGGL(xpack_silu_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.x,
                               reinterpret_cast<u32x4*>(a.xp), a.K, a.N);
        else
            hipLaunchKernelGGL(xpack_tm_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a.x,
                               reinterpret_cast<u32x4*>(a.xp), a.K, a.N);
        return hipGetLastError();
    }
    u32x4* xp = reinterpret_cast<u32x4*>(a.xp);
    const int64_t chunks = (a.K / 8) * a.N;
    if ((chunks + 255) / 256 > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(xpack_col_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, stream, a.x, xp, a.K,
                       a.N);
    return hipGetLastError();
}

bool tiled_direct_x(const GemmArgs& a, const TiledShape& t) {
    if (a.tm || a.xp_ready || a.act || a.N % 8 != 0 || a.N > 65536) return false;
    if (t.xpf != 1 || t.wpf > 2) return false;
    return (t.bn == 64 && t.bm == 96 && t.wm == 3) || (t.bm == 128 && (t.bn == 64 || t.bn == 128) && t.wm == 4) ||
           (t.bm == 256 && t.bn == 128 && t.wm == 4) || (t.bm == 512 && t.bn == 128 && t.wm == 8);
}

hipError_t launch_tiled(const GemmArgs& a, const TiledShape& t, hipStream_t stream) {
    const bool dx = tiled_direct_x(a, t);
    if (!dx) {
        const hipError_t e = launch_xpack(a, stream);
        if (e != hipSuccess) return e;
    }
    if (t.wm == 8) {
        if (t.bm == 512 && t.bn == 128) return launch_bmbn<512, 128, 8, 8>(a, t, dx, stream);
        return hipErrorInvalidValue;
    }
    if (t.wm == 3) {
        if (t.bm == 96 && t.bn == 64) return launch_bmbn<96, 64, 3, 3>(a, t, dx, stream);
        return hipErrorInvalidValue;
    }
    if (t.wm == 2) {
        if (t.bm == 256 && t.bn == 256) return launch_bmbn<256, 256, 2>(a, t, dx, stream);
        if (t.bm == 256 && t.bn == 128) return launch_bmbn<256, 128, 2>(a, t, dx, stream);
        if (t.bm == 128 && t.bn == 256) return launch_bmbn<128, 256, 2>(a, t, dx, stream);
        if (t.bm == 128 && t.bn == 128) return launch_bmbn<128, 128, 2>(a, t, dx, stream);
        return hipErrorInvalidValue;
    }
    if (t.bm == 256 && t.bn == 256) return launch_bmbn<256, 256>(a, t, dx, stream);
    if (t.bm == 256 && t.bn == 128) return launch_bmbn<256, 128>(a, t, dx, stream);
    if (t.bm == 256 && t.bn == 64) return launch_bmbn<256, 64>(a, t, dx, stream);
    if (t.bm == 128 && t.bn == 256) return launch_bmbn<128, 256>(a, t, dx, stream);
    if (t.bm == 128 && t.bn == 128) return launch_bmbn<128, 128>(a, t, dx, stream);
    if (t.bm == 128 && t.bn == 64) return launch_bmbn<128, 64>(a, t, dx, stream);
    return hipErrorInvalidValue;
}

}  // namespace w4a16
