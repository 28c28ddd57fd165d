// Narrow W4A16 kernel for a few activation columns (N up to 64): still the
// bandwidth-bound side of the PerfXLLM page on Snapdragon 8 Gen2, §3.3
// item 1 (few tokens make B tall and thin), where the weight stream decides
// the time and every weight byte must be read once, early and coalesced.
//
// A workgroup of WM waves (four, or three: 48-row tiles put a 12288-row
// matrix on 256 CUs, one tile each) owns BM = WM x 16 RB rows and a
// contiguous range of groups along K (splitk workgroups share a row tile).
// At the start it copies the activations of its groups from L2 straight
// into LDS, where all its waves read them; it never touches them in HBM
// again.  [K, N] activations with N a multiple of 8 are copied from X
// itself, eight k rows per octet stored in dequant order and read back with
// the transposing LDS read (ds_read_b64_tr_b16), which hands each lane one
// column's k; any other layout or N goes through the re-layout launch first
// (16-byte chunks: eight k of one column in dequant order).
// Each wave streams the packed weights of its 16 RB rows through a ring of
// PF register stages (one 128-k group per stage, 16 bytes per lane and
// 16-row block), so PF groups of every wave are in flight while it works;
// there is no barrier in the main loop.  Words are dequantized in registers
// to the exact fp16 codes q - z and meet the activations in
// v_mfma_f32_16x16x32_f16 with the activations as the A operand (16
// columns as rows) and the weights as B (16 weight rows as columns); each
// group's fp32 sums are scaled by s into the accumulators, so each lane
// ends with one weight row and four consecutive output columns: one 8-byte
// store.  Split-K partials are summed in order by the last workgroup of a
// tile.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int kNarrowMaxLds = 160 * 1024;
typedef short short4v __attribute__((ext_vector_type(4)));
// cache-policy operand of the weight loads: non-temporal (each weight byte
// is read once; 4-5 % faster at N = 8 and 16 than the default policy)
constexpr int kNonTemporal = 2;

// Wait until at most n vector-memory operations are outstanding.  Inline
// assembly with a memory clobber, so that the compiler keeps every load
// issued before it above it (the count includes loads the compiler cannot
// see, the buffer-to-LDS copies).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(n) : "memory");
}

// The eight codes of a packed word as exact fp16 (q - z), in the k order
// 0, 4, 1, 5, 2, 6, 3, 7 that the activation chunks use: nibbles at bits
// 0-3 of a half are OR-ed into fp16 1024 (ulp 1), nibbles at bits 4-7 into
// fp16 64 (ulp 1/16), and 1024 + z / 64 + z are subtracted.  The scale is
// applied later, to the group's float32 sums.
struct QMinusZ {
    uint32_t b1024, b64;   // bias constants in vector registers
    half2v z1024, z64;
    __device__ __forceinline__ void init() {
        b1024 = 0x64006400u;
        b64 = 0x54005400u;
    }
    __device__ __forceinline__ void set(uint32_t z) {
        z1024 = as_h2(0x64006400u | z | (z << 16));
        z64 = as_h2(0x54005400u | (z << 4) | (z << 20));
    }
    __device__ __forceinline__ half8 operator()(uint32_t w) const {
        const uint32_t w8 = w >> 8;
        const half2v p0 = as_h2(and_or(w, 0x000F000Fu, b1024)) - z1024;
        const half2v p1 = as_h2(and_or(w, 0x00F000F0u, b64)) - z64;
        const half2v p2 = as_h2(and_or(w8, 0x000F000Fu, b1024)) - z1024;
        const half2v p3 = as_h2(and_or(w8, 0x00F000F0u, b64)) - z64;
        return __builtin_bit_cast(half8, u32x4{as_u32(p0), as_u32(p1), as_u32(p2), as_u32(p3)});
    }
};

// Piece permutation of an in-place activation octet with 64 staged columns
// (16-byte pieces, eight per 128-byte row): the piece index is XORed with
// a mask of its row p and of the parity g of the 16-lane group that reads
// it (octet index / 4), so that the eight 32-byte segments a half-wave's
// transposing read takes (two groups x four rows, rows 128 bytes apart)
// cover 256 distinct bytes of banks.  An involution: the copy and the read
// apply the same XOR.  4096x4096 N = 64 / 40: 13.2 -> 11.8 us; the same
// idea for 16 and 32 columns (the two groups' octets start on the same
// banks) was 1-2 % slower or level, so those keep the plain layout.
template <int NCOL>
__host__ __device__ constexpr int dx_piece_xor(int p, int g) {
    return NCOL == 64 ? 4 * ((p >> 1) & 1) + 2 * g : 0;
}

template <int NC, int PF, int kRB, int WK, int WM, bool DX>
__global__ void __launch_bounds__(64 * WM * WK) narrow_kernel(GemmArgs a, int splitk) {
    constexpr int NCOL = 16 * NC;            // staged columns (N padded to 16 NC)
    constexpr int kNarrowBM = 16 * WM * kRB; // rows per workgroup (16 kRB per wave)
    constexpr int NT = 64 * WM * WK;         // threads: WM waves along M times WK along K
    constexpr int NW = WM * WK;              // waves
    constexpr int WLOADS = kRB;         // weight loads per wave and stage
    static_assert(PF * WLOADS < 64, "vmcnt range");
    // dynamic LDS: the activation chunks, then the split-K flag (all of
    // the 160 KB is dynamic, so that the kernel may ask for every byte)
    extern __shared__ __attribute__((aligned(16))) unsigned char xs[];

    const int64_t M = a.M, N = a.N, K = a.K;
    const int G = a.G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave_m = wave % WM, wave_k = wave / WM;
    const int r16 = lane & 15;   // weight row in a 16-row block / activation column in a 16-column block
    const int kq = lane >> 4;    // k-quarter of the 32-k MFMA step (words 4 kq .. 4 kq + 3 of a group)

    const int64_t row0 = (int64_t)blockIdx.x * kNarrowBM;
    const int sidx = blockIdx.y;
    const int g0 = (int)((int64_t)G * sidx / splitk);
    const int g1 = (int)((int64_t)G * (sidx + 1) / splitk);
    const int ng = g1 - g0;      // >= WK since splitk <= G / WK
    const int64_t KW = K / 8;
    // the groups of this wave: [gw0, gw0 + ngw) of the workgroup's range
    const int gw0 = ng * wave_k / WK, ngw = ng * (wave_k + 1) / WK - gw0;

    // ---- activation chunks of groups [g0, g1), columns [0, NCOL): LDS chunk
    // (o, n) = X chunk (16 g0 + o, n) at (o NCOL + n) * 16.  Wave w issues
    // instructions j = w, w + NW, ...; instruction j fills chunks
    // [64 j, 64 j + 64).  Columns past N re-read column N - 1.
    if constexpr (!DX) {
        const i32x4 xres = raw_rsrc(a.xp + (int64_t)g0 * 16 * N * 8, (int64_t)ng * 16 * N * 16);
        const int nins = ng * 16 * NCOL / 64;
        for (int j = wave; j < nins; j += NW) {
            const int c = 64 * j + lane;
            const int o = c / NCOL, n = c % NCOL;
            const int64_t nn = n < N ? n : N - 1;
            buffer_load_lds16(xres, xs + 64 * j * 16, (int)((o * N + nn) * 16), 0);
        }
    } else {
        // X read in place ([K, N] rows, N a multiple of 8): octet o of the
        // range holds its eight k rows of NCOL halves in dequant order
        // (k offsets 0, 4, 1, 5, 2, 6, 3, 7), so that two transposing reads
        // of four rows each give a lane one column's eight k in the order
        // the weight words unpack to.  With 64 columns the octet's 16-byte
        // pieces are permuted (dx_piece_xor) so that the two 16-lane groups
        // of a half-wave, which read octets four apart, and the four rows
        // each reads fall on distinct banks.  Chunks past N re-read the
        // row's last.
        const i32x4 xres = raw_rsrc(a.x + (int64_t)g0 * 128 * N, (int64_t)ng * 128 * N * 2);
        const int nins = ng * 16 * NCOL / 64;
        const int n8 = (int)(N >> 3);
        for (int j = wave; j < nins; j += NW) {
            const int c = 64 * j + lane;
            const int o = c / NCOL;
            const int w = (c % NCOL) ^ dx_piece_xor<NCOL>((c % NCOL) / (NCOL / 8), (o >> 2) & 1);
            const int p = w / (NCOL / 8), cc = w % (NCOL / 8);
            const int r = (p >> 1) + 4 * (p & 1);
            const int ccl = cc < n8 ? cc : n8 - 1;
            buffer_load_lds16(xres, xs + 64 * j * 16, (int)(((8 * o + r) * N + 8 * ccl) * 2), 0);
        }
    }

    // ---- weights of this lane: rows row0 + 16 (kRB wave + rb) + r16 (clamped
    // to the last row), words 4 kq .. 4 kq + 3 of each group
    const int64_t rows_left = M - row0;
    const int tile_rows = (int)(rows_left < kNarrowBM ? rows_left : kNarrowBM);
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(a.qpk + row0 * KW, (int64_t)tile_rows * KW * 4);
    int woff[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        int r = 16 * (kRB * wave_m + rb) + r16;
        r = r < tile_rows ? r : tile_rows - 1;
        woff[rb] = (int)((r * KW + 4 * kq) * 4);
    }

    // ---- scales and zero words of the tile's rows and groups, staged in LDS
    // once ([group][row] halves and [word][row] words, rows padded by two
    // halves / one word so that the stores below hit distinct banks, and so
    // that the 16 rows a lane group reads are consecutive).  Consecutive
    // threads take consecutive groups (words) of one row, GP (ZP2) slots per
    // row, GP the power of two >= the groups (words) of the range: one load
    // instruction reads a few rows' contiguous runs instead of one value
    // from each of 64 rows.  The loads are issued before the weight
    // prefetch, the LDS stores after it; slots past the range reload the
    // row's last value.
    constexpr int SP = kNarrowBM + 2, ZP = kNarrowBM + 1;   // padded row counts
    // loads per thread at most: plans keep ngmax <= 16 NT / BM (NT / BM a
    // power of two), so GP <= 16 NT / BM and BM GP / NT <= 16 scale passes;
    // a range of ngmax groups spans at most 2 NT / BM + 1 zero words, so
    // ZP2 <= 4 NT / BM and at most 4 zero passes
    constexpr int SMAX = 16, ZMAX = 4;
    const int ngmax = (G + splitk - 1) / splitk;
    const int zw0 = g0 >> 3, nzw = ((g1 - 1) >> 3) - zw0 + 1;
    uint16_t* sl = reinterpret_cast<uint16_t*>(xs + (size_t)ngmax * 16 * NCOL * 16);
    uint32_t* zl = reinterpret_cast<uint32_t*>(sl + (size_t)ngmax * SP);
    const int lgp = ng > 1 ? 32 - __builtin_clz((unsigned)(ng - 1)) : 0;     // GP = 1 << lgp >= ng
    const int lzp = nzw > 1 ? 32 - __builtin_clz((unsigned)(nzw - 1)) : 0;   // ZP2 = 1 << lzp >= nzw
    const int sg = tid & ((1 << lgp) - 1), sr0 = tid >> lgp, srs = NT >> lgp;
    const int zg = tid & ((1 << lzp) - 1), zr0 = tid >> lzp, zrs = NT >> lzp;
    const int spass = (tile_rows + srs - 1) / srs, zpass = (tile_rows + zrs - 1) / zrs;   // uniform
    const __amdgpu_buffer_rsrc_t sres = buffer_rsrc(a.scales + row0 * G, (int64_t)tile_rows * G * 2);
    const __amdgpu_buffer_rsrc_t zres = buffer_rsrc(a.zpk + row0 * a.ZW, (int64_t)tile_rows * a.ZW * 4);
    // Every one of the SMAX scale and ZMAX zero loads is issued (passes past
    // spass / zpass reload the last pass): a load under a branch leaves a
    // merge of loaded and unloaded values, and the compiler then widens the
    // loaded one right after its load, waiting there for every load before
    // it, the activation copies included, before a weight load is issued.
    uint32_t sv[SMAX], zv[ZMAX];
    {
        const int gc = sg < ng ? sg : ng - 1, wc = zg < nzw ? zg : nzw - 1;
#pragma unroll
        for (int j = 0; j < SMAX; ++j) {
            int r = sr0 + srs * (j < spass ? j : spass - 1);
            r = r < tile_rows ? r : tile_rows - 1;
            sv[j] = __builtin_amdgcn_raw_buffer_load_b16(sres, (r * G + g0 + gc) * 2, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < ZMAX; ++j) {
            int r = zr0 + zrs * (j < zpass ? j : zpass - 1);
            r = r < tile_rows ? r : tile_rows - 1;
            zv[j] = __builtin_amdgcn_raw_buffer_load_b32(zres, (r * a.ZW + zw0 + wc) * 4, 0, 0);
        }
    }

    // ring of PF stages of packed words
    u32x4 wr[PF][kRB];
    auto load = [&](int slot, int g) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
            wr[slot][rb] = __builtin_amdgcn_raw_buffer_load_b128(wres, woff[rb], g * 64, kNonTemporal);
    };
    // groups past the range reload the last one (no branch around loads),
    // slot by slot in the order the loop refills them, so that the wait
    // counts at the top of a round are the same on entry and on repeat
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        load(p, g0 + gw0 + (p < ngw ? p : ngw - 1));
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < SMAX; ++j)
        if (j < spass) {
            const int r = sr0 + srs * j;
            if (sg < ng && r < tile_rows) sl[sg * SP + r] = (uint16_t)sv[j];
        }
#pragma unroll
    for (int j = 0; j < ZMAX; ++j)
        if (j < zpass) {
            const int r = zr0 + zrs * j;
            if (zg < nzw && r < tile_rows) zl[zg * ZP + r] = zv[j];
        }
    // the activation copies were issued before the scale, zero and these
    // PF * WLOADS weight loads
    wait_vmcnt<PF * WLOADS>();
    __syncthreads();

    floatx4 acc[kRB][NC];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    QMinusZ qz[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) qz[rb].init();

    // activation fragment of MFMA step t, block cb, local group s: chunk
    // (16 s + 4 kq + t, 16 cb + r16)
    // DX: lane (r16, kq) reads row (r16 >> 2) (+ 4) of octet 4 kq + t, 8 bytes
    // at column 16 cb + 4 (r16 & 3), at the position the piece permutation
    // gives: with 64 columns the 32-byte column segment cb moves to cb ^ xcb
    const int dxg = kq & 1, dxj = r16 >> 2;
    const int xcb = NCOL == 64 ? 2 * ((dxj >> 1) & 1) + dxg : 0;
    const unsigned char* xl = DX ? xs + (4 * kq) * NCOL * 16 + dxj * NCOL * 2 + (r16 & 3) * 8
                                 : xs + ((4 * kq) * NCOL + r16) * 16;

    // Each stage's four MFMA steps start from zero and give the group's
    // float32 sums of (q - z) x; the group's scale multiplies them into the
    // accumulators one stage later (so that multiply waits for nothing).
    floatx4 part[kRB][NC];
    float sprev[kRB];
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb) {
        sprev[rb] = 0.f;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) part[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
    auto retire = [&]() {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[rb][cb][j] = fmaf(sprev[rb], part[rb][cb][j], acc[rb][cb][j]);
    };

    // LDS operands of a stage (the activation fragments of all four steps,
    // the zero word and the scale of each row block), read one stage ahead
    // so that their latency hides behind the previous stage's work
    half8 xn[4][NC];
    uint32_t zn[kRB];
    uint16_t sn[kRB];
    auto fetch = [&](int s) {
        const int gl = gw0 + (s < ngw ? s : ngw - 1), g = g0 + gl;
        const unsigned char* xg = xl + gl * 16 * NCOL * 16;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                if constexpr (DX) {
                    // lanes 4 j .. 4 j + 3 of a 16-lane group read row 4 h + j of
                    // the octet (columns 16 cb + 4 (lane % 4) ..); the transpose
                    // hands lane i column 16 cb + i of the four rows
                    const unsigned char* b = xg + t * NCOL * 16 + (cb ^ xcb) * 32;
                    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) short4v*)(b));
                    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) short4v*)(b + 4 * NCOL * 2));
                    xn[t][cb] = __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                } else {
                    xn[t][cb] = *reinterpret_cast<const half8*>(xg + (t * NCOL + 16 * cb) * 16);
                }
            }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            const int r = 16 * (kRB * wave_m + rb) + r16;
            zn[rb] = zl[((g >> 3) - zw0) * ZP + r] >> (4 * (g & 7));
            sn[rb] = sl[gl * SP + r];
        }
    };
    fetch(0);

    // stage s of this wave: group g0 + gw0 + s, local index gw0 + s
    auto stage = [&](int p, int s) {
        half8 xf[4][NC];
        float scur[kRB];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) xf[t][cb] = xn[t][cb];
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            qz[rb].set(zn[rb] & 0xFu);
            scur[rb] = (float)__builtin_bit_cast(_Float16, sn[rb]);
        }
        fetch(s + 1);
        floatx4 np[kRB][NC];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb) {
                const half8 wf = qz[rb](wr[p][rb][t]);
#pragma unroll
                for (int cb = 0; cb < NC; ++cb)
                    np[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        xf[t][cb], wf, t == 0 ? floatx4{0.f, 0.f, 0.f, 0.f} : np[rb][cb], 0, 0, 0);
            }
        retire();
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb) {
            sprev[rb] = scur[rb];
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) part[rb][cb] = np[rb][cb];
        }
    };
    // full rounds of PF groups: each slot is refilled with the group PF ahead
    // (or the last group again) right after use, with no branch around loads
    int s0 = 0;
    for (; s0 + PF <= ngw; s0 += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            stage(p, s0 + p);
            const int sn = s0 + p + PF < ngw ? s0 + p + PF : ngw - 1;
            load(p, g0 + gw0 + sn);
            // keep the refill here: sunk to the end of the round, it would
            // leave nothing in flight at the start of the next one
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // the last ngw % PF groups are already in their slots
#pragma unroll
    for (int p = 0; p < PF - 1; ++p)
        if (s0 + p < ngw) stage(p, s0 + p);
    retire();

    // ---- waves along K meet in LDS (over the activation chunks, which
    // every wave has finished reading): wave_k > 0 parks its sums, wave_k 0
    // adds them in order and goes on alone
    if (WK > 1) {
        floatx4* red = reinterpret_cast<floatx4*>(xs);
        __syncthreads();
        if (wave_k > 0) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                for (int cb = 0; cb < NC; ++cb)
                    red[((((wave_k - 1) * WM + wave_m) * kRB + rb) * NC + cb) * 64 + lane] = acc[rb][cb];
        }
        __syncthreads();
        if (wave_k == 0) {
            for (int k = 1; k < WK; ++k)
#pragma unroll
                for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                    for (int cb = 0; cb < NC; ++cb)
                        acc[rb][cb] += red[((((k - 1) * WM + wave_m) * kRB + rb) * NC + cb) * 64 + lane];
        }
    }

    // ---- epilogue: lane holds row 16 (kRB wave + rb) + r16 and columns
    // 16 cb + 4 kq .. + 3
    auto store_c = [&](int rb, int cb, const floatx4& v) {
        const int64_t row = row0 + 16 * (kRB * wave_m + rb) + r16;
        const int64_t col = 16 * cb + 4 * kq;
        if (row >= M || col >= N) return;
        if (a.tm) {
            // token-major output: the 16 lanes of a k-quarter write 16
            // consecutive rows of one column
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (col + j < N) a.c[(col + j) * M + row] = (uint16_t)f32_to_h16_bits(v[j]);
        } else if (col + 4 <= N && (N & 3) == 0) {
            uint2 u;
            u.x = f32_to_h16_bits(v[0]) | (f32_to_h16_bits(v[1]) << 16);
            u.y = f32_to_h16_bits(v[2]) | (f32_to_h16_bits(v[3]) << 16);
            *reinterpret_cast<uint2*>(a.c + row * N + col) = u;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (col + j < N) a.c[row * N + col + j] = (uint16_t)f32_to_h16_bits(v[j]);
        }
    };
    if (splitk == 1) {
        if (wave_k == 0) {
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                for (int cb = 0; cb < NC; ++cb) store_c(rb, cb, acc[rb][cb]);
        }
        return;
    }

    // ---- split-K: every split stores its fp32 partial tile; the last
    // workgroup of a row tile to arrive adds them in split order, its own
    // from its registers, and stores C.  A partial tile is kept in the
    // register layout of the WM waves that hold the sums
    // ([wave][block][element][lane], 256 contiguous bytes per element, a
    // private slot per split and tile): every access is one coalesced store
    // or load with no mask, and a split's loads are all in flight at once.
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
    constexpr int kAgent = 16;                  // cache policy sc1
    constexpr int SLOT = kRB * NC * 4 * 64;     // floats per wave and split
    const __amdgpu_buffer_rsrc_t pres =
        buffer_rsrc(a.part, (int64_t)splitk * gridDim.x * WM * SLOT * 4);
    auto slot_off = [&](int s, int rb, int cb) {   // uniform byte offset of a block
        return (int)(((((int64_t)s * gridDim.x + blockIdx.x) * WM + wave_m) * SLOT + (rb * NC + cb) * 4 * 64) * 4);
    };
    const int lo = lane * 4;
    if (wave_k == 0) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                const int so = slot_off(sidx, rb, cb);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __builtin_amdgcn_raw_buffer_store_b32(f32_bits(acc[rb][cb][j]), pres,
                                                          lo + j * 256, so, kAgent);
            }
    }
    int* flag = reinterpret_cast<int*>(zl + (size_t)((ngmax + 15) / 8) * ZP);
    __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == (unsigned)(splitk - 1);
        if (last) {
            __hip_atomic_store(a.counters + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *flag = last;
    }
    __syncthreads();
    if (!*flag || wave_k != 0) return;
    // the sum runs in split order, (p_0 + ... + p_(sidx-1)) + own +
    // p_(sidx+1) + ..., the order of a plain left-to-right sum whichever
    // split arrives last
    auto load_part = [&](int s, floatx4 (&p)[kRB][NC]) {
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) {
                const int so = slot_off(s, rb, cb);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    p[rb][cb][j] = __builtin_bit_cast(float,
                                                      __builtin_amdgcn_raw_buffer_load_b32(pres, lo + j * 256, so, kAgent));
            }
    };
    floatx4 p[kRB][NC];
    if (sidx > 0) {
        floatx4 pre[kRB][NC];
        load_part(0, pre);
        for (int s = 1; s < sidx; ++s) {
            load_part(s, p);
#pragma unroll
            for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
                for (int cb = 0; cb < NC; ++cb) pre[rb][cb] += p[rb][cb];
        }
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) acc[rb][cb] = pre[rb][cb] + acc[rb][cb];
    }
    for (int s = sidx + 1; s < splitk; ++s) {
        load_part(s, p);
#pragma unroll
        for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NC; ++cb) acc[rb][cb] += p[rb][cb];
    }
#pragma unroll
    for (int rb = 0; rb < kRB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) store_c(rb, cb, acc[rb][cb]);
}

template <int NC, int PF, int RB, int WK, int WM, bool DX>
hipError_t launch_nc(const GemmArgs& a, const NarrowShape& s, hipStream_t stream) {
    constexpr int BM = 16 * WM * RB;
    dim3 grid((unsigned)((a.M + BM - 1) / BM), (unsigned)s.splitk);
    const size_t lds = narrow_lds_bytes(a, s);
    // allow up to 160 KB of dynamic LDS, once per kernel; a refusal is kept
    // here (and cleared from the runtime's last error) and reported only to
    // a launch that needs more than the default 64 KB
    static const hipError_t lds_ok = [] {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&narrow_kernel<NC, PF, RB, WK, WM, DX>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, kNarrowMaxLds);
        if (e != hipSuccess) (void)hipGetLastError();
        return e;
    }();
    if (lds_ok != hipSuccess && lds > 65536) return lds_ok;
    hipLaunchKernelGGL((narrow_kernel<NC, PF, RB, WK, WM, DX>), grid, dim3(64 * WM * WK), lds, stream, a, s.splitk);
    return hipGetLastError();
}

template <int NC, int RB, int WK, int WM>
hipError_t launch_pf(const GemmArgs& a, const NarrowShape& s, hipStream_t stream) {
    const bool dx = narrow_direct_x(a);
    switch (s.pf) {
        case 4: return dx ? launch_nc<NC, 4, RB, WK, WM, true>(a, s, stream)
                          : launch_nc<NC, 4, RB, WK, WM, false>(a, s, stream);
        case 8: return dx ? launch_nc<NC, 8, RB, WK, WM, true>(a, s, stream)
                          : launch_nc<NC, 8, RB, WK, WM, false>(a, s, stream);
        case 16: return dx ? launch_nc<NC, 16, RB, WK, WM, true>(a, s, stream)
                           : launch_nc<NC, 16, RB, WK, WM, false>(a, s, stream);
        default: return hipErrorInvalidValue;
    }
}

// three waves along M only with one wave along K
template <int NC, int RB>
hipError_t launch_wk(const GemmArgs& a, const NarrowShape& s, hipStream_t stream) {
    if (s.wm == 3) return s.wk == 1 ? launch_pf<NC, RB, 1, 3>(a, s, stream) : hipErrorInvalidValue;
    switch (s.wk) {
        case 1: return launch_pf<NC, RB, 1, 4>(a, s, stream);
        case 2: return launch_pf<NC, RB, 2, 4>(a, s, stream);
        case 4: return launch_pf<NC, RB, 4, 4>(a, s, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int NC>
hipError_t launch_rb(const GemmArgs& a, const NarrowShape& s, hipStream_t stream) {
    return s.rb == 1 ? launch_wk<NC, 1>(a, s, stream) : launch_wk<NC, 2>(a, s, stream);
}

}  // namespace

size_t narrow_lds_bytes(const GemmArgs& a, const NarrowShape& s) {
    const int64_t ngmax = (a.G + s.splitk - 1) / s.splitk;
    const int64_t bm = 16 * s.wm * s.rb;
    const size_t chunks = (size_t)ngmax * 16 * s.ncol * 16;                           // activation chunks
    const size_t red = (size_t)(s.wk - 1) * s.wm * s.rb * (s.ncol / 16) * 64 * 16;   // K-wave sums (reuse)
    return (chunks > red ? chunks : red)
           + (size_t)ngmax * (bm + 2) * 2            // scales ([group][row], rows padded by two halves)
           + (size_t)((ngmax + 15) / 8) * (bm + 1) * 4   // zero words (a range of ngmax groups spans at most this many)
           + 16;                                     // split-K flag
}

bool narrow_direct_x(const GemmArgs& a) { return !a.tm && !a.xp_ready && !a.act && a.N % 8 == 0; }

bool narrow_supported(const NarrowShape& s) {
    return (s.ncol == 16 || s.ncol == 32 || s.ncol == 64) && (s.pf == 4 || s.pf == 8 || s.pf == 16) &&
           (s.rb == 1 || s.rb == 2) && (s.wk == 1 || s.wk == 2 || s.wk == 4) &&
           (s.wm == 4 || (s.wm == 3 && s.wk == 1)) && s.splitk >= 1;
}

const char* narrow_check(const GemmArgs& a, const NarrowShape& s) {
    if (!narrow_supported(s))
        return "ncol must be 16, 32 or 64, the prefetch depth 4, 8 or 16, rb 1 or 2, wk 1, 2 or 4, wm 4 (or 3 with wk 1)";
    if (a.N > s.ncol) return "N exceeds the plan's columns";
    if ((int64_t)s.splitk * s.wk > a.G) return "splitk * wk exceeds the number of groups";
    if ((a.G + s.splitk - 1) / s.splitk > 16 * (4 * s.wk / s.rb))
        return "more than 16 * 4 wk / rb groups per workgroup; raise splitk";
    if (narrow_lds_bytes(a, s) > (size_t)kNarrowMaxLds)
        return "the workgroup's activation chunks exceed 160 KB of LDS; raise splitk";
    // 32-bit buffer offsets over the activation chunks and a 128-row weight tile
    if (a.K * a.N * 2 >= ((int64_t)1 << 31)) return "K * N too large";
    if (a.K > ((int64_t)1 << 24)) return "K above 2^24";
    // 32-bit buffer offsets over the split partials
    if ((int64_t)narrow_partial_bytes(a, s) > 0x7FFFFFFF) return "the split partial tiles exceed 2^31 - 1 bytes";
    return nullptr;
}

int64_t narrow_row_tiles(const GemmArgs& a, const NarrowShape& s) {
    const int64_t bm = 16 * s.wm * s.rb;
    return (a.M + bm - 1) / bm;
}

size_t narrow_partial_bytes(const GemmArgs& a, const NarrowShape& s) {
    return s.splitk <= 1 ? 0 : (size_t)s.splitk * (size_t)narrow_row_tiles(a, s) * (16 * s.wm * s.rb) * s.ncol * 4;
}

hipError_t launch_narrow(const GemmArgs& a, const NarrowShape& s, hipStream_t stream) {
    if (!narrow_direct_x(a)) {
        const hipError_t e = launch_xpack(a, stream);
        if (e != hipSuccess) return e;
    }
    switch (s.ncol) {
        case 16: return launch_rb<1>(a, s, stream);
        case 32: return launch_rb<2>(a, s, stream);
        case 64: return launch_rb<4>(a, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
