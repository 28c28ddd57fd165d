// Tiled W4A16 kernel for many activation columns: the compute-bound regime
// of PerfXLLM §3.3 item 1 (many tokens), which blocks the product into tiles
// held in shared memory.
//
// A workgroup of four waves owns a BM x BN tile of C and walks K in stages of
// 64.  Each stage copies the packed weights (BM rows x 32 bytes) and the
// activations (64 x BN fp16, transposed so that each 16-byte LDS word holds
// eight k of one column, in the dequant order) from global memory into a
// double-buffered LDS tile.  Each wave owns a (BM/2) x (BN/2) sub-tile made
// of 32x32 MFMA blocks: per 16-k step, a lane reads one packed weight word
// (eight k of one row), dequantizes it in registers to fp16 (q - z) * s and
// feeds it as the A operand of v_mfma_f32_32x32x16_f16, with fp32
// accumulation.  The scale is folded into the fp16 operand here (one fp16
// rounding per weight), since one accumulator spans all groups.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int BK = 64;

// 16-byte slot of activation column n inside one k-octet row of the LDS
// tile; the XOR spreads the eight columns a thread writes over all banks.
__device__ __forceinline__ int xslot(int n) { return n ^ ((n >> 3) & 7); }

template <int BM, int BN, bool VECX>
__global__ void __launch_bounds__(256, 1) tiled_kernel(GemmArgs a, int splitk) {
    constexpr int WR = BM / 2, WC = BN / 2;       // wave sub-tile
    constexpr int TR = WR / 32, TC = WC / 32;     // 32x32 MFMA blocks per wave
    constexpr int XBYTES = 8 * BN * 16;           // one stage of activations
    constexpr int WBYTES = BM * 32;               // one stage of packed weights
    constexpr int XBLK = BN;                      // 8x8 activation blocks per stage
    __shared__ __attribute__((aligned(16))) unsigned char xs[2][XBYTES];
    __shared__ __attribute__((aligned(16))) unsigned char ws[2][WBYTES];
    __shared__ int flag;

    const int64_t M = a.M, N = a.N, K = a.K;
    const int G = a.G;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_r = wave >> 1, wave_c = wave & 1;
    const int li = lane & 31;      // A row / B column / C column inside a 32-block
    const int h = lane >> 5;       // which half of the 16-k step

    // ---- tile of this workgroup: XCD-contiguous, then grouped along M
    const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN;
    const int64_t T = ntm * ntn;
    int64_t L = blockIdx.x;
    if (T % 8 == 0) L = (L % 8) * (T / 8) + L / 8;
    constexpr int64_t GM = 4;
    const int64_t group = L / (GM * ntn);
    const int64_t first_m = group * GM;
    const int64_t gsz = (ntm - first_m) < GM ? (ntm - first_m) : GM;
    const int64_t tm = first_m + (L % (GM * ntn)) % gsz;
    const int64_t tn = (L % (GM * ntn)) / gsz;
    const int64_t row0 = tm * BM, col0 = tn * BN;
    const int64_t tile_id = tm * ntn + tn;

    const int sidx = blockIdx.y;
    const int nst = (int)(K / BK);
    const int st0 = (int)((int64_t)nst * sidx / splitk);
    const int st1 = (int)((int64_t)nst * (sidx + 1) / splitk);

    const int64_t KW = K / 8;

    // ---- copy assignment
    // weights: chunk c = tid + 256 t -> (half = c / BM, row = c % BM)
    constexpr int WCH = (BM * 2) / 256;
    const uint32_t* wsrc[WCH];
    int wdst[WCH];
#pragma unroll
    for (int t = 0; t < WCH; ++t) {
        const int c = tid + 256 * t;
        const int hh = c / BM, r = c % BM;
        int64_t row = row0 + r;
        if (row > M - 1) row = M - 1;
        wsrc[t] = a.qpk + row * KW + hh * 4;
        wdst[t] = hh * (BM * 16) + r * 16;
    }
    // activations: block b = tid (if < XBLK) -> (k-octet ko, column octet nb)
    const bool xcopy = tid < XBLK;
    const int xko = tid / (BN / 8), xnb = tid % (BN / 8);
    const int64_t xcol = col0 + xnb * 8;

    // scale / zero rows of this lane (A-operand rows)
    const uint16_t* srow[TR];
    const uint32_t* zrow[TR];
#pragma unroll
    for (int rt = 0; rt < TR; ++rt) {
        int64_t row = row0 + wave_r * WR + rt * 32 + li;
        if (row > M - 1) row = M - 1;
        srow[rt] = a.scales + row * G;
        zrow[rt] = a.zpk + row * a.ZW;
    }

    u32x4 wreg[WCH];
    u32x4 xreg[8];

    auto load_stage = [&](int st) {
        const int64_t kw0 = (int64_t)st * (BK / 8);
#pragma unroll
        for (int t = 0; t < WCH; ++t)
            wreg[t] = *reinterpret_cast<const u32x4*>(wsrc[t] + kw0);
        if (xcopy) {
            const int64_t k = (int64_t)st * BK + xko * 8;
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                if (VECX) {
                    if (xcol < N)
                        xreg[r] = *reinterpret_cast<const u32x4*>(a.x + (k + r) * N + xcol);
                    else
                        xreg[r] = u32x4{0u, 0u, 0u, 0u};
                } else {
                    uint32_t hv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        hv[e] = (xcol + e < N) ? (uint32_t)a.x[(k + r) * N + xcol + e] : 0u;
                    xreg[r] = u32x4{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16),
                                    hv[4] | (hv[5] << 16), hv[6] | (hv[7] << 16)};
                }
            }
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int t = 0; t < WCH; ++t)
            *reinterpret_cast<u32x4*>(&ws[buf][wdst[t]]) = wreg[t];
        if (xcopy) {
            // transpose the 8 (k) x 8 (n) block: column c gets the pairs
            // (k0, k4), (k1, k5), (k2, k6), (k3, k7)
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const int d = cc >> 1;
                u32x4 o;
                if ((cc & 1) == 0) {
                    o.x = pair_lo(xreg[0][d], xreg[4][d]);
                    o.y = pair_lo(xreg[1][d], xreg[5][d]);
                    o.z = pair_lo(xreg[2][d], xreg[6][d]);
                    o.w = pair_lo(xreg[3][d], xreg[7][d]);
                } else {
                    o.x = pair_hi(xreg[0][d], xreg[4][d]);
                    o.y = pair_hi(xreg[1][d], xreg[5][d]);
                    o.z = pair_hi(xreg[2][d], xreg[6][d]);
                    o.w = pair_hi(xreg[3][d], xreg[7][d]);
                }
                const int n = xnb * 8 + cc;
                *reinterpret_cast<u32x4*>(&xs[buf][(xko * BN + xslot(n)) * 16]) = o;
            }
        }
    };

    floatx16 acc[TR][TC];
#pragma unroll
    for (int rt = 0; rt < TR; ++rt)
#pragma unroll
        for (int ct = 0; ct < TC; ++ct)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[rt][ct][e] = 0.f;

    // raw scale / zero words of a stage's group, loaded one stage ahead so
    // that waiting for them never waits for the next stage's tile loads
    uint32_t zraw[TR], sraw[TR];
    auto load_sz = [&](int st, uint32_t* zr, uint32_t* sr) {
        const int g = (st * BK) / kGroup;
#pragma unroll
        for (int rt = 0; rt < TR; ++rt) {
            zr[rt] = zrow[rt][g >> 3];
            sr[rt] = srow[rt][g];
        }
    };

    if (st0 < st1) {
        load_sz(st0, zraw, sraw);
        load_stage(st0);
        store_stage(0);
    }
    __syncthreads();

    for (int st = st0; st < st1; ++st) {
        const int cur = (st - st0) & 1;
        const bool more = st + 1 < st1;
        uint32_t znext[TR], snext[TR];
        if (more) {
            load_sz(st + 1, znext, snext);
            load_stage(st + 1);
        }

        // scale and zero of this stage's group for each A row of the lane
        const int g = (st * BK) / kGroup;
        uint32_t zb[TR];
        half2v s2[TR];
#pragma unroll
        for (int rt = 0; rt < TR; ++rt) {
            zb[rt] = zero_bias((zraw[rt] >> (4 * (g & 7))) & 0xFu);
            s2[rt] = as_h2(sraw[rt] | (sraw[rt] << 16));
        }

        u32x4 wv[TR];
#pragma unroll
        for (int rt = 0; rt < TR; ++rt)
            wv[rt] = *reinterpret_cast<const u32x4*>(
                &ws[cur][h * (BM * 16) + (wave_r * WR + rt * 32 + li) * 16]);

#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            half8 b[TC];
            const int ko = 4 * h + kk;
#pragma unroll
            for (int ct = 0; ct < TC; ++ct) {
                const int n = wave_c * WC + ct * 32 + li;
                b[ct] = *reinterpret_cast<const half8*>(&xs[cur][(ko * BN + xslot(n)) * 16]);
            }
#pragma unroll
            for (int rt = 0; rt < TR; ++rt) {
                const uint32_t word = kk == 0 ? wv[rt].x : kk == 1 ? wv[rt].y : kk == 2 ? wv[rt].z : wv[rt].w;
                const half8 av = dequant_word_scaled(word, zb[rt], s2[rt]);
#pragma unroll
                for (int ct = 0; ct < TC; ++ct)
                    acc[rt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, b[ct], acc[rt][ct], 0, 0, 0);
            }
        }

        if (more) {
            store_stage(cur ^ 1);
#pragma unroll
            for (int rt = 0; rt < TR; ++rt) {
                zraw[rt] = znext[rt];
                sraw[rt] = snext[rt];
            }
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds rows (e / 4) * 8 + 4 h + e % 4, column li
#pragma unroll
    for (int rt = 0; rt < TR; ++rt)
#pragma unroll
        for (int ct = 0; ct < TC; ++ct) {
            const int64_t col = col0 + wave_c * WC + ct * 32 + li;
            if (col < N) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = row0 + wave_r * WR + rt * 32 + (e >> 2) * 8 + 4 * h + (e & 3);
                    if (row < M) {
                        if (splitk == 1)
                            a.c[row * N + col] = (uint16_t)f32_to_h16_bits(acc[rt][ct][e]);
                        else
                            a.part[((int64_t)sidx * M + row) * N + col] = acc[rt][ct][e];
                    }
                }
            }
        }
    if (splitk == 1) return;

    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = atomicAdd(a.counters + tile_id, 1u);
        const int last = prev == (unsigned)(splitk - 1);
        if (last) atomicExch(a.counters + tile_id, 0u);
        flag = last;
    }
    __syncthreads();
    if (!flag) return;
    __threadfence();
    const int64_t rows_here = (M - row0) < BM ? (M - row0) : BM;
    const int64_t cols_here = (N - col0) < BN ? (N - col0) : BN;
    const int64_t total = rows_here * cols_here;
    for (int64_t e = tid; e < total; e += 256) {
        const int64_t row = row0 + e / cols_here;
        const int64_t col = col0 + e % cols_here;
        float v = 0.f;
        for (int s = 0; s < splitk; ++s)
            v += __builtin_nontemporal_load(a.part + ((int64_t)s * M + row) * N + col);
        a.c[row * N + col] = (uint16_t)f32_to_h16_bits(v);
    }
}

template <int BM, int BN>
hipError_t launch_bmbn(const GemmArgs& a, const TiledShape& t, hipStream_t stream) {
    const int64_t tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
    dim3 grid((unsigned)tiles, (unsigned)t.splitk);
    const bool vecx = (a.N % 8) == 0;
    if (vecx)
        hipLaunchKernelGGL((tiled_kernel<BM, BN, true>), grid, dim3(256), 0, stream, a, t.splitk);
    else
        hipLaunchKernelGGL((tiled_kernel<BM, BN, false>), grid, dim3(256), 0, stream, a, t.splitk);
    return hipGetLastError();
}

}  // namespace

bool tiled_supported(const TiledShape& t) {
    const bool bm_ok = t.bm == 128 || t.bm == 256;
    const bool bn_ok = t.bn == 64 || t.bn == 128 || t.bn == 256;
    return bm_ok && bn_ok && t.splitk >= 1;
}

int64_t tiled_tiles(const GemmArgs& a, const TiledShape& t) {
    return ((a.M + t.bm - 1) / t.bm) * ((a.N + t.bn - 1) / t.bn);
}

hipError_t launch_tiled(const GemmArgs& a, const TiledShape& t, hipStream_t stream) {
    if (t.bm == 256 && t.bn == 256) return launch_bmbn<256, 256>(a, t, stream);
    if (t.bm == 256 && t.bn == 128) return launch_bmbn<256, 128>(a, t, stream);
    if (t.bm == 256 && t.bn == 64) return launch_bmbn<256, 64>(a, t, stream);
    if (t.bm == 128 && t.bn == 256) return launch_bmbn<128, 256>(a, t, stream);
    if (t.bm == 128 && t.bn == 128) return launch_bmbn<128, 128>(a, t, stream);
    if (t.bm == 128 && t.bn == 64) return launch_bmbn<128, 64>(a, t, stream);
    return hipErrorInvalidValue;
}

}  // namespace w4a16
