// Skinny W4A16 kernel: few activation columns (N <= 64), the bandwidth-bound
// regime of PerfXLLM §3.3 (item 1 for few tokens, item 2 for one token).
//
// Every packed weight word is read from HBM exactly once, with 16-byte loads:
// lane (r, kb) of a wave reads words 4kb .. 4kb+3 of one 128-weight group of
// row r, so one load per lane brings in a whole group of 16 rows.  Each word
// is dequantized in registers to eight exact fp16 (q - z) values, which form
// the A operand of a 16x16x32 fp16 MFMA; the activations, staged once per
// workgroup in LDS in the matching order, form the B operand.  The four MFMAs
// of a group accumulate in fp32 and the group's scale is applied once to that
// fp32 partial (PerfXLLM §3.3 item 2 keeps scale and zero in shared memory:
// both are staged in LDS per workgroup).
//
// Work split (PerfXLLM §3.3 item 2 tiles both dimensions of the weight
// matrix): a workgroup owns 16 * rb * wm rows; its wk waves along K each take
// a contiguous run of groups and are summed through LDS; `splitk`
// workgroups may share one row tile, their fp32 partials summed in a fixed
// order by the last one to arrive.
#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

struct SkinnyLds {
    int ngs_max;    // groups per workgroup (upper bound)
    int bmw;        // rows per workgroup
    size_t x_off, s_off, z_off, flag_off, red_bytes, total;
};

template <int NCOL>
__host__ __device__ inline SkinnyLds skinny_layout(int G, int splitk, int rb, int wm, int wk) {
    constexpr int NB = NCOL >= 16 ? NCOL / 16 : 1;
    SkinnyLds L;
    L.ngs_max = (G + splitk - 1) / splitk;
    L.bmw = 16 * rb * wm;
    L.x_off = 0;
    size_t xb = (size_t)L.ngs_max * 16 * NCOL * 16;
    L.s_off = xb;
    size_t sb = (size_t)L.ngs_max * L.bmw * 2;
    L.z_off = L.s_off + ((sb + 15) & ~(size_t)15);
    size_t zb = (size_t)L.ngs_max * L.bmw;
    L.flag_off = L.z_off + ((zb + 15) & ~(size_t)15);
    size_t main_bytes = L.flag_off + 16;
    L.red_bytes = (size_t)(wk > 1 ? wk - 1 : 0) * wm * rb * NB * 4 * 64 * 4;
    L.total = main_bytes > L.red_bytes + 16 ? main_bytes : L.red_bytes + 16;
    // the arrival flag must not alias the reduction buffer
    if (L.flag_off < L.red_bytes) {
        L.flag_off = (L.red_bytes + 15) & ~(size_t)15;
        L.total = L.flag_off + 16;
        if (L.total < main_bytes) L.total = main_bytes;
    }
    return L;
}

template <int NCOL, int RB>
__global__ void __launch_bounds__(512) skinny_kernel(GemmArgs a, int wm, int wk, int splitk) {
    constexpr int NB = NCOL >= 16 ? NCOL / 16 : 1;
    constexpr int PF = 8 / RB;                 // groups prefetched per wave
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

    const int M = (int)a.M, N = (int)a.N, G = a.G;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wave_m = wave % wm;
    const int wave_k = wave / wm;
    const int nthreads = blockDim.x;
    const int li = lane & 15;     // MFMA row (A) / column (B) within a 16-block
    const int kb = lane >> 4;     // which quarter of the 32-k MFMA step

    const SkinnyLds L = skinny_layout<NCOL>(G, splitk, RB, wm, wk);
    unsigned char* xs = smem + L.x_off;
    uint16_t* ss = reinterpret_cast<uint16_t*>(smem + L.s_off);
    uint8_t* zs = smem + L.z_off;

    const int bmw = L.bmw;
    const int64_t tile_row0 = (int64_t)blockIdx.x * bmw;
    const int sidx = blockIdx.y;
    const int gs0 = (int)((int64_t)G * sidx / splitk);
    const int gs1 = (int)((int64_t)G * (sidx + 1) / splitk);
    const int ngs = gs1 - gs0;
    const int gw0 = gs0 + ngs * wave_k / wk;
    const int gw1 = gs0 + ngs * (wave_k + 1) / wk;
    const int ng = gw1 - gw0;

    // ---- issue the first weight loads before anything else
    const int64_t KW = a.K / 8;
    const uint32_t* wrow[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        int64_t row = tile_row0 + wave_m * 16 * RB + rb * 16 + li;
        if (row > M - 1) row = M - 1;
        wrow[rb] = a.qpk + row * KW + kb * 4;
    }
    u32x4 buf[PF][RB];
#pragma unroll
    for (int p = 0; p < PF; ++p) {
        if (p < ng) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
                buf[p][rb] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(wrow[rb] + (int64_t)(gw0 + p) * 16));
        }
    }

    // ---- stage activations (in dequant order), scales and zeros in LDS
    if (NCOL == 1) {
        for (int f = threadIdx.x; f < ngs * 16; f += nthreads) {
            const int gl = f >> 4, i = (f >> 2) & 3, q = f & 3;
            const int64_t k0 = (int64_t)(gs0 + gl) * kGroup + q * 32 + i * 8;
            u32x4 v = *reinterpret_cast<const u32x4*>(a.x + k0);
            *reinterpret_cast<u32x4*>(xs + (size_t)f * 16) = permute_k8(v);
        }
    } else {
        for (int u = threadIdx.x; u < ngs * 16 * NCOL; u += nthreads) {
            const int f = u / NCOL, j = u - f * NCOL;
            const int gl = f >> 4, i = (f >> 2) & 3, q = f & 3;
            const int64_t k0 = (int64_t)(gs0 + gl) * kGroup + q * 32 + i * 8;
            u32x4 r = {0u, 0u, 0u, 0u};
            if (j < N) {
                const uint16_t* col = a.x + k0 * N + j;
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = col[(int64_t)e * N];
                r.x = h[0] | (h[4] << 16);
                r.y = h[1] | (h[5] << 16);
                r.z = h[2] | (h[6] << 16);
                r.w = h[3] | (h[7] << 16);
            }
            *reinterpret_cast<u32x4*>(xs + (size_t)u * 16) = r;
        }
    }
    for (int e = threadIdx.x; e < ngs * bmw; e += nthreads) {
        const int gl = e / bmw, r = e - gl * bmw;
        int64_t row = tile_row0 + r;
        if (row > M - 1) row = M - 1;
        const int g = gs0 + gl;
        ss[e] = a.scales[row * G + g];
        zs[e] = (uint8_t)((a.zpk[row * a.ZW + (g >> 3)] >> (4 * (g & 7))) & 0xFu);
    }
    __syncthreads();

    // ---- main loop over this wave's groups
    floatx4 acc[RB][NB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};

    const int rowoff_a = wave_m * 16 * RB + li;        // A-operand row of this lane
    const int rowoff_c = wave_m * 16 * RB + 4 * kb;    // first C row of this lane

    for (int gb = 0; gb < ng; gb += PF) {
#pragma unroll
        for (int p = 0; p < PF; ++p) {
            const int gi = gb + p;
            if (gi < ng) {
                u32x4 w[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) w[rb] = buf[p][rb];
                if (gi + PF < ng) {
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        buf[p][rb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                            wrow[rb] + (int64_t)(gw0 + gi + PF) * 16));
                }
                const int gl = gw0 + gi - gs0;
                uint32_t zb[RB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) zb[rb] = zero_bias(zs[gl * bmw + rowoff_a + rb * 16]);
                floatx4 part[RB][NB];
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int cb = 0; cb < NB; ++cb) part[rb][cb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    half8 b[NB];
                    const size_t fbase = ((size_t)(gl * 16 + i * 4 + kb)) * NCOL;
#pragma unroll
                    for (int cb = 0; cb < NB; ++cb) {
                        const int j = cb * 16 + li;
                        if (NCOL >= 16 || j < NCOL) {
                            b[cb] = *reinterpret_cast<const half8*>(xs + (fbase + j) * 16);
                        } else {
                            b[cb] = half8{0, 0, 0, 0, 0, 0, 0, 0};
                        }
                    }
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb) {
                        const uint32_t word = i == 0 ? w[rb].x : i == 1 ? w[rb].y : i == 2 ? w[rb].z : w[rb].w;
                        const half8 av = dequant_word(word, zb[rb]);
#pragma unroll
                        for (int cb = 0; cb < NB; ++cb)
                            part[rb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, b[cb], part[rb][cb], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    const uint2 sv = *reinterpret_cast<const uint2*>(ss + gl * bmw + rowoff_c + rb * 16);
                    const float s0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv.x & 0xFFFF));
                    const float s1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv.x >> 16));
                    const float s2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv.y & 0xFFFF));
                    const float s3 = (float)__builtin_bit_cast(_Float16, (uint16_t)(sv.y >> 16));
#pragma unroll
                    for (int cb = 0; cb < NB; ++cb) {
                        acc[rb][cb][0] = __builtin_fmaf(s0, part[rb][cb][0], acc[rb][cb][0]);
                        acc[rb][cb][1] = __builtin_fmaf(s1, part[rb][cb][1], acc[rb][cb][1]);
                        acc[rb][cb][2] = __builtin_fmaf(s2, part[rb][cb][2], acc[rb][cb][2]);
                        acc[rb][cb][3] = __builtin_fmaf(s3, part[rb][cb][3], acc[rb][cb][3]);
                    }
                }
            }
        }
    }

    // ---- sum the wk waves of a row block through LDS
    if (wk > 1) {
        __syncthreads();   // everyone is done with the staged activations
        float* red = reinterpret_cast<float*>(smem);
        if (wave_k > 0) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const size_t idx = (((((size_t)(wave_k - 1) * wm + wave_m) * RB + rb) * NB + cb) * 4 + r) * 64 + lane;
                        red[idx] = acc[rb][cb][r];
                    }
        }
        __syncthreads();
        if (wave_k == 0) {
            for (int kk = 1; kk < wk; ++kk) {
#pragma unroll
                for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                    for (int cb = 0; cb < NB; ++cb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const size_t idx = (((((size_t)(kk - 1) * wm + wave_m) * RB + rb) * NB + cb) * 4 + r) * 64 + lane;
                            acc[rb][cb][r] += red[idx];
                        }
            }
        }
    }

    // ---- epilogue
    if (wave_k == 0) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int cb = 0; cb < NB; ++cb) {
                const int col = cb * 16 + li;
                if (col < N) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int64_t row = tile_row0 + rowoff_c + rb * 16 + r;
                        if (row < M) {
                            if (splitk == 1)
                                a.c[row * N + col] = (uint16_t)f32_to_h16_bits(acc[rb][cb][r]);
                            else
                                a.part[((int64_t)sidx * M + row) * N + col] = acc[rb][cb][r];
                        }
                    }
                }
            }
    }
    if (splitk == 1) return;

    // ---- split-K: the last workgroup of a row tile sums the partials in order
    int* flag = reinterpret_cast<int*>(smem + L.flag_off);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = atomicAdd(a.counters + blockIdx.x, 1u);
        const int last = prev == (unsigned)(splitk - 1);
        if (last) atomicExch(a.counters + blockIdx.x, 0u);
        *flag = last;
    }
    __syncthreads();
    if (!*flag) return;
    __threadfence();
    const int64_t rows_here = (M - tile_row0) < bmw ? (M - tile_row0) : bmw;
    const int64_t total = rows_here * N;
    for (int64_t e = threadIdx.x; e < total; e += nthreads) {
        const int64_t row = tile_row0 + e / N;
        const int64_t col = e - (e / N) * N;
        float v = 0.f;
        for (int s = 0; s < splitk; ++s)
            v += __builtin_nontemporal_load(a.part + ((int64_t)s * M + row) * N + col);
        a.c[row * N + col] = (uint16_t)f32_to_h16_bits(v);
    }
}

template <int NCOL>
size_t lds_for(const GemmArgs& a, const SkinnyShape& s) {
    return skinny_layout<NCOL>(a.G, s.splitk, s.rb, s.wm, s.wk).total;
}

template <int NCOL, int RB>
hipError_t launch_one(const GemmArgs& a, const SkinnyShape& s, hipStream_t stream) {
    const size_t lds = lds_for<NCOL>(a, s);
    const int64_t bmw = 16 * RB * s.wm;
    dim3 grid((unsigned)((a.M + bmw - 1) / bmw), (unsigned)s.splitk);
    dim3 block((unsigned)(64 * s.wm * s.wk));
    hipLaunchKernelGGL((skinny_kernel<NCOL, RB>), grid, block, lds, stream, a, s.wm, s.wk, s.splitk);
    return hipGetLastError();
}

template <int NCOL>
hipError_t launch_rb(const GemmArgs& a, const SkinnyShape& s, hipStream_t stream) {
    return s.rb == 1 ? launch_one<NCOL, 1>(a, s, stream) : launch_one<NCOL, 2>(a, s, stream);
}

}  // namespace

bool skinny_supported(const SkinnyShape& s) {
    const bool ncol_ok = s.ncol == 1 || s.ncol == 2 || s.ncol == 4 || s.ncol == 8 ||
                         s.ncol == 16 || s.ncol == 32 || s.ncol == 64;
    return ncol_ok && (s.rb == 1 || s.rb == 2) && s.wm >= 1 && s.wk >= 1 &&
           s.wm * s.wk <= 8 && s.splitk >= 1;
}

int64_t skinny_row_tiles(const GemmArgs& a, const SkinnyShape& s) {
    const int64_t bmw = 16LL * s.rb * s.wm;
    return (a.M + bmw - 1) / bmw;
}

size_t skinny_lds_bytes(const GemmArgs& a, const SkinnyShape& s) {
    switch (s.ncol) {
        case 1: return lds_for<1>(a, s);
        case 2: return lds_for<2>(a, s);
        case 4: return lds_for<4>(a, s);
        case 8: return lds_for<8>(a, s);
        case 16: return lds_for<16>(a, s);
        case 32: return lds_for<32>(a, s);
        case 64: return lds_for<64>(a, s);
        default: return 0;
    }
}

hipError_t launch_skinny(const GemmArgs& a, const SkinnyShape& s, hipStream_t stream) {
    switch (s.ncol) {
        case 1: return launch_rb<1>(a, s, stream);
        case 2: return launch_rb<2>(a, s, stream);
        case 4: return launch_rb<4>(a, s, stream);
        case 8: return launch_rb<8>(a, s, stream);
        case 16: return launch_rb<16>(a, s, stream);
        case 32: return launch_rb<32>(a, s, stream);
        case 64: return launch_rb<64>(a, s, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
