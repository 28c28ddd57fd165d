// C ABI of the W4A16 linear layer: argument checks, plan choice, dispatch.
//
// Every check happens on the host before any HIP call.  The two regimes of
// PerfXLLM §3.3 item 1 (few tokens: bandwidth-bound; many tokens:
// compute-bound, each with its own tiling) map to the skinny and the tiled
// kernel; w4a16_plan_default() picks one from the shape.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <math.h>
#include <string>
#include <vector>

#include "../../include/w4a16.h"
#include "launch.hpp"

using namespace w4a16;

namespace {

thread_local std::string g_err;

constexpr int kGroupSize = 128;
constexpr int64_t kMaxDim = (int64_t)1 << 31;   // each of M, N, K below 2^31
// Split reductions keep one arrival counter per output tile at a fixed place,
// the first 64 KB of the workspace, so partial sums of one call can never
// land on the counters of another call with a different shape.
constexpr int64_t kCounterSlots = 16384;
// compute units of an MI355X (default plans balance tiles over them)
constexpr int64_t kCus = 256;
constexpr size_t kCounterBytes = kCounterSlots * 4;

int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int ok() {
    g_err.clear();
    return W4A16_OK;
}

bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

int check_dims(int64_t M, int64_t N, int64_t K, int32_t group_size) {
    if (group_size != kGroupSize)
        return fail(W4A16_ERR_UNSUPPORTED, "group_size must be 128, got %d", (int)group_size);
    if (M < 1 || N < 1 || K < kGroupSize)
        return fail(W4A16_ERR_INVALID_ARG, "need M >= 1, N >= 1, K >= 128 (M=%lld N=%lld K=%lld)",
                    (long long)M, (long long)N, (long long)K);
    if (K % kGroupSize)
        return fail(W4A16_ERR_INVALID_ARG, "K=%lld is not a multiple of 128", (long long)K);
    if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return fail(W4A16_ERR_INVALID_ARG, "M, N and K must each be below 2^31");
    // byte sizes used below: M*K/2, M*N*4*splitk; keep them far from overflow
    if ((double)M * (double)K > 9.0e18 || (double)M * (double)N * 4.0 * 64.0 > 9.0e18)
        return fail(W4A16_ERR_INVALID_ARG, "problem too large");
    return W4A16_OK;
}

int64_t groups_of(int64_t K) { return K / kGroupSize; }
int64_t zwords_of(int64_t K) { return (groups_of(K) + 7) / 8; }

bool skinny_columns(int64_t N) { return (N >= 1 && N <= 8) || N == 16 || N == 32; }

GemmArgs make_args(int64_t M, int64_t N, int64_t K, int32_t layout = W4A16_LAYOUT_KN) {
    GemmArgs a;
    memset(&a, 0, sizeof(a));
    a.tm = layout == W4A16_LAYOUT_TOKEN ? 1 : 0;
    a.M = M;
    a.N = N;
    a.K = K;
    a.G = (int32_t)groups_of(K);
    a.ZW = (int32_t)zwords_of(K);
    return a;
}

SkinnyShape skinny_of(const w4a16_plan& p) { return SkinnyShape{p.ncol, p.rb, p.wm, p.wk, p.splitk}; }
TiledShape tiled_of(const w4a16_plan& p) {
    return TiledShape{p.bm, p.bn, p.splitk, p.wm == 0 ? 4 : p.wm, p.pf == 0 ? 1 : p.pf, p.xpf == 0 ? 1 : p.xpf,
                      p.wk == 0 ? 1 : p.wk};
}
NarrowShape narrow_of(const w4a16_plan& p) {
    return NarrowShape{p.ncol, p.pf, p.splitk, p.rb == 0 ? 2 : p.rb, p.wk == 0 ? 1 : p.wk, p.wm == 0 ? 4 : p.wm};
}

int check_plan(const GemmArgs& a, const w4a16_plan& p);

// Default plan (measured on MI355X on the LLaMA-7B shapes; any valid plan
// is correct, this one only decides speed).
//
// Narrow kernel for 8 <= N <= 32 (see below).  Skinny kernel for N < 8,
// for N = 8 and 16 on a small [K, N] matrix, and for N = 32 when the
// matrix is small and no narrow plan fits
// (below 2^25 weights the tiled kernel has too few tiles to stream the
// weights fast).  One 16-row block per wave (several waves along M share
// the staged activations when N grows), about eight groups per wave along K
// so that all of a wave's weight loads are in flight at once, and a split
// across workgroups only when the staged activations would not fit in LDS.
//
// Tiled kernel otherwise: 256 x 128 tiles from N = 4096 on (from N = 1024
// when that still gives 256 tiles), 128 x 128 from N = 256, 128 x 64 below
// (weights two stages ahead), 512 x 128 tiles of eight waves instead of
// 256 x 128 where they load the CUs as evenly (e.g. N = 1024 and 4096 at
// M = 12288, not N = 2048); a split along K only when there are too few
// tiles to fill the chip (N <= 32: two-way, four-way under 64 tiles; larger
// N: two-way up to N = 128 and for long rows, K >= 8192).
//
// Token-major layout: the same choice, except that the skinny kernel takes
// token-major activations only up to N = 8 (N = 16 and 32 go to the narrow
// or tiled kernel).
w4a16_plan default_plan(int64_t M, int64_t N, int64_t K, int32_t layout = W4A16_LAYOUT_KN) {
    w4a16_plan p;
    memset(&p, 0, sizeof(p));
    const int64_t G = groups_of(K);
    const GemmArgs a = make_args(M, N, K, layout);
    // narrow kernel for 8 <= N <= 32 (N = 8 and 16 on a small [K, N] matrix
    // go to the skinny kernel: 4096x4096 8.1 / 8.7 against 9.2 / 9.2 us), a
    // ring of 4 groups per wave (against 8: 12288x4096 N = 32 16.3 -> 15.2
    // us, 4096x11008 N = 16 / 32 13.0 / 17.5 -> 12.3 / 15.6 us, 22016x4096
    // N = 16 15.9 -> 15.2 us, the rest equal), one wave along K per row block, the
    // smallest split whose activations fit in LDS (each workgroup then holds
    // a CU's LDS, so about 192 workgroups stream best):
    // - 16 staged columns: 64 rows per workgroup, 128 (96 when those still
    //   fit one per CU) when 64-row tiles outnumber the CUs;
    // - 32 staged columns: 128 rows where 64-row tiles would give at least
    //   one workgroup per CU, with more splits while the workgroups still
    //   fit one per CU and 96-row tiles (three waves) where those do
    //   (12288x4096: 13.9 -> 13.7 us; 4096x11008: 15.6 -> 15.0 us; 22016x4096,
    //   in place of the tiled kernel: 27.5 -> 25.7 us), else 64 rows and
    //   more splits up to one workgroup per CU (4096x4096: 9.7 -> 9.4 us).
    const bool small = M * K < ((int64_t)1 << 25);
    const bool small_kn = small && !a.tm && (N == 8 || N == 16);
    if (N >= 8 && N <= 32 && !small_kn) {
        p.kernel = W4A16_KERNEL_NARROW;
        p.ncol = N <= 16 ? 16 : 32;
        p.pf = 4;
        p.wk = 1;
        auto fits = [&](const w4a16_plan& q) {
            const std::string saved = g_err;
            const int st = check_plan(a, q);
            g_err = saved;
            return st == W4A16_OK;
        };
        // smallest feasible split with 64-row tiles
        p.rb = 1;
        int64_t smin = 0;
        for (int64_t splitk = 1; splitk <= G && !smin; ++splitk) {
            p.splitk = (int32_t)splitk;
            if (fits(p)) smin = splitk;
        }
        const int64_t t64 = (M + 63) / 64, t128 = (M + 127) / 128;
        bool use = smin > 0;
        if (use && p.ncol == 16) {
            p.rb = t64 > kCus ? 2 : 1;
            p.splitk = (int32_t)smin;
            if (p.rb == 1) {
                // more splits while every workgroup still has a CU of its own
                // (4096x11008 N = 8 / 16: 13.6 -> 13.0 us)
                while (t64 * (p.splitk + 1) <= kCus) {
                    w4a16_plan q = p;
                    q.splitk = p.splitk + 1;
                    if (!fits(q)) break;
                    p = q;
                }
            } else if (p.splitk == 1 && (M + 95) / 96 <= kCus) {
                // 96-row tiles (three waves) where 128-row tiles leave CUs
                // idle (22016x4096 N = 8 / 16: 17.4 -> 15.9 us)
                p.wm = 3;
            }
            use = fits(p);
        } else if (use) {
            if (t64 * smin >= kCus) {
                p.rb = 2;
                p.splitk = (int32_t)smin;
                while (t128 * (p.splitk + 1) <= kCus) {
                    w4a16_plan q = p;
                    q.splitk = p.splitk + 1;
                    if (!fits(q)) break;
                    p = q;
                }
                if ((M + 95) / 96 * p.splitk <= kCus) {
                    w4a16_plan q = p;
                    q.wm = 3;
                    if (fits(q)) p = q;
                }
                use = fits(p);
            } else {
                p.splitk = (int32_t)smin;
                while (t64 * (p.splitk + 1) <= kCus) {
                    w4a16_plan q = p;
                    q.splitk = p.splitk + 1;
                    if (!fits(q)) break;
                    p = q;
                }
            }
        }
        if (use) return p;
        memset(&p, 0, sizeof(p));
    }
    // 33 <= N <= 64: the narrow kernel with 64 staged columns where its
    // smallest feasible split still leaves every workgroup a CU
    // (4096x4096 N = 40 / 64: 19.9 / 20.4 -> 14.3 / 14.4 us against the
    // tiled kernel; at 12288 rows or K = 11008 the tiled kernel stays)
    if (N > 32 && N <= 64) {
        p.kernel = W4A16_KERNEL_NARROW;
        p.ncol = 64;
        p.pf = 4;
        p.rb = 1;
        p.wk = 1;
        const int64_t t64 = (M + 63) / 64;
        auto fits64 = [&](const w4a16_plan& q) {
            const std::string saved = g_err;
            const int st = check_plan(a, q);
            g_err = saved;
            return st == W4A16_OK;
        };
        for (int64_t splitk = 1; splitk <= G && t64 * splitk <= kCus; ++splitk) {
            p.splitk = (int32_t)splitk;
            if (fits64(p)) {
                // more splits, up to six, while the workgroups still fit
                // the CUs (2048x4096 / 1024x4096 N = 64: 12.9 / 12.7 ->
                // 12.1 / 12.0 us at six)
                while (p.splitk < 6 && t64 * (p.splitk + 1) <= kCus && G / (p.splitk + 1) >= 4) {
                    w4a16_plan q = p;
                    q.splitk = p.splitk + 1;
                    if (!fits64(q)) break;
                    p = q;
                }
                return p;
            }
        }
        memset(&p, 0, sizeof(p));
    }
    if (N < 8 || (!a.tm && skinny_columns(N) && small)) {
        p.kernel = W4A16_KERNEL_SKINNY;
        p.ncol = (int32_t)N;
        p.rb = 1;
        p.wm = N <= 8 || small_kn ? 1 : 4;
        const int64_t rows = 16LL * p.rb * p.wm;
        const int64_t tiles = (M + rows - 1) / rows;
        for (int64_t splitk = 1; splitk <= G; ++splitk) {
            const int64_t ngs = (G + splitk - 1) / splitk;
            int64_t wk = (ngs + 4) / 8;
            if (wk < 1) wk = 1;
            while (wk * p.wm > 16) wk /= 2;
            // small grids: more waves along K (at least two groups each);
            // up to twice as many while every wave keeps four groups
            // (measured: 12288x4096 N = 1, 2 and 22016x4096 N = 1 gain
            // 2-6 %)
            while (wk * 2 * p.wm <= 16 && ngs >= 4 * wk &&
                   (tiles * splitk * p.wm * wk < 2048 ||
                    (tiles * splitk * p.wm * wk < 8192 && ngs >= 8 * wk)))
                wk *= 2;
            p.wk = (int32_t)wk;
            p.splitk = (int32_t)splitk;
            if (splitk > 1 && tiles > kCounterSlots) break;
            const std::string saved = g_err;
            const int st = check_plan(a, p);
            g_err = saved;
            if (st == W4A16_OK) return p;
        }
        memset(&p, 0, sizeof(p));
    }
    p.kernel = W4A16_KERNEL_TILED;
    p.wm = 4;
    if (N < 1024) {
        // Few columns: 128-row tiles, as many workgroups as CUs or a little
        // fewer.  128-column tiles when N > 64 and they alone give 160 or more
        // (at N <= 64 half of each would be empty: 22016x4096 N = 64 38.2
        // against 25.7 us with 96 x 64 tiles), with two
        // K slices while that is one workgroup per CU (12288x4096 N = 192 /
        // 256: 43.3 / 45.2 -> 40.2 / 41.4 us; 22016x4096 N = 128, 172
        // tiles: 50.0 -> 41.6 us); else 64-column tiles, weights two stages
        // ahead, split along K up to 256 workgroups while every split keeps
        // 8 groups (4096x4096 N = 128: 20.4 -> 17.2 us at four splits;
        // 4096x11008 N = 64: 26.8 -> 21.6 us at eight).
        const int64_t tm = (M + 127) / 128;
        const int64_t t128 = tm * ((N + 127) / 128), t64 = tm * ((N + 63) / 64);
        p.bm = 128;
        p.splitk = 1;
        if (N > 64 && t128 >= 160) {
            p.bn = 128;
            if (t128 <= kCus) p.wk = 2;
        } else if (N > 64 && t128 >= 96 && G >= 64 && t128 <= kCounterSlots) {
            // long K: 128-column tiles split along K to fill the CUs
            // (4096x11008 N = 384 / 512: 67.3 / 75.4 -> 61.2 / 67.8 us; at
            // K = 4096 the 64-column tiles stay ahead)
            p.bn = 128;
            p.pf = 2;
            p.splitk = (int32_t)(kCus / t128);
        } else {
            p.bn = 64;
            p.pf = 2;
            if (t64 <= kCounterSlots)
                while (p.splitk < 8 && t64 * (p.splitk + 1) <= kCus && G / (p.splitk + 1) >= 8) ++p.splitk;
            // 96-row tiles of three waves where 128-row ones leave a fifth
            // of the CUs idle and these nearly fill them (12288x4096 N = 48
            // / 64 / 128: 21.7 / 21.2 / 28.7 -> 20.3 / 20.3 / 27.6 us;
            // 11008x4096 N = 64 / 128: 21.3 / 28.7 -> 20.7 / 27.5 us)
            const int64_t t96 = ((M + 95) / 96) * ((N + 63) / 64);
            if (t64 * p.splitk < 200 && t96 * p.splitk >= 224 && t96 * p.splitk <= kCus &&
                (p.splitk == 1 || t96 <= kCounterSlots)) {
                p.bm = 96;
                p.wm = 3;
            }
        }
        return p;
    }
    // 256-row tiles from N = 1024 on when they still give 256 tiles
    p.bm = (N >= 4096 || ((M + 255) / 256) * ((N + 127) / 128) >= 256) ? 256 : 128;
    p.bn = 128;
    // 512 x 128 tiles of eight waves (weights two stages ahead) when they
    // give a CU no more rows than 256 x 128 tiles do: with one of them per
    // CU against two of the others, the busiest CU then has the same work
    // and the activation chunks are staged half as often
    if (M >= 512) {
        const int64_t t256 = ((M + 255) / 256) * ((N + 127) / 128);
        const int64_t t512 = ((M + 511) / 512) * ((N + 127) / 128);
        if ((t512 + kCus - 1) / kCus * 512 <= (t256 + kCus - 1) / kCus * 256) {
            p.bm = 512;
            p.wm = 8;
            p.pf = 2;
        }
    }
    const int64_t t = ((M + p.bm - 1) / p.bm) * ((N + p.bn - 1) / p.bn);
    int64_t splitk = 1;
    if (t < 160 && t <= kCounterSlots && K >= 8192) splitk = 2;
    while (splitk > G) splitk /= 2;
    p.splitk = (int32_t)splitk;
    return p;
}

int64_t tiles_of(const GemmArgs& a, const w4a16_plan& p) {
    if (p.kernel == W4A16_KERNEL_NARROW) return narrow_row_tiles(a, narrow_of(p));
    return p.kernel == W4A16_KERNEL_SKINNY ? skinny_row_tiles(a, skinny_of(p))
                                           : tiled_tiles(a, tiled_of(p));
}

// Workspace layout: [counters: 64 KB][fp32 partials: splitk * M * N for the
// skinny kernel, splitk whole tiles per tile (in the register layout of the
// waves that hold the sums) for the tiled and narrow kernels]
// [tiled and narrow kernels: activation chunks, K * N fp16, at a 256-byte boundary].
size_t partial_bytes(const GemmArgs& a, const w4a16_plan& p) {
    if (p.kernel == W4A16_KERNEL_TILED) return tiled_partial_bytes(a, tiled_of(p));
    if (p.kernel == W4A16_KERNEL_NARROW) return narrow_partial_bytes(a, narrow_of(p));
    return p.splitk <= 1 ? 0 : (size_t)p.splitk * (size_t)a.M * (size_t)a.N * 4;
}
size_t chunks_offset(const GemmArgs& a, const w4a16_plan& p) {
    return (kCounterBytes + partial_bytes(a, p) + 255) & ~(size_t)255;
}
// (no chunk area where the plan reads x in place)
size_t workspace_bytes_for(const GemmArgs& a, const w4a16_plan& p) {
    if (p.kernel == W4A16_KERNEL_TILED)
        return chunks_offset(a, p) + (tiled_direct_x(a, tiled_of(p)) ? 0 : xpack_bytes(a));
    if (p.kernel == W4A16_KERNEL_NARROW)
        return chunks_offset(a, p) + (narrow_direct_x(a) ? 0 : xpack_bytes(a));
    if (p.splitk <= 1) return 0;
    return kCounterBytes + partial_bytes(a, p);
}

int check_plan(const GemmArgs& a, const w4a16_plan& p) {
    if (p.splitk > 65535)
        return fail(W4A16_ERR_UNSUPPORTED, "splitk=%d above the grid limit 65535", p.splitk);
    if (p.kernel == W4A16_KERNEL_SKINNY) {
        const SkinnyShape s = skinny_of(p);
        if (!skinny_supported(s))
            return fail(W4A16_ERR_UNSUPPORTED, "skinny plan invalid (ncol=%d rb=%d wm=%d wk=%d splitk=%d)",
                        p.ncol, p.rb, p.wm, p.wk, p.splitk);
        if (p.ncol != a.N)
            return fail(W4A16_ERR_UNSUPPORTED, "skinny plan is built for %d columns but N=%lld", p.ncol,
                        (long long)a.N);
        if (p.splitk > a.G)
            return fail(W4A16_ERR_UNSUPPORTED, "splitk=%d exceeds the %d groups of a row", p.splitk, a.G);
        if (p.splitk > 1 && tiles_of(a, p) > kCounterSlots)
            return fail(W4A16_ERR_UNSUPPORTED, "split plans support at most %lld row tiles",
                        (long long)kCounterSlots);
        const char* why = skinny_check(a, s);
        if (why) return fail(W4A16_ERR_UNSUPPORTED, "skinny plan: %s", why);
        return W4A16_OK;
    }
    if (p.kernel == W4A16_KERNEL_TILED) {
        const TiledShape t = tiled_of(p);
        if (!tiled_supported(t))
            return fail(W4A16_ERR_UNSUPPORTED, "tiled plan invalid (bm=%d bn=%d splitk=%d)", p.bm, p.bn,
                        p.splitk);
        if (p.splitk > 1 && tiles_of(a, p) > kCounterSlots)
            return fail(W4A16_ERR_UNSUPPORTED, "split plans support at most %lld tiles",
                        (long long)kCounterSlots);
        if (p.splitk > a.G)
            return fail(W4A16_ERR_UNSUPPORTED, "splitk=%d exceeds the %d groups of a row", p.splitk, a.G);
        const char* why = tiled_check(a, t);
        if (why) return fail(W4A16_ERR_UNSUPPORTED, "tiled plan: %s", why);
        return W4A16_OK;
    }
    if (p.kernel == W4A16_KERNEL_NARROW) {
        const NarrowShape n = narrow_of(p);
        if (!narrow_supported(n))
            return fail(W4A16_ERR_UNSUPPORTED, "narrow plan invalid (ncol=%d pf=%d splitk=%d)", p.ncol, p.pf,
                        p.splitk);
        if (p.splitk > 1 && tiles_of(a, p) > kCounterSlots)
            return fail(W4A16_ERR_UNSUPPORTED, "split plans support at most %lld row tiles",
                        (long long)kCounterSlots);
        const char* why = narrow_check(a, n);
        if (why) return fail(W4A16_ERR_UNSUPPORTED, "narrow plan: %s", why);
        return W4A16_OK;
    }
    return fail(W4A16_ERR_UNSUPPORTED, "unknown kernel id %d", p.kernel);
}

int check_layout(int32_t layout) {
    if (layout != W4A16_LAYOUT_KN && layout != W4A16_LAYOUT_TOKEN)
        return fail(W4A16_ERR_INVALID_ARG, "unknown layout %d", layout);
    return W4A16_OK;
}

// dry: check everything, launch nothing (a composite call validates all of
// its steps before it enqueues the first one)
int run_gemm(const uint32_t* qpk, const void* scales, const uint32_t* zpk, const void* x, void* c,
             int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t layout, const w4a16_plan* plan_in,
             void* workspace, size_t workspace_bytes, void* stream, bool dry = false, int32_t act = 0) {
    int st = check_dims(M, N, K, group_size);
    if (st) return st;
    st = check_layout(layout);
    if (st) return st;
    if (act && layout != W4A16_LAYOUT_TOKEN)
        return fail(W4A16_ERR_INVALID_ARG, "the gated activation prologue takes token-major activations");
    if (!qpk || !scales || !zpk || !x || !c)
        return fail(W4A16_ERR_INVALID_ARG, "null data pointer");
    if (!aligned16(qpk) || !aligned16(scales) || !aligned16(zpk) || !aligned16(x) || !aligned16(c))
        return fail(W4A16_ERR_MISALIGNED, "every data pointer must be 16-byte aligned");
    const int64_t G = groups_of(K);
    const size_t nq = (size_t)M * (size_t)(K / 8) * 4, ns = (size_t)M * G * 2,
                 nz = (size_t)M * zwords_of(K) * 4, nx = (size_t)K * N * 2 * (act ? 2 : 1), nc = (size_t)M * N * 2;
    if (overlaps(c, nc, qpk, nq) || overlaps(c, nc, scales, ns) || overlaps(c, nc, zpk, nz) ||
        overlaps(c, nc, x, nx))
        return fail(W4A16_ERR_INVALID_ARG, "output overlaps an input");

    GemmArgs a = make_args(M, N, K, layout);
    a.act = act ? 1 : 0;
    const w4a16_plan p = plan_in ? *plan_in : default_plan(M, N, K, layout);
    st = check_plan(a, p);
    if (st) return st;
    const size_t need = workspace_bytes_for(a, p);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(W4A16_ERR_MISALIGNED, "workspace must be 16-byte aligned");
        if (overlaps(workspace, need, c, nc) || overlaps(workspace, need, qpk, nq) ||
            overlaps(workspace, need, scales, ns) || overlaps(workspace, need, zpk, nz) ||
            overlaps(workspace, need, x, nx))
            return fail(W4A16_ERR_INVALID_ARG, "workspace overlaps a data buffer");
        a.counters = static_cast<uint32_t*>(workspace);
        a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
        // the chunk area, where the plan has one (workspace_bytes_for)
        if (need > chunks_offset(a, p) &&
            (p.kernel == W4A16_KERNEL_TILED || p.kernel == W4A16_KERNEL_NARROW))
            a.xp = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + chunks_offset(a, p));
    }
    a.qpk = qpk;
    a.scales = static_cast<const uint16_t*>(scales);
    a.zpk = zpk;
    a.x = static_cast<const uint16_t*>(x);
    a.c = static_cast<uint16_t*>(c);
    if (dry) return ok();

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = p.kernel == W4A16_KERNEL_SKINNY   ? launch_skinny(a, skinny_of(p), s)
                   : p.kernel == W4A16_KERNEL_NARROW ? launch_narrow(a, narrow_of(p), s)
                                                     : launch_tiled(a, tiled_of(p), s);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Candidate plans for the tuner: every kernel family that can take the
// shape, over the plan fields that matter (the default plan first).
std::vector<w4a16_plan> candidate_plans(const GemmArgs& a) {
    std::vector<w4a16_plan> out;
    auto add = [&](w4a16_plan p) {
        const std::string saved = g_err;
        const int st = check_plan(a, p);
        g_err = saved;
        if (st == W4A16_OK) out.push_back(p);
    };
    w4a16_plan p;
    memset(&p, 0, sizeof(p));
    add(default_plan(a.M, a.N, a.K, a.tm ? W4A16_LAYOUT_TOKEN : W4A16_LAYOUT_KN));
    const int64_t N = a.N;
    if (skinny_columns(N)) {
        for (int wm : {1, 2, 4})
            for (int wk : {1, 2, 4, 8, 16})
                for (int splitk : {1, 2, 3, 4}) {
                    if (wm * wk > 16) continue;
                    memset(&p, 0, sizeof(p));
                    p.kernel = W4A16_KERNEL_SKINNY;
                    p.ncol = (int32_t)N;
                    p.rb = 1;
                    p.wm = wm;
                    p.wk = wk;
                    p.splitk = splitk;
                    add(p);
                }
    }
    if (N <= 64) {
        for (int ncol : {16, 32, 64})
            for (int pf : {4, 8, 16})
                for (int rb : {1, 2})
                    for (int wk : {1, 2, 4})
                        for (int wm : {4, 3})
                            for (int splitk : {1, 2, 3, 4, 6, 8}) {
                                if (ncol < N || (wm == 3 && wk != 1)) continue;
                                memset(&p, 0, sizeof(p));
                                p.kernel = W4A16_KERNEL_NARROW;
                                p.ncol = ncol;
                                p.pf = pf;
                                p.rb = rb;
                                p.wk = wk;
                                p.wm = wm;
                                p.splitk = splitk;
                                add(p);
                            }
    }
    if (N >= 8) {
        const int pipes[][2] = {{0, 0}, {2, 0}, {2, 2}, {4, 2}, {4, 3}};   // (pf, xpf)
        for (int bm : {128, 256, 512})
            for (int bn : {64, 128, 256})
                for (int wm : {4, 2, 8})
                    for (const auto& pp : pipes)
                        for (int wk : {1, 2})
                            for (int splitk : {1, 2, 3, 4}) {
                                memset(&p, 0, sizeof(p));
                                p.kernel = W4A16_KERNEL_TILED;
                                p.bm = bm;
                                p.bn = bn;
                                p.wm = wm;
                                p.wk = wk;
                                p.pf = pp[0];
                                p.xpf = pp[1];
                                p.splitk = splitk;
                                add(p);
                            }
        for (int pf : {1, 2})   // 96 x 64 tiles of three waves
            for (int splitk : {1, 2, 3, 4}) {
                memset(&p, 0, sizeof(p));
                p.kernel = W4A16_KERNEL_TILED;
                p.bm = 96;
                p.bn = 64;
                p.wm = 3;
                p.pf = pf;
                p.splitk = splitk;
                add(p);
            }
    }
    return out;
}

// Residual add + RMS normalization feeding the GEMM (token-major).  The
// normalized activations go into the workspace's chunk region: in the chunk
// layout for the tiled and narrow kernels (which then skip their own
// rewrite), row-major [N, K] for the skinny kernel (which reads x directly).
size_t norm_workspace_bytes(const GemmArgs& a, const w4a16_plan& p) { return chunks_offset(a, p) + xpack_bytes(a); }

int check_eps(float eps) {
    if (!(eps >= 0.f) || eps > 3.0e38f) return fail(W4A16_ERR_INVALID_ARG, "eps must be finite and >= 0");
    return W4A16_OK;
}

// h may be the residual buffer itself (updated in place), never a partial overlap
bool bad_stream_alias(const void* h, const void* r, size_t n) { return h != r && overlaps(h, n, r, n); }

int run_gemm_norm(const uint32_t* qpk, const void* scales, const uint32_t* zpk, const void* x, const void* residual,
                  const void* gamma, float eps, void* h, void* c, int64_t M, int64_t N, int64_t K,
                  int32_t group_size, const w4a16_plan* plan_in, void* workspace, size_t workspace_bytes,
                  void* stream, bool dry = false) {
    int st = check_dims(M, N, K, group_size);
    if (st) return st;
    st = check_eps(eps);
    if (st) return st;
    if (!qpk || !scales || !zpk || !x || !residual || !gamma || !h || !c)
        return fail(W4A16_ERR_INVALID_ARG, "null data pointer");
    if (!aligned16(qpk) || !aligned16(scales) || !aligned16(zpk) || !aligned16(x) || !aligned16(residual) ||
        !aligned16(gamma) || !aligned16(h) || !aligned16(c))
        return fail(W4A16_ERR_MISALIGNED, "every data pointer must be 16-byte aligned");
    const int64_t G = groups_of(K);
    const size_t nq = (size_t)M * (size_t)(K / 8) * 4, ns = (size_t)M * G * 2,
                 nz = (size_t)M * zwords_of(K) * 4, nx = (size_t)K * N * 2, nc = (size_t)M * N * 2,
                 ng = (size_t)K * 2;
    if (overlaps(c, nc, qpk, nq) || overlaps(c, nc, scales, ns) || overlaps(c, nc, zpk, nz) ||
        overlaps(c, nc, x, nx) || overlaps(c, nc, residual, nx) || overlaps(c, nc, gamma, ng) ||
        overlaps(c, nc, h, nx))
        return fail(W4A16_ERR_INVALID_ARG, "output overlaps another buffer");
    if (overlaps(h, nx, x, nx) || overlaps(h, nx, gamma, ng) || overlaps(h, nx, qpk, nq) ||
        overlaps(h, nx, scales, ns) || overlaps(h, nx, zpk, nz) || bad_stream_alias(h, residual, nx))
        return fail(W4A16_ERR_INVALID_ARG, "h overlaps an input (only h == residual is allowed)");

    GemmArgs a = make_args(M, N, K, W4A16_LAYOUT_TOKEN);
    const w4a16_plan p = plan_in ? *plan_in : default_plan(M, N, K, W4A16_LAYOUT_TOKEN);
    st = check_plan(a, p);
    if (st) return st;
    const size_t need = norm_workspace_bytes(a, p);
    if (!workspace || workspace_bytes < need)
        return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4A16_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    if (overlaps(workspace, need, c, nc) || overlaps(workspace, need, qpk, nq) ||
        overlaps(workspace, need, scales, ns) || overlaps(workspace, need, zpk, nz) ||
        overlaps(workspace, need, x, nx) || overlaps(workspace, need, residual, nx) ||
        overlaps(workspace, need, gamma, ng) || overlaps(workspace, need, h, nx))
        return fail(W4A16_ERR_INVALID_ARG, "workspace overlaps a data buffer");
    uint16_t* y = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + chunks_offset(a, p));
    a.counters = static_cast<uint32_t*>(workspace);
    a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    a.qpk = qpk;
    a.scales = static_cast<const uint16_t*>(scales);
    a.zpk = zpk;
    a.c = static_cast<uint16_t*>(c);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // one launch: the skinny kernel normalizes while it stages (every
    // workgroup reads all of x and the residual, so h must not be the
    // residual itself, and one workgroup must cover all of K)
    if (p.kernel == W4A16_KERNEL_SKINNY && p.splitk == 1 && h != residual) {
        GemmArgs an = a;
        an.norm = 1;
        an.eps = eps;
        an.x = static_cast<const uint16_t*>(x);
        an.res = static_cast<const uint16_t*>(residual);
        an.gamma = static_cast<const uint16_t*>(gamma);
        an.hout = static_cast<uint16_t*>(h);
        const char* why = skinny_check(an, skinny_of(p));
        if (!why) {
            if (dry) return ok();
            hipError_t e = launch_skinny(an, skinny_of(p), s);
            if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
            return ok();
        }
    }
    const bool chunks = p.kernel != W4A16_KERNEL_SKINNY;
    if (chunks) {
        a.xp = y;
        a.xp_ready = 1;
        a.x = y;   // unused: the chunks are ready
    } else {
        a.x = y;   // the skinny kernel reads the normalized rows [N, K]
    }
    if (dry) return ok();

    hipError_t e = launch_add_rmsnorm(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(residual),
                                      static_cast<const uint16_t*>(gamma), eps, static_cast<uint16_t*>(h), y, N, K,
                                      chunks, s);
    if (e == hipSuccess)
        e = p.kernel == W4A16_KERNEL_SKINNY   ? launch_skinny(a, skinny_of(p), s)
            : p.kernel == W4A16_KERNEL_NARROW ? launch_narrow(a, narrow_of(p), s)
                                              : launch_tiled(a, tiled_of(p), s);
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Decode attention: the head dimension is fixed at 128 (LLaMA-7B); a split
// along the keys needs the workspace's counters and per-split partials.
constexpr int64_t kAttnHeadDim = 128;

size_t attn_workspace_bytes(const AttnArgs& a, const AttnShape& sh) {
    const int64_t splits = attn_splits(a, sh);
    if (splits <= 1) return 0;
    return kCounterBytes + (size_t)a.B * (size_t)a.H * (size_t)splits * (kAttnHeadDim + 2) * 4;
}

int make_attn(int64_t B, int64_t H, int64_t D, int64_t S, int64_t max_len, float rope_base, float scale,
              AttnArgs& a) {
    if (D != kAttnHeadDim) return fail(W4A16_ERR_UNSUPPORTED, "head dimension must be 128, got %lld", (long long)D);
    if (B < 1 || B > 65535 || H < 1 || H > 65535)
        return fail(W4A16_ERR_INVALID_ARG, "need 1 <= B, H <= 65535 (B=%lld H=%lld)", (long long)B, (long long)H);
    if (S < 1 || max_len < 1 || max_len > S || S >= kMaxDim)
        return fail(W4A16_ERR_INVALID_ARG, "need 1 <= max_len <= S < 2^31 (S=%lld max_len=%lld)", (long long)S,
                    (long long)max_len);
    if ((double)B * (double)H * (double)S * (double)D * 2.0 > 9.0e18)
        return fail(W4A16_ERR_INVALID_ARG, "cache size overflows");
    if (!(rope_base > 0.f) || rope_base > 3.0e38f)
        return fail(W4A16_ERR_INVALID_ARG, "rope_base must be finite and > 0");
    if (!(scale > 0.f) || scale > 3.0e38f) return fail(W4A16_ERR_INVALID_ARG, "scale must be finite and > 0");
    memset(&a, 0, sizeof(a));
    a.B = (int32_t)B;
    a.H = (int32_t)H;
    a.S = S;
    a.max_len = max_len;
    a.theta1 = pow((double)rope_base, -2.0 / (double)D);
    a.scale = scale;
    return W4A16_OK;
}

// A workgroup shape for these arguments: supported, at most kAttnMaxSplits
// splits, and a counter per (sequence, head) when it splits.
int check_attn_shape(const AttnArgs& a, const AttnShape& sh) {
    if (!attn_shape_supported(sh))
        return fail(W4A16_ERR_UNSUPPORTED, "keys per wave must be 16, 32 or 64 and waves 4, 8 or 16 (got %d, %d)",
                    sh.kpw, sh.waves);
    if (attn_splits(a, sh) > kAttnMaxSplits)
        return fail(W4A16_ERR_UNSUPPORTED, "more than %d splits along the keys (max_len %lld)", kAttnMaxSplits,
                    (long long)a.max_len);
    if (attn_splits(a, sh) > 1 && (int64_t)a.B * a.H > kCounterSlots)
        return fail(W4A16_ERR_UNSUPPORTED, "split attention supports at most %lld (sequence, head) pairs",
                    (long long)kCounterSlots);
    return W4A16_OK;
}

AttnShape shape_or_default(const AttnArgs& a, int32_t kpw, int32_t waves) {
    return (kpw == 0 && waves == 0) ? attn_default_shape(a) : AttnShape{kpw, waves};
}

int run_attention(const void* qkv, void* k_cache, void* v_cache, const int32_t* pos, void* out, int64_t B, int64_t H,
                  int64_t D, int64_t S, int64_t max_len, float rope_base, float scale, void* workspace,
                  size_t workspace_bytes, void* stream, bool dry = false, int32_t kpw = 0, int32_t waves = 0) {
    AttnArgs a;
    int st = make_attn(B, H, D, S, max_len, rope_base, scale, a);
    if (st) return st;
    const AttnShape sh = shape_or_default(a, kpw, waves);
    st = check_attn_shape(a, sh);
    if (st) return st;
    if (!qkv || !k_cache || !v_cache || !pos || !out) return fail(W4A16_ERR_INVALID_ARG, "null data pointer");
    if (!aligned16(qkv) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) ||
        (((uintptr_t)pos) & 3))
        return fail(W4A16_ERR_MISALIGNED, "qkv, caches and out must be 16-byte aligned, pos 4-byte aligned");
    const size_t nq = (size_t)B * 3 * H * D * 2, nc = (size_t)B * H * S * D * 2, no = (size_t)B * H * D * 2,
                 np = (size_t)B * 4;
    if (overlaps(out, no, qkv, nq) || overlaps(out, no, k_cache, nc) || overlaps(out, no, v_cache, nc) ||
        overlaps(out, no, pos, np))
        return fail(W4A16_ERR_INVALID_ARG, "out overlaps another buffer");
    if (overlaps(k_cache, nc, v_cache, nc) || overlaps(k_cache, nc, qkv, nq) || overlaps(v_cache, nc, qkv, nq) ||
        overlaps(k_cache, nc, pos, np) || overlaps(v_cache, nc, pos, np))
        return fail(W4A16_ERR_INVALID_ARG, "a cache overlaps another buffer");
    const size_t need = attn_workspace_bytes(a, sh);
    if (need > 0) {
        if (!workspace || workspace_bytes < need)
            return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                        workspace ? workspace_bytes : (size_t)0);
        if (!aligned16(workspace)) return fail(W4A16_ERR_MISALIGNED, "workspace must be 16-byte aligned");
        if (overlaps(workspace, need, qkv, nq) || overlaps(workspace, need, k_cache, nc) ||
            overlaps(workspace, need, v_cache, nc) || overlaps(workspace, need, out, no) ||
            overlaps(workspace, need, pos, np))
            return fail(W4A16_ERR_INVALID_ARG, "workspace overlaps a data buffer");
        a.counters = static_cast<uint32_t*>(workspace);
        a.part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kCounterBytes);
    }
    a.qkv = static_cast<const uint16_t*>(qkv);
    a.k_cache = static_cast<uint16_t*>(k_cache);
    a.v_cache = static_cast<uint16_t*>(v_cache);
    a.pos = pos;
    a.out = static_cast<uint16_t*>(out);
    if (dry) return ok();
    hipError_t e = launch_decode_attn(a, sh, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}


int run_silu_mul(const void* gu, void* act, int64_t N, int64_t I, void* stream, bool dry = false) {
    if (N < 1 || N >= kMaxDim || I < 8 || I % 8 || I >= kMaxDim / 2)
        return fail(W4A16_ERR_INVALID_ARG, "need N >= 1, I >= 8, I %% 8 == 0 (N=%lld I=%lld)", (long long)N,
                    (long long)I);
    if (!gu || !act) return fail(W4A16_ERR_INVALID_ARG, "null data pointer");
    if (!aligned16(gu) || !aligned16(act)) return fail(W4A16_ERR_MISALIGNED, "gu and act must be 16-byte aligned");
    if (overlaps(gu, (size_t)N * I * 4, act, (size_t)N * I * 2))
        return fail(W4A16_ERR_INVALID_ARG, "act overlaps gu");
    if (dry) return ok();
    hipError_t e = launch_silu_mul(static_cast<const uint16_t*>(gu), static_cast<uint16_t*>(act), N, I,
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

// Decoder layer workspace: [shared region: the largest workspace any step
// needs, steps run one after another][qkv][attention output][gate/up][the
// stream after the attention's residual add], each at a 256-byte boundary.
// The down projection forms silu(gate) * up itself.
struct LayerLayout {
    size_t shared, qkv, attn, gu, h, total;
};

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

int layer_layout(int64_t B, int64_t H, int64_t D, int64_t I, int64_t S, int64_t max_len, LayerLayout& L) {
    AttnArgs aa;
    int st = make_attn(B, H, D, S, max_len, 10000.f, 1.f, aa);
    if (st) return st;
    if (I < 128 || I % 128 || I >= kMaxDim / 2)
        return fail(W4A16_ERR_INVALID_ARG, "I must be a positive multiple of 128, got %lld", (long long)I);
    const int64_t HD = H * D;
    st = check_dims(3 * HD, B, HD, kGroupSize);
    if (!st) st = check_dims(2 * I, B, HD, kGroupSize);
    if (!st) st = check_dims(HD, B, I, kGroupSize);
    if (st) return st;
    st = check_attn_shape(aa, attn_default_shape(aa));
    if (st) return st;
    size_t shared = attn_workspace_bytes(aa, attn_default_shape(aa));
    auto grow = [&](size_t v) { shared = v > shared ? v : shared; };
    {
        const GemmArgs a = make_args(3 * HD, B, HD, W4A16_LAYOUT_TOKEN);
        grow(norm_workspace_bytes(a, default_plan(3 * HD, B, HD, W4A16_LAYOUT_TOKEN)));
    }
    {
        const GemmArgs a = make_args(HD, B, HD, W4A16_LAYOUT_TOKEN);
        grow(workspace_bytes_for(a, default_plan(HD, B, HD, W4A16_LAYOUT_TOKEN)));
    }
    {
        const GemmArgs a = make_args(2 * I, B, HD, W4A16_LAYOUT_TOKEN);
        grow(norm_workspace_bytes(a, default_plan(2 * I, B, HD, W4A16_LAYOUT_TOKEN)));
    }
    {
        const GemmArgs a = make_args(HD, B, I, W4A16_LAYOUT_TOKEN);
        grow(workspace_bytes_for(a, default_plan(HD, B, I, W4A16_LAYOUT_TOKEN)));
    }
    grow(kCounterBytes);
    L.shared = round256(shared);
    L.qkv = L.shared;
    L.attn = L.qkv + round256((size_t)B * 3 * HD * 2);
    L.gu = L.attn + round256((size_t)B * HD * 2);
    L.h = L.gu + round256((size_t)B * 2 * I * 2);
    L.total = L.h + round256((size_t)B * HD * 2);
    return W4A16_OK;
}

int run_decode_layer(const w4a16_decoder_layer* ly, int64_t B, int64_t H, int64_t D, int64_t I, int64_t S,
                     int64_t max_len, const int32_t* pos, float eps, float rope_base, void* residual, void* x,
                     void* workspace, size_t workspace_bytes, void* stream) {
    if (!ly) return fail(W4A16_ERR_INVALID_ARG, "layer is NULL");
    LayerLayout L;
    int st = layer_layout(B, H, D, I, S, max_len, L);
    if (st) return st;
    if (!workspace || workspace_bytes < L.total)
        return fail(W4A16_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(W4A16_ERR_MISALIGNED, "workspace must be 16-byte aligned");
    if (!residual || !x) return fail(W4A16_ERR_INVALID_ARG, "null data pointer");
    const size_t nh = (size_t)B * H * D * 2;
    if (overlaps(residual, nh, x, nh)) return fail(W4A16_ERR_INVALID_ARG, "residual overlaps x");
    if (overlaps(workspace, L.total, residual, nh) || overlaps(workspace, L.total, x, nh))
        return fail(W4A16_ERR_INVALID_ARG, "workspace overlaps residual or x");
    char* w = static_cast<char*>(workspace);
    void* shared = w;
    void* qkv = w + L.qkv;
    void* attn = w + L.attn;
    void* gu = w + L.gu;
    void* hbuf = w + L.h;
    const int64_t HD = H * D;
    const float scale = (float)(1.0 / sqrt((double)D));
    // every step checked first (dry), then enqueued
    for (int pass = 0; pass < 2; ++pass) {
        const bool dry = pass == 0;
        // the stream goes residual -> hbuf -> residual, so that no
        // normalizing step writes the buffer it reads (the skinny kernel's
        // one-launch prologue needs that)
        st = run_gemm_norm(ly->qkv.q_packed, ly->qkv.scales, ly->qkv.z_packed, x, residual, ly->attn_norm, eps,
                           hbuf, qkv, 3 * HD, B, HD, kGroupSize, nullptr, shared, L.shared, stream, dry);
        if (!st)
            st = run_attention(qkv, ly->k_cache, ly->v_cache, pos, attn, B, H, D, S, max_len, rope_base, scale,
                               shared, L.shared, stream, dry);
        if (!st)
            st = run_gemm(ly->o.q_packed, ly->o.scales, ly->o.z_packed, attn, x, HD, B, HD, kGroupSize,
                          W4A16_LAYOUT_TOKEN, nullptr, shared, L.shared, stream, dry);
        if (!st)
            st = run_gemm_norm(ly->gate_up.q_packed, ly->gate_up.scales, ly->gate_up.z_packed, x, hbuf,
                               ly->mlp_norm, eps, residual, gu, 2 * I, B, HD, kGroupSize, nullptr, shared, L.shared,
                               stream, dry);
        if (!st)
            st = run_gemm(ly->down.q_packed, ly->down.scales, ly->down.z_packed, gu, x, HD, B, I, kGroupSize,
                          W4A16_LAYOUT_TOKEN, nullptr, shared, L.shared, stream, dry, 1);
        if (st) return st;
    }
    return ok();
}

}  // namespace

namespace w4a16 {
int set_last_error(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}
}  // namespace w4a16

extern "C" {

const char* w4a16_status_string(int status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_INVALID_ARG: return "invalid argument";
        case W4A16_ERR_UNSUPPORTED: return "unsupported";
        case W4A16_ERR_MISALIGNED: return "misaligned pointer";
        case W4A16_ERR_WORKSPACE: return "workspace missing or too small";
        case W4A16_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

const char* w4a16_last_error(void) { return g_err.c_str(); }

int w4a16_version(void) { return 101; }

int w4a16_pack(const uint8_t* q, const uint8_t* z, int64_t M, int64_t K, int32_t group_size,
               uint32_t* q_packed, uint32_t* z_packed, void* stream) {
    int st = check_dims(M, 1, K, group_size);
    if (st) return st;
    if (!q && !z) return fail(W4A16_ERR_INVALID_ARG, "nothing to pack: q and z are both NULL");
    if ((q && !q_packed) || (z && !z_packed))
        return fail(W4A16_ERR_INVALID_ARG, "a code array is given without its packed output");
    if ((q && !aligned16(q)) || (z && !aligned16(z)) || (q_packed && !aligned16(q_packed)) ||
        (z_packed && !aligned16(z_packed)))
        return fail(W4A16_ERR_MISALIGNED, "every pointer must be 16-byte aligned");
    const int64_t G = groups_of(K);
    const size_t nq = (size_t)M * K, nqp = (size_t)M * (K / 8) * 4, nzc = (size_t)M * G,
                 nzp = (size_t)M * zwords_of(K) * 4;
    if (q && (overlaps(q_packed, nqp, q, nq) || (z && overlaps(q_packed, nqp, z, nzc)) ||
              (z && overlaps(q_packed, nqp, z_packed, nzp))))
        return fail(W4A16_ERR_INVALID_ARG, "packed weights overlap another buffer");
    if (z && (overlaps(z_packed, nzp, z, nzc) || (q && overlaps(z_packed, nzp, q, nq))))
        return fail(W4A16_ERR_INVALID_ARG, "packed zeros overlap another buffer");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (q) {
        hipError_t e = launch_pack_rows(q, q_packed, M, K, s);
        if (e != hipSuccess) return fail(W4A16_ERR_HIP, "pack launch failed: %s", hipGetErrorString(e));
    }
    if (z) {
        hipError_t e = launch_pack_rows(z, z_packed, M, G, s);
        if (e != hipSuccess) return fail(W4A16_ERR_HIP, "pack launch failed: %s", hipGetErrorString(e));
    }
    return ok();
}

int64_t w4a16_stream_read_sink_words(int64_t bytes, int32_t waves, int32_t loads) {
    const bool pow2 = waves >= 1 && waves <= 16 && !(waves & (waves - 1)) && loads >= 1 && loads <= 16 &&
                      !(loads & (loads - 1));
    if (bytes < 16 || bytes % 16 || !pow2) return 0;
    const int64_t nw = stream_read_waves(bytes, loads);
    return (nw + waves - 1) / waves * waves;
}

int w4a16_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t waves, int32_t loads, void* stream) {
    if (!buf || !sink) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (bytes < 16 || bytes % 16 || bytes > ((int64_t)1 << 40))
        return fail(W4A16_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 (got %lld)", (long long)bytes);
    if (waves != 1 && waves != 2 && waves != 4 && waves != 8 && waves != 16)
        return fail(W4A16_ERR_INVALID_ARG, "waves must be 1, 2, 4, 8 or 16 (got %d)", (int)waves);
    if (loads != 1 && loads != 2 && loads != 4 && loads != 8 && loads != 16)
        return fail(W4A16_ERR_INVALID_ARG, "loads must be 1, 2, 4, 8 or 16 (got %d)", (int)loads);
    if (!aligned16(buf) || !aligned16(sink)) return fail(W4A16_ERR_MISALIGNED, "pointers must be 16-byte aligned");
    const int64_t words = w4a16_stream_read_sink_words(bytes, waves, loads);
    if (overlaps(sink, (size_t)words * 4, buf, (size_t)bytes))
        return fail(W4A16_ERR_INVALID_ARG, "sink overlaps the buffer");
    const hipError_t e = launch_stream_read(buf, bytes, sink, waves, loads, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "stream read launch failed: %s", hipGetErrorString(e));
    return ok();
}

int w4a16_quantize(const void* w, int64_t M, int64_t K, int32_t group_size, uint32_t* q_packed, void* scales,
                   uint32_t* z_packed, void* stream) {
    int st = check_dims(M, 1, K, group_size);
    if (st) return st;
    if (!w || !q_packed || !scales || !z_packed) return fail(W4A16_ERR_INVALID_ARG, "null pointer");
    if (!aligned16(w) || !aligned16(q_packed) || !aligned16(scales) || !aligned16(z_packed))
        return fail(W4A16_ERR_MISALIGNED, "every pointer must be 16-byte aligned");
    const int64_t G = groups_of(K);
    const size_t nw = (size_t)M * K * 2, nq = (size_t)M * (K / 8) * 4, ns = (size_t)M * G * 2,
                 nz = (size_t)M * zwords_of(K) * 4;
    if (overlaps(q_packed, nq, w, nw) || overlaps(scales, ns, w, nw) || overlaps(z_packed, nz, w, nw) ||
        overlaps(q_packed, nq, scales, ns) || overlaps(q_packed, nq, z_packed, nz) ||
        overlaps(scales, ns, z_packed, nz))
        return fail(W4A16_ERR_INVALID_ARG, "the outputs overlap each other or the input");
    hipError_t e = launch_quantize(static_cast<const uint16_t*>(w), q_packed, static_cast<uint16_t*>(scales),
                                   z_packed, M, K, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "quantize launch failed: %s", hipGetErrorString(e));
    return ok();
}

int w4a16_plan_default(int64_t M, int64_t N, int64_t K, int32_t group_size, w4a16_plan* plan) {
    int st = check_dims(M, N, K, group_size);
    if (st) return st;
    if (!plan) return fail(W4A16_ERR_INVALID_ARG, "plan is NULL");
    *plan = default_plan(M, N, K);
    return ok();
}

size_t w4a16_workspace_size_plan(int64_t M, int64_t N, int64_t K, int32_t group_size,
                                 const w4a16_plan* plan) {
    if (check_dims(M, N, K, group_size) || !plan) return 0;
    GemmArgs a = make_args(M, N, K);
    if (check_plan(a, *plan)) return 0;
    return workspace_bytes_for(a, *plan);
}

size_t w4a16_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size) {
    if (check_dims(M, N, K, group_size)) return 0;
    GemmArgs a = make_args(M, N, K);
    return workspace_bytes_for(a, default_plan(M, N, K));
}

int w4a16_kernel_name(int64_t M, int64_t N, int64_t K, int32_t group_size, const w4a16_plan* plan, char* buf,
                      size_t len) {
    int st = check_dims(M, N, K, group_size);
    if (st) return st;
    if (!buf || len == 0) return fail(W4A16_ERR_INVALID_ARG, "null or empty name buffer");
    GemmArgs a = make_args(M, N, K);
    const w4a16_plan p = plan ? *plan : default_plan(M, N, K);
    st = check_plan(a, p);
    if (st) return st;
    if (p.kernel == W4A16_KERNEL_SKINNY)
        snprintf(buf, len, "skinny_kernel<%d, %d>", p.ncol, skinny_pf(a, skinny_of(p)));
    else if (p.kernel == W4A16_KERNEL_NARROW)
        snprintf(buf, len, "narrow_kernel<%d, %d, %d, %d, %d, %s>", p.ncol / 16, p.pf, narrow_of(p).rb,
                 narrow_of(p).wk, narrow_of(p).wm, narrow_direct_x(a) ? "true" : "false");
    else
    {
        const TiledShape t = tiled_of(p);
        const bool dx = tiled_direct_x(a, t);
        snprintf(buf, len, "%s<%d, %d, %d, %d, %d, %d>",
                 t.wk == 2 ? (dx ? "tiled_k2_dx_kernel" : "tiled_k2_kernel") : (dx ? "tiled_dx_kernel" : "tiled_kernel"),
                 t.bm, t.bn, t.wm, t.wm == 8 ? 8 : t.wm == 3 ? 3 : 4, t.wpf, t.xpf);
    }
    return ok();
}

int w4a16_gemv(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed, const void* x,
               void* c, int64_t M, int64_t K, int32_t group_size, void* stream) {
    int st = check_dims(M, 1, K, group_size);
    if (st) return st;
    w4a16_plan p = default_plan(M, 1, K);
    GemmArgs a = make_args(M, 1, K);
    if (workspace_bytes_for(a, p) != 0)
        return fail(W4A16_ERR_UNSUPPORTED, "K=%lld needs a split reduction; use w4a16_gemm", (long long)K);
    return run_gemm(q_packed, scales, z_packed, x, c, M, 1, K, group_size, W4A16_LAYOUT_KN, &p, nullptr, 0,
                    stream);
}

int w4a16_gemm(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed, const void* x,
               void* c, int64_t M, int64_t N, int64_t K, int32_t group_size, void* workspace,
               size_t workspace_bytes, void* stream) {
    return run_gemm(q_packed, scales, z_packed, x, c, M, N, K, group_size, W4A16_LAYOUT_KN, nullptr, workspace,
                    workspace_bytes, stream);
}

int w4a16_gemm_plan(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed,
                    const void* x, void* c, int64_t M, int64_t N, int64_t K, int32_t group_size,
                    const w4a16_plan* plan, void* workspace, size_t workspace_bytes, void* stream) {
    if (!plan) return fail(W4A16_ERR_INVALID_ARG, "plan is NULL");
    return run_gemm(q_packed, scales, z_packed, x, c, M, N, K, group_size, W4A16_LAYOUT_KN, plan, workspace,
                    workspace_bytes, stream);
}

int w4a16_gemm_ex(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed, const void* x, void* c,
                  int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t layout, const w4a16_plan* plan,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return run_gemm(q_packed, scales, z_packed, x, c, M, N, K, group_size, layout, plan, workspace,
                    workspace_bytes, stream);
}

int w4a16_plan_default_ex(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t layout, w4a16_plan* plan) {
    int st = check_dims(M, N, K, group_size);
    if (st) return st;
    st = check_layout(layout);
    if (st) return st;
    if (!plan) return fail(W4A16_ERR_INVALID_ARG, "plan is NULL");
    *plan = default_plan(M, N, K, layout);
    return ok();
}

size_t w4a16_workspace_size_ex(int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t layout,
                               const w4a16_plan* plan) {
    if (check_dims(M, N, K, group_size) || check_layout(layout)) return 0;
    GemmArgs a = make_args(M, N, K, layout);
    const w4a16_plan p = plan ? *plan : default_plan(M, N, K, layout);
    if (check_plan(a, p)) return 0;
    return workspace_bytes_for(a, p);
}

int w4a16_add_rmsnorm(const void* x, const void* residual, const void* gamma, float eps, void* h, void* y,
                      int64_t N, int64_t K, void* stream) {
    if (N < 1 || N >= kMaxDim || K < 8 || K >= kMaxDim || K % 8)
        return fail(W4A16_ERR_INVALID_ARG, "need N >= 1, K >= 8, K %% 8 == 0, both below 2^31 (N=%lld K=%lld)",
                    (long long)N, (long long)K);
    int st = check_eps(eps);
    if (st) return st;
    if (!x || !residual || !gamma || !h || !y) return fail(W4A16_ERR_INVALID_ARG, "null data pointer");
    if (!aligned16(x) || !aligned16(residual) || !aligned16(gamma) || !aligned16(h) || !aligned16(y))
        return fail(W4A16_ERR_MISALIGNED, "every data pointer must be 16-byte aligned");
    const size_t nx = (size_t)N * (size_t)K * 2, ng = (size_t)K * 2;
    if (overlaps(y, nx, x, nx) || overlaps(y, nx, residual, nx) || overlaps(y, nx, gamma, ng) ||
        overlaps(y, nx, h, nx))
        return fail(W4A16_ERR_INVALID_ARG, "y overlaps another buffer");
    if (overlaps(h, nx, x, nx) || overlaps(h, nx, gamma, ng) || bad_stream_alias(h, residual, nx))
        return fail(W4A16_ERR_INVALID_ARG, "h overlaps an input (only h == residual is allowed)");
    hipError_t e = launch_add_rmsnorm(static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(residual),
                                      static_cast<const uint16_t*>(gamma), eps, static_cast<uint16_t*>(h),
                                      static_cast<uint16_t*>(y), N, K, false, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(W4A16_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

size_t w4a16_gemm_add_rmsnorm_workspace_size(int64_t M, int64_t N, int64_t K, int32_t group_size,
                                             const w4a16_plan* plan) {
    if (check_dims(M, N, K, group_size)) return 0;
    GemmArgs a = make_args(M, N, K, W4A16_LAYOUT_TOKEN);
    const w4a16_plan p = plan ? *plan : default_plan(M, N, K, W4A16_LAYOUT_TOKEN);
    if (check_plan(a, p)) return 0;
    return norm_workspace_bytes(a, p);
}

int w4a16_gemm_add_rmsnorm(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed, const void* x,
                           const void* residual, const void* gamma, float eps, void* h, void* c, int64_t M,
                           int64_t N, int64_t K, int32_t group_size, const w4a16_plan* plan, void* workspace,
                           size_t workspace_bytes, void* stream) {
    return run_gemm_norm(q_packed, scales, z_packed, x, residual, gamma, eps, h, c, M, N, K, group_size, plan,
                         workspace, workspace_bytes, stream);
}

size_t w4a16_decode_attention_workspace_size_plan(int64_t B, int64_t H, int64_t D, int64_t S, int64_t max_len,
                                                  int32_t keys_per_wave, int32_t waves) {
    AttnArgs a;
    const std::string saved = g_err;
    int st = make_attn(B, H, D, S, max_len, 10000.f, 1.f, a);
    const AttnShape sh = shape_or_default(a, keys_per_wave, waves);
    if (!st) st = check_attn_shape(a, sh);
    g_err = saved;
    return st ? 0 : attn_workspace_bytes(a, sh);
}

size_t w4a16_decode_attention_workspace_size(int64_t B, int64_t H, int64_t D, int64_t S, int64_t max_len) {
    return w4a16_decode_attention_workspace_size_plan(B, H, D, S, max_len, 0, 0);
}

int w4a16_decode_attention_plan(const void* qkv, void* k_cache, void* v_cache, const int32_t* pos, void* out,
                                int64_t B, int64_t H, int64_t D, int64_t S, int64_t max_len, float rope_base,
                                float scale, int32_t keys_per_wave, int32_t waves, void* workspace,
                                size_t workspace_bytes, void* stream) {
    return run_attention(qkv, k_cache, v_cache, pos, out, B, H, D, S, max_len, rope_base, scale, workspace,
                         workspace_bytes, stream, false, keys_per_wave, waves);
}

int w4a16_decode_attention(const void* qkv, void* k_cache, void* v_cache, const int32_t* pos, void* out, int64_t B,
                           int64_t H, int64_t D, int64_t S, int64_t max_len, float rope_base, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
    return run_attention(qkv, k_cache, v_cache, pos, out, B, H, D, S, max_len, rope_base, scale, workspace,
                         workspace_bytes, stream);
}

int w4a16_silu_mul(const void* gu, void* act, int64_t N, int64_t I, void* stream) {
    return run_silu_mul(gu, act, N, I, stream);
}

size_t w4a16_decode_layer_workspace_size(int64_t B, int64_t H, int64_t D, int64_t I, int64_t S, int64_t max_len) {
    LayerLayout L;
    const std::string saved = g_err;
    const int st = layer_layout(B, H, D, I, S, max_len, L);
    g_err = saved;
    return st ? 0 : L.total;
}

int w4a16_decode_layer(const w4a16_decoder_layer* layer, int64_t B, int64_t H, int64_t D, int64_t I, int64_t S,
                       int64_t max_len, const int32_t* pos, float eps, float rope_base, void* residual, void* x,
                       void* workspace, size_t workspace_bytes, void* stream) {
    return run_decode_layer(layer, B, H, D, I, S, max_len, pos, eps, rope_base, residual, x, workspace,
                            workspace_bytes, stream);
}

int w4a16_tune(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed, const void* x, void* c,
               int64_t M, int64_t N, int64_t K, int32_t group_size, int32_t layout, void* workspace,
               size_t workspace_bytes, void* flush, size_t flush_bytes, int32_t iters, w4a16_plan* best,
               float* best_us, int32_t* n_tried, void* stream) {
    int st = check_dims(M, N, K, group_size);
    if (st) return st;
    st = check_layout(layout);
    if (st) return st;
    if (!best) return fail(W4A16_ERR_INVALID_ARG, "best is NULL");
    if (iters < 1 || iters > 100000) return fail(W4A16_ERR_INVALID_ARG, "iters must be in 1..100000");
    if (flush && (flush_bytes == 0 || !aligned16(flush)))
        return fail(W4A16_ERR_INVALID_ARG, "flush buffer must be 16-byte aligned and non-empty");
    const GemmArgs a = make_args(M, N, K, layout);
    const std::vector<w4a16_plan> cands = candidate_plans(a);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipEvent_t ev[2];
    if (hipEventCreate(&ev[0]) != hipSuccess) return fail(W4A16_ERR_HIP, "hipEventCreate failed");
    if (hipEventCreate(&ev[1]) != hipSuccess) {
        hipEventDestroy(ev[0]);
        return fail(W4A16_ERR_HIP, "hipEventCreate failed");
    }
    float best_t = 0.f;
    int tried = 0;
    w4a16_plan winner;
    memset(&winner, 0, sizeof(winner));
    int status = W4A16_OK;
    for (const w4a16_plan& p : cands) {
        if (workspace_bytes_for(a, p) > (workspace ? workspace_bytes : 0)) continue;
        // one untimed call (also validates every argument)
        status = run_gemm(q_packed, scales, z_packed, x, c, M, N, K, group_size, layout, &p, workspace,
                          workspace_bytes, stream);
        if (status) break;
        float total = 0.f;
        for (int i = 0; i < iters && !status; ++i) {
            if (flush && hipMemsetAsync(flush, i & 0xFF, flush_bytes, s) != hipSuccess)
                status = fail(W4A16_ERR_HIP, "flush failed");
            if (!status && hipEventRecord(ev[0], s) != hipSuccess) status = fail(W4A16_ERR_HIP, "event record failed");
            if (!status)
                status = run_gemm(q_packed, scales, z_packed, x, c, M, N, K, group_size, layout, &p, workspace,
                                  workspace_bytes, stream);
            if (!status && hipEventRecord(ev[1], s) != hipSuccess) status = fail(W4A16_ERR_HIP, "event record failed");
            float ms = 0.f;
            if (!status && (hipEventSynchronize(ev[1]) != hipSuccess || hipEventElapsedTime(&ms, ev[0], ev[1]) != hipSuccess))
                status = fail(W4A16_ERR_HIP, "event timing failed");
            total += ms;
        }
        if (status) break;
        const float us = total * 1e3f / (float)iters;
        if (tried == 0 || us < best_t) {
            best_t = us;
            winner = p;
        }
        ++tried;
    }
    hipEventDestroy(ev[0]);
    hipEventDestroy(ev[1]);
    if (status) return status;
    if (tried == 0) return fail(W4A16_ERR_WORKSPACE, "no candidate plan fits the %zu-byte workspace", workspace_bytes);
    *best = winner;
    if (best_us) *best_us = best_t;
    if (n_tried) *n_tried = tried;
    return ok();
}

int w4a16_gemm_silu(const uint32_t* q_packed, const void* scales, const uint32_t* z_packed, const void* gu, void* c,
                    int64_t M, int64_t N, int64_t K, int32_t group_size, const w4a16_plan* plan, void* workspace,
                    size_t workspace_bytes, void* stream) {
    return run_gemm(q_packed, scales, z_packed, gu, c, M, N, K, group_size, W4A16_LAYOUT_TOKEN, plan, workspace,
                    workspace_bytes, stream, false, 1);
}

}  // extern "C"
