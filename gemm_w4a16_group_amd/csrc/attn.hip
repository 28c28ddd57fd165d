// Fused decode attention: one step of multi-head attention per sequence,
// with the rotary encoding of q and k, QK^T, the softmax and PV in one
// kernel (the third fusion of §3.2 of the PerfXLLM page; the rotary
// encoding read as LLaMA's: channel pairs (2i, 2i + 1) of a head turned by
// pos * base^(-2i / D)).
//
// Layouts (fp16 unless stated):
//   qkv      [B, 3 H D]     the new token of each sequence, q | k | v
//   k_cache  [B, H, S, D]   positions 0 .. p - 1 hold earlier keys (rotated)
//   v_cache  [B, H, S, D]
//   pos      int32 [B]      position p of the new token
//   out      [B, H D]
// The step stores fp16(rope(k, p)) and fp16(v) at position p and attends
// over keys 0 .. p.  D = 128.
//
// HBM-bound on the cache: 2 * 2 D bytes per key.  Grid (H, B, splits): a
// workgroup of four waves takes 4 * KPW consecutive keys of one head (flash-
// decoding split along the keys, so that one sequence fills the chip); each
// wave KPW keys in rounds of 8: lane (key slot lane / 8, channel block
// lane % 8) owns 16 channels of one key.  A wave issues all of its K and V
// loads (16 bytes per lane per load, each key's 256 bytes read by 8 adjacent
// lanes) before any arithmetic, then rotates q while they are in flight.
// Scores: 16 fp32 FMAs per lane and a 3-step butterfly over the channel
// blocks.  Softmax with the wave's maximum; values weighted in fp32; partial
// sums reduced over key slots (butterfly), then over the four waves in LDS.
// With several splits, each one that holds keys up to p writes (max, sum,
// o[D]) with agent-coherent stores and the last of them to arrive (an
// arrival counter in the workspace, compared with the number of such
// splits) merges them in split order, with all of the merge's loads in
// flight at once; workgroups past p leave without taking part, so a graph
// captured for a large max_len pays little for the unused part of it.  The
// split is the slowest grid dimension: workgroups are dispatched in grid
// order, so every sequence's early (live) splits go out before the late
// ones that short sequences leave empty.  With the split fastest, those
// empty workgroups sat between live ones holding CU slots while their one
// load (the position) waited behind the live ones' cache stream: eight
// 361-key sequences took 44.5 us with max_len = 2022 against 16.5 us with
// max_len = 361.
//
// Angles: theta_i = theta_1^i from theta_1 = base^(-2/D) (double, from the
// host), p * theta_i in double, reduced modulo 2 pi in double (two-part
// constant), then sine and cosine in float32: the rotation is float32-exact
// to about 1e-7 of the pair's norm at any position.
#include <math.h>

#include "device.hpp"
#include "launch.hpp"

namespace w4a16 {

namespace {

constexpr int kHeadDim = 128;
constexpr double kTwoPiHi = 6.283185307179586;
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189535;

__device__ __forceinline__ float h2f_lo(uint32_t w) { return (float)as_h2(w)[0]; }
__device__ __forceinline__ float h2f_hi(uint32_t w) { return (float)as_h2(w)[1]; }
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ uint32_t word_of(const u32x4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int KPW, int W>
__global__ void __launch_bounds__(64 * W) decode_attn_kernel(AttnArgs a) {
    constexpr int R = KPW / 8;   // rounds of 8 keys per wave
    constexpr int D = kHeadDim;
    constexpr int NT = 64 * W;
    const int h = blockIdx.x, b = blockIdx.y, split = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int part = lane & 7, kslot = lane >> 3;
    const int H = a.H;
    const int64_t S = a.S;
    const int p = a.pos[b];
    const bool valid = p >= 0 && (int64_t)p < a.max_len;
    const int64_t slab = ((int64_t)b * H + h) * S * D;
    const int64_t wg0 = (int64_t)split * W * KPW;
    const int64_t j0 = wg0 + (int64_t)wave * KPW;
    // a workgroup whose keys all lie past p has nothing to read
    const bool live = valid && wg0 <= (int64_t)p;

    __shared__ float so[W][D];
    __shared__ float sm[W], sl[W];
    __shared__ int last_flag;
    float M = -INFINITY, L = 0.f, O = 0.f;   // this workgroup's (max, sum, o[tid])

    if (live) {
        // ---- 1. every K and V load of the wave; rows past p read row p
        // (cached, masked below)
        u32x4 kr[R][2], vr[R][2];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t j = j0 + 8 * r + kslot;
            j = j < (int64_t)p ? j : (int64_t)p;
            const u32x4* kp = reinterpret_cast<const u32x4*>(a.k_cache + slab + j * D + 16 * part);
            kr[r][0] = kp[0];
            kr[r][1] = kp[1];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int64_t j = j0 + 8 * r + kslot;
            j = j < (int64_t)p ? j : (int64_t)p;
            const u32x4* vp = reinterpret_cast<const u32x4*>(a.v_cache + slab + j * D + 16 * part);
            vr[r][0] = vp[0];
            vr[r][1] = vp[1];
        }
        const uint16_t* row = a.qkv + (int64_t)b * 3 * H * D + (int64_t)h * D + 16 * part;
        const u32x4 q0 = reinterpret_cast<const u32x4*>(row)[0], q1 = reinterpret_cast<const u32x4*>(row)[1];
        const u32x4 k0 = reinterpret_cast<const u32x4*>(row + H * D)[0],
                    k1 = reinterpret_cast<const u32x4*>(row + H * D)[1];
        const u32x4 v0 = reinterpret_cast<const u32x4*>(row + 2 * H * D)[0],
                    v1 = reinterpret_cast<const u32x4*>(row + 2 * H * D)[1];

        // ---- 2. rotation of this lane's 8 channel pairs (pairs 8 part .. + 7)
        float qf[16];
        uint32_t kn[8];   // the new key, rotated, as stored (fp16 pairs)
        {
            const double pd = (double)p;
            double th = 1.0, pw = a.theta1;
            for (int e = 8 * part; e; e >>= 1) {   // theta_1^(8 part)
                if (e & 1) th *= pw;
                pw *= pw;
            }
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const double ang = pd * th;
                const double kq = rint(ang * kInvTwoPi);
                double rr = fma(-kq, kTwoPiHi, ang);
                rr = fma(-kq, kTwoPiLo, rr);
                float sn, cs;
                sincosf((float)rr, &sn, &cs);
                const uint32_t qw = word_of(t < 4 ? q0 : q1, t & 3), kw = word_of(t < 4 ? k0 : k1, t & 3);
                const float x0 = h2f_lo(qw), x1 = h2f_hi(qw);
                qf[2 * t] = (x0 * cs - x1 * sn) * a.scale;
                qf[2 * t + 1] = (x0 * sn + x1 * cs) * a.scale;
                const float y0 = h2f_lo(kw), y1 = h2f_hi(kw);
                kn[t] = pack_h2(y0 * cs - y1 * sn, y0 * sn + y1 * cs);
                th *= a.theta1;
            }
        }

        // ---- 3. scores (the new key replaces cache row p)
        float sc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t j = j0 + 8 * r + kslot;
            const bool is_new = j == (int64_t)p;
            float d = 0.f;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t w = is_new ? kn[t] : word_of(t < 4 ? kr[r][0] : kr[r][1], t & 3);
                d = fmaf(qf[2 * t], h2f_lo(w), d);
                d = fmaf(qf[2 * t + 1], h2f_hi(w), d);
            }
            d += __shfl_xor(d, 1);
            d += __shfl_xor(d, 2);
            d += __shfl_xor(d, 4);
            sc[r] = j <= (int64_t)p ? d : -INFINITY;
        }
        float m = sc[0];
#pragma unroll
        for (int r = 1; r < R; ++r) m = fmaxf(m, sc[r]);
        m = fmaxf(m, __shfl_xor(m, 8));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));

        // ---- 4. weighted values
        float l = 0.f, o[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) o[i] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int64_t j = j0 + 8 * r + kslot;
            const bool is_new = j == (int64_t)p;
            const float w = sc[r] == -INFINITY ? 0.f : __expf(sc[r] - m);
            l += w;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const uint32_t vw =
                    is_new ? word_of(t < 4 ? v0 : v1, t & 3) : word_of(t < 4 ? vr[r][0] : vr[r][1], t & 3);
                o[2 * t] = fmaf(w, h2f_lo(vw), o[2 * t]);
                o[2 * t + 1] = fmaf(w, h2f_hi(vw), o[2 * t + 1]);
            }
        }
        // over the eight key slots (lanes of equal part)
#pragma unroll
        for (int mk = 8; mk <= 32; mk <<= 1) {
            l += __shfl_xor(l, mk);
#pragma unroll
            for (int i = 0; i < 16; ++i) o[i] += __shfl_xor(o[i], mk);
        }

        // ---- 5. the new token's key and value go into the cache (the eight
        // lanes of one key slot of one wave)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (j0 + 8 * r + kslot == (int64_t)p) {
                u32x4* kd = reinterpret_cast<u32x4*>(a.k_cache + slab + (int64_t)p * D + 16 * part);
                u32x4* vd = reinterpret_cast<u32x4*>(a.v_cache + slab + (int64_t)p * D + 16 * part);
                kd[0] = u32x4{kn[0], kn[1], kn[2], kn[3]};
                kd[1] = u32x4{kn[4], kn[5], kn[6], kn[7]};
                vd[0] = v0;
                vd[1] = v1;
            }
        }

        // ---- 6. the four waves meet in LDS
        if (kslot == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) so[wave][16 * part + i] = o[i];
        }
        if (lane == 0) {
            sm[wave] = m;
            sl[wave] = l;
        }
        __syncthreads();
        M = sm[0];
#pragma unroll
        for (int w = 1; w < W; ++w) M = fmaxf(M, sm[w]);
        float ew[W];
#pragma unroll
        for (int w = 0; w < W; ++w) ew[w] = sm[w] == -INFINITY ? 0.f : __expf(sm[w] - M);
        L = 0.f;
#pragma unroll
        for (int w = 0; w < W; ++w) L = fmaf(ew[w], sl[w], L);
        if (tid < D) {
#pragma unroll
            for (int w = 0; w < W; ++w) O = fmaf(ew[w], so[w][tid], O);
        }
    }

    uint16_t* outp = a.out + (int64_t)b * H * D + (int64_t)h * D;
    const int splits = gridDim.z;
    if (splits == 1) {
        // an invalid position leaves L = 0: the output is NaN
        if (tid < D) outp[tid] = (uint16_t)f32_to_h16_bits(O / L);
        return;
    }

    // ---- 7. several splits: only the live ones (keys up to p) take part;
    // each stores its partials, and the last of them to arrive merges them.
    // A workgroup past p leaves at once; an invalid position has no live
    // split, and split 0 writes the sequence's NaN outputs.
    if (!valid) {
        if (split == 0 && tid < D) outp[tid] = (uint16_t)f32_to_h16_bits(__builtin_nanf(""));
        return;
    }
    if (!live) return;
    const int nlive = (int)((int64_t)p / ((int64_t)W * KPW)) + 1;   // splits 0 .. nlive - 1 hold keys <= p
    const int64_t head = (int64_t)b * H + h;
    float* part_base = a.part + (head * splits + split) * (D + 2);
    if (tid < D) __hip_atomic_store(part_base + tid, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == D) __hip_atomic_store(part_base + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == D + 1) __hip_atomic_store(part_base + D + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // Every thread waits until its partial stores (relaxed agent-scope
    // atomics) have completed, the workgroup meets, and one thread adds one
    // to the head's counter
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
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(a.counters + head, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = prev == (unsigned)(nlive - 1);
        if (last) {
            __hip_atomic_store(a.counters + head, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        last_flag = last;
    }
    __syncthreads();
    if (!last_flag) return;

    // The merge issues all of its loads before it uses any: every split's
    // maximum and sum (into LDS), and this thread's first eight value
    // partials (thread = (channel tid % 128, class tid / 128), class c takes
    // splits c, c + NC, ... of the live ones).  Every thread then forms the
    // weights and the total sum over the live splits in split order, so the
    // result is the same whichever workgroup merges.
    constexpr int NC = NT / D;
    __shared__ float sms[kAttnMaxSplits], sls[kAttnMaxSplits];
    __shared__ float oh[NC][D];
    const float* pb = a.part + head * splits * (D + 2);   // the head's partials (stride: every split)
    const int ch = tid & (D - 1), cls = tid / D;
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int s = cls + NC * i < nlive ? cls + NC * i : 0;
        v[i] = __hip_atomic_load(pb + s * (D + 2) + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int s = tid; s < nlive; s += NT) {
        sms[s] = __hip_atomic_load(pb + s * (D + 2) + D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sls[s] = __hip_atomic_load(pb + s * (D + 2) + D + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int s = 0; s < nlive; ++s) mx = fmaxf(mx, sms[s]);
    float ls = 0.f;
    for (int s = 0; s < nlive; ++s) {
        const float ms = sms[s];
        ls = fmaf(ms == -INFINITY ? 0.f : __expf(ms - mx), sls[s], ls);
    }
    auto weight = [&](int s) {
        const float ms = sms[s];
        return ms == -INFINITY ? 0.f : __expf(ms - mx);
    };
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (cls + NC * i < nlive) acc = fmaf(weight(cls + NC * i), v[i], acc);
    for (int s0 = cls + 8 * NC; s0 < nlive; s0 += 8 * NC) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int s = s0 + NC * i < nlive ? s0 + NC * i : 0;
            v[i] = __hip_atomic_load(pb + s * (D + 2) + ch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (s0 + NC * i < nlive) acc = fmaf(weight(s0 + NC * i), v[i], acc);
    }
    oh[cls][ch] = acc;
    __syncthreads();
    if (tid < D) {
        float o = oh[0][tid];
#pragma unroll
        for (int c = 1; c < NC; ++c) o += oh[c][tid];
        outp[tid] = (uint16_t)f32_to_h16_bits(o / ls);
    }
}

}  // namespace

// Sixteen waves (1024 threads, at most 128 registers each) only with 16 keys
// per wave: more would spill.
bool attn_shape_supported(const AttnShape& sh) {
    return ((sh.kpw == 16 || sh.kpw == 32 || sh.kpw == 64) && (sh.waves == 4 || sh.waves == 8)) ||
           (sh.kpw == 16 && sh.waves == 16);
}

AttnShape attn_default_shape(const AttnArgs& a) {
    // four waves; the largest span that still gives 512 workgroups, at least 16 keys per wave
    for (int kpw = 64; kpw >= 16; kpw /= 2) {
        const AttnShape sh{kpw, 4};
        if ((int64_t)a.B * a.H * attn_splits(a, sh) >= 512) return sh;
    }
    return AttnShape{16, 4};
}

int64_t attn_splits(const AttnArgs& a, const AttnShape& sh) {
    const int64_t span = (int64_t)sh.kpw * sh.waves;
    return (a.max_len + span - 1) / span;
}

template <int KPW, int W>
hipError_t launch_attn_t(const AttnArgs& a, const dim3& grid, hipStream_t stream) {
    hipLaunchKernelGGL((decode_attn_kernel<KPW, W>), grid, dim3(64 * W), 0, stream, a);
    return hipGetLastError();
}

template <int KPW>
hipError_t launch_attn_w(const AttnArgs& a, int waves, const dim3& grid, hipStream_t stream) {
    switch (waves) {
        case 4: return launch_attn_t<KPW, 4>(a, grid, stream);
        case 8: return launch_attn_t<KPW, 8>(a, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_attn(const AttnArgs& a, const AttnShape& sh, hipStream_t stream) {
    const dim3 grid((unsigned)a.H, (unsigned)a.B, (unsigned)attn_splits(a, sh));
    if (sh.kpw == 16 && sh.waves == 16) return launch_attn_t<16, 16>(a, grid, stream);
    switch (sh.kpw) {
        case 16: return launch_attn_w<16>(a, sh.waves, grid, stream);
        case 32: return launch_attn_w<32>(a, sh.waves, grid, stream);
        case 64: return launch_attn_w<64>(a, sh.waves, grid, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace w4a16
