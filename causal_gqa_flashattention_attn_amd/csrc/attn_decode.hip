// attn_decode.hip -- one decode step of grouped-query attention against a key/value cache.
//
// The pages say the attention supports a KV cache for autoregressive generation ("NanoEuler"
// article on ainews.cool, section "technical deep dive", attention item).  Each (batch, query
// head) has one new query; it attends to the cached keys 0 .. lens[b] - 1 of its key/value head
// (its own position included), with scale 1/sqrt(D).  Any RoPE has been applied by the caller.
//
// The step reads the whole cache once and does about 4 flops per byte of it, so it is bound by
// HBM bandwidth, not by arithmetic: it runs on the vector ALUs, with every lane streaming 16
// bytes of a key (value) row per load.  The work is split over the cache length (split-KV):
//   decode_split  grid (split, batch x kv head x query-head chunk), 4 waves of 64 keys each;
//                 one work-group serves every query head of its key/value head, so each cache
//                 row is read once.  Each lane keeps an online softmax (running maximum, sum,
//                 output slice) per query head over the keys it saw; lanes are merged by
//                 shuffles, then wave 0 merges the waves (one query head per group of lanes,
//                 every wave's state read at once), and the split's (o / l, lse) goes to the
//                 workspace.
//   decode_merge  per (batch, query head): log-sum-exp of the splits' lse, weighted sum of their
//                 outputs.  Splits past lens[b] are neither computed nor read.
// When one split covers the whole cache (Tc <= 512: 4 or 8 waves of 64 keys), the split kernel
// writes o and lse itself and the merge launch is skipped: for short caches the step is then a
// single launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace ne {
namespace {

constexpr int kDecWaves = 4;
constexpr int kDecKeysPerWave = 64;
constexpr int kDecSplit = kDecWaves * kDecKeysPerWave;  // keys per split (several splits)
constexpr int kDecWavesOne = 8;                         // waves of a single split (Tc <= 512)


struct DecArgs {
    const void *q, *k, *v;
    const int *lens;
    void *o;
    float *lse;
    float *part_o, *part_lse;  // workspace: [nsplit][B][Hq][D] and [nsplit][B][Hq]
    int B, Hq, Hkv, Tc, G, nhc, nsplit;
    int xcd;  // 1: blockIdx.y interleaved so that a key/value head's head chunks share an XCD
    float qscale;  // log2(e) / sqrt(D): scores in base-2 units
};

// Lane geometry: a lane streams E elements (16 bytes) of a row; LPK lanes cover a row of D;
// one wave-wide load covers KPI rows; a wave's KPW keys take NIT loads, issued PASS at a time
// (fewer at once for wide head groups, whose per-head state takes the registers).  WIDE: up
// to 16 at once (a single split: with two waves per SIMD, each has the registers), so that a
// wave's keys are one round of loads.
template <int D, typename T, int GC, int KPW = kDecKeysPerWave, bool WIDE = false>
struct DecCfg {
    static constexpr int E = 16 / sizeof(T);
    static constexpr int LPK = D / E;
    static constexpr int KPI = 64 / LPK;
    static constexpr int NIT = KPW / KPI;
    static constexpr int PMAX = WIDE && GC * E <= 16 ? 16 : GC <= 4 ? 8 : 4;
    static constexpr int PASS = NIT < PMAX ? NIT : PMAX;
    static_assert(LPK >= 1 && 64 % LPK == 0 && NIT % PASS == 0, "unsupported head size");
};

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes of a row, kept raw until used.
template <typename T>
__device__ __forceinline__ u32x4_t load_raw16(const T *p) {
    return *reinterpret_cast<const u32x4_t *>(p);
}

// Element e of a raw 16-byte chunk as fp32.
template <typename T>
__device__ __forceinline__ float raw_elt(const u32x4_t &r, int e) {
    if constexpr (sizeof(T) == 4) {
        return __uint_as_float(r[e]);
    } else {
        const unsigned w = r[e >> 1];
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    }
}

template <typename T>
__device__ __forceinline__ void load_row16(const T *p, float (&x)[16 / sizeof(T)]) {
    const u32x4_t r = load_raw16<T>(p);
#pragma unroll
    for (int e = 0; e < 16 / (int)sizeof(T); ++e) x[e] = raw_elt<T>(r, e);
}

template <typename T>
__device__ __forceinline__ T to_elt(float x) {
    return (T)x;
}

// Sum over each aligned group of N lanes (N = 1 .. 32, a power of two), left in every lane of the
// group, by DPP moves (plain VALU operations): swaps within quads, then the mirror of each 8- and
// 16-lane row; a group of 32 then adds the other 16-lane row by a lane swap (both rows add the
// same two values, so every lane of the group holds the same sum).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32,
                  "group of 1 .. 32 lanes");
    auto dpp = [](float v, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), decltype(ctrl)::value,
                                                       0xf, 0xf, false));
    };
    if constexpr (N >= 2) x += dpp(x, std::integral_constant<int, 0xB1>{});   // quad_perm 1,0,3,2
    if constexpr (N >= 4) x += dpp(x, std::integral_constant<int, 0x4E>{});   // quad_perm 2,3,0,1
    if constexpr (N >= 8) x += dpp(x, std::integral_constant<int, 0x141>{});  // row_half_mirror
    if constexpr (N >= 16) x += dpp(x, std::integral_constant<int, 0x140>{}); // row_mirror
    if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
    return x;
}

// Running (m, l, o) of one query head over some keys: scores in base 2, o unnormalised.
template <int E>
struct DecState {
    float m, l, o[E];
};

template <int E>
__device__ __forceinline__ void dec_merge(DecState<E> &a, float m2, float l2, const float (&o2)[E]) {
    const float mn = fmaxf(a.m, m2);
    const float s1 = fast_exp2(a.m - mn), s2 = fast_exp2(m2 - mn);
    a.l = a.l * s1 + l2 * s2;
#pragma unroll
    for (int e = 0; e < E; ++e) a.o[e] = a.o[e] * s1 + o2[e] * s2;
    a.m = mn;
}

// NW waves of KPW keys per work-group.  ONE: a single split covers the cache, so the work-group
// writes o and lse (o = 0, lse = -inf for an empty cache) instead of its workspace entries.
template <int D, typename T, int GC, int NW, bool ONE, int KPW = kDecKeysPerWave>
__global__ void __launch_bounds__(64 * NW) decode_split(DecArgs a) {
    using C = DecCfg<D, T, GC, KPW, ONE && NW <= 8>;
    constexpr int E = C::E;
    // Grid: (split, batch x kv head x head chunk); a single split is a 1-D grid of the latter.
    const int s = ONE ? 0 : blockIdx.x;
    int y = ONE ? blockIdx.x : blockIdx.y;
    int hc;
    if (a.xcd) {
        // Work-groups are dealt to the 8 XCDs in turn, so y, y + 8, ... share an XCD (and its
        // L2): those take the head chunks of one key/value head, whose rows each of them reads.
        const int lane8 = y % 8, rest = y / 8;
        hc = rest % a.nhc;
        y = (rest / a.nhc) * 8 + lane8;
    } else {
        hc = y % a.nhc;
        y /= a.nhc;
    }
    const int g = y % a.Hkv;
    const int b = y / a.Hkv;
    const int len = min(max(a.lens[b], 0), a.Tc);
    const int k0 = s * NW * KPW;
    if (!ONE && k0 >= len) return;  // past the cached length: the merge does not read this split
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int sub = lane % C::LPK, kl = lane / C::LPK;
    const int h0 = g * a.G + hc * GC;
    const int gn = min(GC, a.G - hc * GC);

    float qv[GC][E];
    DecState<E> st[GC];
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
        float x[E];
        if (gi < gn)
            load_row16<T>(static_cast<const T *>(a.q) + ((size_t)b * a.Hq + h0 + gi) * D + sub * E, x);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            qv[gi][e] = gi < gn ? x[e] * a.qscale : 0.f;
            st[gi].o[e] = 0.f;
        }
        st[gi].m = kNegBig;
        st[gi].l = 0.f;
    }

    const size_t row0 = ((size_t)b * a.Hkv + g) * a.Tc;
    const T *kb = static_cast<const T *>(a.k) + row0 * D + sub * E;
    const T *vb = static_cast<const T *>(a.v) + row0 * D + sub * E;
    const int kw = k0 + wave * KPW;
#pragma unroll
    for (int p0 = 0; p0 < C::NIT; p0 += C::PASS) {
        if (kw + p0 * C::KPI >= len) break;  // wave-uniform
        // Every load of the pass is requested before the first is used.
        u32x4_t kr[C::PASS], vr[C::PASS];
#pragma unroll
        for (int i = 0; i < C::PASS; ++i) {
            const int j = min(kw + (p0 + i) * C::KPI + kl, len - 1);
            kr[i] = load_raw16<T>(kb + (size_t)j * D);
            vr[i] = load_raw16<T>(vb + (size_t)j * D);
        }
        // Scores of the pass's keys, then one running-maximum update per head, then the sums.
        float sc[C::PASS][GC];
#pragma unroll
        for (int i = 0; i < C::PASS; ++i) {
            const bool valid = kw + (p0 + i) * C::KPI + kl < len;
#pragma unroll
            for (int gi = 0; gi < GC; ++gi) {
                float d = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) d = fmaf(qv[gi][e], raw_elt<T>(kr[i], e), d);
                d = group_sum<C::LPK>(d);  // the row's dot product: its LPK lanes together
                sc[i][gi] = valid ? d : -INFINITY;
            }
        }
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) {
            float pm = sc[0][gi];
#pragma unroll
            for (int i = 1; i < C::PASS; ++i) pm = fmaxf(pm, sc[i][gi]);
            const float mn = fmaxf(st[gi].m, pm);
            const float al = fast_exp2(st[gi].m - mn);
            st[gi].l *= al;
#pragma unroll
            for (int e = 0; e < E; ++e) st[gi].o[e] *= al;
            st[gi].m = mn;
        }
#pragma unroll
        for (int i = 0; i < C::PASS; ++i)
#pragma unroll
            for (int gi = 0; gi < GC; ++gi) {
                const float p = fast_exp2(sc[i][gi] - st[gi].m);
                st[gi].l += p;
#pragma unroll
                for (int e = 0; e < E; ++e) st[gi].o[e] = fmaf(p, raw_elt<T>(vr[i], e), st[gi].o[e]);
            }
    }

    // Merge the KPI lanes that hold the same slice of different keys (xor over the key index).
#pragma unroll
    for (int w = C::LPK; w < 64; w <<= 1)
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) {
            float o2[E];
#pragma unroll
            for (int e = 0; e < E; ++e) o2[e] = __shfl_xor(st[gi].o[e], w, 64);
            const float m2 = __shfl_xor(st[gi].m, w, 64), l2 = __shfl_xor(st[gi].l, w, 64);
            dec_merge<E>(st[gi], m2, l2, o2);
        }

    // Each wave's state goes to LDS for wave 0 to merge.
    __shared__ float red[NW][GC][D + 2];
    if (kl == 0)
#pragma unroll
        for (int gi = 0; gi < GC; ++gi) {
#pragma unroll
            for (int e = 0; e < E; ++e) red[wave][gi][sub * E + e] = st[gi].o[e];
            if (sub == 0) {
                red[wave][gi][D] = st[gi].m;
                red[wave][gi][D + 1] = st[gi].l;
            }
        }
    __syncthreads();
    if (wave != 0) return;
    // Wave 0 merges the waves' states: each group of LPK lanes takes one query head (the lanes'
    // slices of its output), reads every wave's (m, l, o) at once, and sums them weighted by
    // 2^(m_w - M) with M the largest m, in wave order.
    constexpr int HPP = 64 / C::LPK;  // heads merged at once
    for (int g0 = 0; g0 < GC; g0 += HPP) {
        const int gi = g0 + kl;
        if (gi >= gn) continue;
        float mw[NW];
        float M = kNegBig;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = red[w][gi][D];
            M = fmaxf(M, mw[w]);
        }
        float L = 0.f, O[E];
#pragma unroll
        for (int e = 0; e < E; ++e) O[e] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float sw = fast_exp2(mw[w] - M);
            L = fmaf(red[w][gi][D + 1], sw, L);
#pragma unroll
            for (int e = 0; e < E; ++e) O[e] = fmaf(red[w][gi][sub * E + e], sw, O[e]);
        }
        const size_t bh = (size_t)b * a.Hq + h0 + gi;
        const size_t ps = (size_t)s * a.B * a.Hq + bh;
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const float ls = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        if constexpr (ONE) {
            T *orow = static_cast<T *>(a.o) + bh * D + sub * E;
#pragma unroll
            for (int e = 0; e < E; ++e) orow[e] = to_elt<T>(O[e] * inv);
            if (sub == 0) a.lse[bh] = ls;
        } else {
            float *po = a.part_o + ps * D + sub * E;
#pragma unroll
            for (int e = 0; e < E; e += 4) *reinterpret_cast<f32x4 *>(po + e) =
                f32x4{O[e] * inv, O[e + 1] * inv, O[e + 2] * inv, O[e + 3] * inv};
            if (sub == 0) a.part_lse[ps] = ls;
        }
    }
}

// One wave per (batch, query head).  The splits' lse are combined across lanes (one split per
// lane, in rounds of 64); the outputs with 16-byte loads, 64 / (D / 4) splits per wave-wide load,
// all loads independent, then summed over the lanes that hold the same columns.
template <int D, typename T>
__global__ void __launch_bounds__(64) decode_merge(DecArgs a) {
    constexpr int LPR = D / 4;       // lanes per output row (4 floats each)
    constexpr int RPW = 64 / LPR;    // rows (splits) per wave-wide load
    const int lane = threadIdx.x;
    const long long bh = blockIdx.x;  // one single-wave work-group each, to reach every CU
    const int b = (int)(bh / a.Hq);
    const int len = min(max(a.lens[b], 0), a.Tc);
    const int ns = (len + kDecSplit - 1) / kDecSplit;
    const size_t stride = (size_t)a.B * a.Hq;
    float mx = -INFINITY;
    for (int s = lane; s < ns; s += 64) mx = fmaxf(mx, a.part_lse[s * stride + bh]);
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) mx = fmaxf(mx, __shfl_xor(mx, w, 64));
    float wsum = 0.f;
    for (int s = lane; s < ns; s += 64) wsum += __expf(a.part_lse[s * stride + bh] - mx);
#pragma unroll
    for (int w = 1; w < 64; w <<= 1) wsum += __shfl_xor(wsum, w, 64);
    const int sub = lane % LPR, r = lane / LPR;
    f32x4 acc{0.f, 0.f, 0.f, 0.f};
    if (mx > -INFINITY)
        for (int s = r; s < ns; s += RPW) {
            const float w = __expf(a.part_lse[s * stride + bh] - mx);
            acc += w * *reinterpret_cast<const f32x4 *>(a.part_o + (s * stride + bh) * D + 4 * sub);
        }
#pragma unroll
    for (int w = LPR; w < 64; w <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], w, 64);
    if (r == 0) {
        const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
        T *orow = static_cast<T *>(a.o) + bh * D + 4 * sub;
#pragma unroll
        for (int e = 0; e < 4; ++e) orow[e] = to_elt<T>(acc[e] * inv);
    }
    if (lane == 0) a.lse[bh] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

template <int D, typename T, int NW, bool ONE, int KPW = kDecKeysPerWave>
const void *pick_split(int gc) {
    return gc == 1   ? (const void *)decode_split<D, T, 1, NW, ONE, KPW>
           : gc == 2 ? (const void *)decode_split<D, T, 2, NW, ONE, KPW>
           : gc == 4 ? (const void *)decode_split<D, T, 4, NW, ONE, KPW>
                     : (const void *)decode_split<D, T, 8, NW, ONE, KPW>;
}

template <int D, typename T>
hipError_t launch_decode_t(DecArgs &a, hipStream_t st) {
    // Query heads per work-group: with several splits, the whole group when it is small, else
    // chunks of 8 (each cache row is read once).  A single split has too few work-groups to
    // fill the chip that way, so it takes one query head per work-group: the heads of a group
    // read its rows again, from the L2 of their XCD.
    const bool one = a.Tc <= kDecWavesOne * kDecKeysPerWave;
    const int gc = one || a.G <= 1 ? 1 : a.G <= 2 ? 2 : a.G <= 4 ? 4 : 8;
    a.nhc = (a.G + gc - 1) / gc;
    a.xcd = a.nhc > 1 && ((long long)a.B * a.Hkv) % 8 == 0;
    void *params[] = {&a};
    const long long gy = (long long)a.B * a.Hkv * a.nhc;
    // A cache of at most 512 keys is one split (4 or 8 waves): no merge.
    if (one) {
        if (gy > 0x7fffffffLL) return hipErrorInvalidValue;
        const int nw = a.Tc <= kDecSplit ? kDecWaves : kDecWavesOne;
        const void *fn = nw == kDecWaves ? pick_split<D, T, kDecWaves, true>(gc)
                                         : pick_split<D, T, kDecWavesOne, true>(gc);
        return hipLaunchKernel(fn, dim3((unsigned)gy), dim3(64 * nw), params, 0, st);
    }
    if (gy > 65535) return hipErrorInvalidValue;
    hipError_t e = hipLaunchKernel(pick_split<D, T, kDecWaves, false>(gc),
                                   dim3((unsigned)a.nsplit, (unsigned)gy), dim3(64 * kDecWaves),
                                   params, 0, st);
    if (e != hipSuccess) return e;
    const long long nbh = (long long)a.B * a.Hq;
    return hipLaunchKernel((const void *)decode_merge<D, T>, dim3((unsigned)nbh), dim3(64), params,
                           0, st);
}

}  // namespace

int decode_splits(int Tc) { return (Tc + kDecSplit - 1) / kDecSplit; }

hipError_t launch_decode(const Shape &s, int bf16, const void *q, const void *k, const void *v,
                         const int *lens, void *o, float *lse, float *part_o, float *part_lse,
                         hipStream_t st) {
    DecArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.lens = lens;
    a.o = o;
    a.lse = lse;
    a.part_o = part_o;
    a.part_lse = part_lse;
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.Tc = s.T;
    a.G = s.G;
    a.nsplit = decode_splits(s.T);
    a.qscale = (float)(1.4426950408889634 / sqrt((double)s.D));
    if (bf16)
        return s.D == 128  ? launch_decode_t<128, __bf16>(a, st)
               : s.D == 64 ? launch_decode_t<64, __bf16>(a, st)
                           : launch_decode_t<32, __bf16>(a, st);
    return s.D == 128  ? launch_decode_t<128, float>(a, st)
           : s.D == 64 ? launch_decode_t<64, float>(a, st)
                       : launch_decode_t<32, float>(a, st);
}

}  // namespace ne
