// attn_f32.hip -- float32 causal grouped-query FlashAttention for gfx950, forward and backward.
//
// The method (NanoEuler's training kernel): exact softmax attention evaluated tile by tile with
// an online softmax, never storing the T x T score matrix ("nanoeuler: un LLM estilo GPT-2
// construido desde cero en C y CUDA", second paragraph; "NanoEuler -- Show HN" Japanese README
// translation, section "Kernels and acceleration"); causal tiles above the diagonal are skipped
// rather than masked ("NanoEuler: a GPT-2 hand-built in pure C/CUDA" (openai-hub),
// implementation details, item "causal mask in attention"); query heads share key/value heads
// (README translations, section "Architecture").
//
// All contractions run on the fp32 matrix cores (v_mfma_f32_32x32x2f32).  Every wave owns 32
// query rows (forward, dQ) or 32 key rows (dK/dV) as the columns of its 32x32 tiles, so softmax
// statistics are per-lane scalars and probability tiles feed the next MFMA from registers.
//
// Kernels:
//   fwd_f32   one work-group per (batch, kv head, query tile); its waves are the group's query
//             heads, so every K/V tile staged in LDS serves all of them.  Per wave:
//             S^T = K Q^T, online softmax (in base 2, scale folded into Q), O^T += V^T P^T.
//   dq_f32    same decomposition; first computes delta_i = dO_i . o_i for its rows (written to
//             the workspace for the dK/dV pass), then per tile S^T, P^T = exp2(S^T - lse2),
//             dP^T = V dO^T, dS^T = P^T (dP^T - delta), dQ^T += K^T dS^T.
//   fwd_f32_1w, dq_f32_1w
//             the same per-tile work in one-wave work-groups, each wave staging its own K/V
//             tiles: for causal self-attention when the group's query heads do not fill a
//             compute unit's four SIMDs evenly (head sizes up to 64).
//   dkdv_f32  one work-group per (batch, kv head, 32-key block); K and V stay in registers, the
//             group's query heads are split over the waves, each streaming its own query
//             blocks through LDS: S = Q K^T, P, dP = dO V^T, dS, dV^T += dO^T P, dK^T += Q^T dS.
//             The waves' partial sums are added in LDS in a fixed order: the two-pass backward
//             uses no atomics, so its results are reproducible bit for bit.
//   dkdvq_f32 the single-pass backward: dkdv_f32 plus dQ added into dq with atomics.
#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "attn_device.hpp"
#include "attn_kernels.hpp"

// Minimum resident waves per SIMD each kernel is compiled for (caps its registers).
#ifndef NE_FWD_WAVES_PER_EU
#define NE_FWD_WAVES_PER_EU 2
#endif
#ifndef NE_DQ_WAVES_PER_EU
#define NE_DQ_WAVES_PER_EU 2
#endif
#ifndef NE_DKDVQ_WAVES_PER_EU
#define NE_DKDVQ_WAVES_PER_EU 2
#endif
#ifndef NE_DKDV_WAVES_PER_EU
#define NE_DKDV_WAVES_PER_EU 2
#endif

namespace ne {

namespace {

template <int D>
struct Cfg {
    static constexpr int LD = D + 4;      // LDS row stride in floats: consecutive rows start 16 B
                                          // apart modulo 128 B, so 8 lanes reading 16 B from 8
                                          // rows hit disjoint banks
    static constexpr int NS = D / 2;      // MFMA k-steps of a contraction over D
    static constexpr int ND = D / 32;     // 32-wide column blocks of D
    static constexpr int C4 = D / 4;      // float4 per row
    static constexpr int RPC = 64 / C4;   // rows per wave-wide float4 chunk
    static constexpr int CH = 32 / RPC;   // chunks per 32-row tile
    static constexpr int MAXC = (CH + 1) / 2;  // chunks per wave (query-tile WGs have >= 2 waves)
};

struct RopeArgs {
    int on;
    double log2_base;  // log2(rope_base)
};

// Rotation of the two adjacent pairs (c, c+1), (c+2, c+3) of a row at position t by
// t * base^(-2i/D), i = pair index; `inv` applies the transpose.  The angle is reduced modulo
// one turn in double precision, so the float32 sine and cosine are accurate at any position.
template <int D>
__device__ __forceinline__ f32x4 rope4(f32x4 x, int t, int c, const RopeArgs &r, bool inv) {
    f32x4 y;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int i = c / 2 + p;
        const double turns = (double)t * exp2(-(2.0 * i / D) * r.log2_base) * 0.15915494309189535;
        const float frac = (float)(turns - rint(turns));
        float sn, cs;
        sincospif(2.0f * frac, &sn, &cs);
        const float a = x[2 * p], b = x[2 * p + 1];
        if (!inv) {
            y[2 * p] = a * cs - b * sn;
            y[2 * p + 1] = a * sn + b * cs;
        } else {
            y[2 * p] = a * cs + b * sn;
            y[2 * p + 1] = b * cs - a * sn;
        }
    }
    return y;
}

struct Args {
    const float *q, *k, *v, *o, *lse, *dO;
    float *out_o, *out_lse, *dq, *dk, *dv, *delta;
    float *qrot;  // dQ pass with RoPE: rotated query rows, written for the dK/dV pass
    int B, Hq, Hkv, T, G;
    int Tk, qoff;      // forward: key length and position of query row 0 (Tk = T, 0 usually)
    int hpw, rb, nqt;  // query-tile kernels
    int paired;        // work-groups take mirrored pairs of tiles or key blocks
    int mstep;         // unpaired causal query tiles: mirrored tiles this many rows of the
                       // launch order apart (0: longest first)
    int nkb;           // key blocks per head (dK/dV)
    float qscale;      // scale * log2(e)
    float scale;       // 1 / sqrt(D)
    RopeArgs rope;
    TLays L;           // tensor layouts
};

// First element of head h of batch b in a tensor of layout l.
__device__ __forceinline__ const float *head_at(const float *p, const TLay &l, int b, int h) {
    return p + b * l.sb + (size_t)h * l.sh;
}
__device__ __forceinline__ float *head_at(float *p, const TLay &l, int b, int h) {
    return p + b * l.sb + (size_t)h * l.sh;
}

struct QTile {
    int b, g, h, qt, r0;  // r0: first query row of this wave
};

// Work-group -> (batch, kv head, head chunk) and its query tiles.  Work-group row t takes tile
// nqt-1-t (under a causal mask the longest tiles go first) and, in paired launches, also tile t
// after it.
struct QTileWork {
    int b, g, hc, qt0, qt1;  // qt1 < 0: a single tile
};

__device__ __forceinline__ QTileWork decode_qwork(const Args &a) {
    const int nhc = a.G / a.hpw;
    const int per = a.B * a.Hkv * nhc;
    const int t = blockIdx.x / per;
    int r = blockIdx.x % per;
    QTileWork w;
    w.hc = r % nhc;
    r /= nhc;
    w.g = r % a.Hkv;
    w.b = r / a.Hkv;
    if (a.mstep > 0) {
        // Rows t and t + mstep of the launch order are `per * mstep` work-groups apart, one
        // stride of the compute units when work-groups go round-robin over them: those rows
        // take mirrored tiles (lengths summing to nqt + 1), so every unit gets the same work.
        // Within each block of 2 mstep rows the long tiles come first.
        const int u = t / (2 * a.mstep), k = t % (2 * a.mstep);
        const int pr = u * a.mstep + k % a.mstep;  // pair index, 0 .. nqt/2 - 1
        w.qt0 = k < a.mstep ? a.nqt - 1 - pr : pr;
    } else {
        // Longest tile first under a causal mask (the order is immaterial otherwise).
        w.qt0 = a.nqt - 1 - t;
    }
    w.qt1 = a.paired && t < w.qt0 ? t : -1;
    return w;
}

__device__ __forceinline__ QTile qtile_of(const Args &a, const QTileWork &w, int qt, int wave) {
    QTile c;
    c.b = w.b;
    c.g = w.g;
    c.qt = qt;
    c.h = w.g * a.G + w.hc * a.hpw + wave / a.rb;
    c.r0 = qt * 32 * a.rb + (wave % a.rb) * 32;
    return c;
}

// K and V tiles of 32 rows, staged global -> registers -> LDS (padded rows), double buffered.
// Rows past the end are loaded from the last row (so every load is unconditional and can stay in
// flight while the current tile is computed) and replaced by zeros when written to LDS.  With
// RoPE the keys arrive already rotated.
template <int D>
struct KVStager {
    using C = Cfg<D>;
    f32x4 k[C::MAXC], v[C::MAXC];

    // kg, vg: the heads' first rows; ks, vs: their row strides (elements).
    __device__ __forceinline__ void load(const float *kg, const float *vg, int ks, int vs,
                                         int tile, int T, int wave, int nw,
                                         int lane) {
        const int c4 = 4 * (lane % C::C4);
#pragma unroll
        for (int i = 0; i < C::MAXC; ++i) {
            const int c = wave + i * nw;
            if (c < C::CH) {
                const int row = min(tile * 32 + c * C::RPC + lane / C::C4, T - 1);
                k[i] = ld4(kg + row * ks + c4);
                v[i] = ld4(vg + row * vs + c4);
            }
        }
    }
    __device__ __forceinline__ void store(float *sK, float *sV, int tile, int T, int wave, int nw,
                                          int lane) {
        const int c4 = 4 * (lane % C::C4);
        const f32x4 zero{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < C::MAXC; ++i) {
            const int c = wave + i * nw;
            if (c < C::CH) {
                const int r = c * C::RPC + lane / C::C4;
                const int row = tile * 32 + r;
                st4(sK + r * C::LD + c4, row < T ? k[i] : zero);
                st4(sV + r * C::LD + c4, row < T ? v[i] : zero);
            }
        }
    }
};

// This lane's query row, columns NS*half .. NS*half+NS-1, scaled; rotated first with RoPE.
// base: the head's first row; rs: the row stride (elements).
template <int D, bool ROPE>
__device__ __forceinline__ void load_row_half(float (&dst)[Cfg<D>::NS], const float *base,
                                             int rs, int row, int T, int half, float mul,
                                             const RopeArgs &rp) {
    using C = Cfg<D>;
    const float *src = base + min(row, T - 1) * rs + C::NS * half;
#pragma unroll
    for (int c = 0; c < C::NS / 4; ++c) {
        f32x4 t = ld4(src + 4 * c);
        if (ROPE) t = rope4<D>(t, row, C::NS * half + 4 * c, rp, false);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[4 * c + i] = t[i] * mul;
    }
}

// The rotation and scaling of a row half loaded raw by load_row_half<D, false> with mul = 1, for
// callers that request other reads before the rotation waits for this one.
template <int D>
__device__ __forceinline__ void rotate_row_half(float (&x)[Cfg<D>::NS], int row, int half,
                                                float mul, const RopeArgs &rp) {
    using C = Cfg<D>;
#pragma unroll
    for (int c = 0; c < C::NS / 4; ++c) {
        const f32x4 t = rope4<D>(f32x4{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]}, row,
                                 C::NS * half + 4 * c, rp, false);
#pragma unroll
        for (int i = 0; i < 4; ++i) x[4 * c + i] = t[i] * mul;
    }
}

// acc += sum_st A[st] * x[st], with A[st] = a[st] read from LDS in 16-byte groups: a chain of NS
// dependent MFMAs over one row of a tile.  The reads are software-pipelined: group g+1 is
// requested before the four MFMAs of group g are issued, and sched_barrier keeps the compiler
// from sinking the read back next to its use, so LDS latency hides behind the matrix core.
template <int NS>
__device__ __forceinline__ f32x16 chain_lds4(const float *a, const float (&x)[NS], f32x16 acc) {
    f32x4 cur = ld4(a);
#pragma unroll
    for (int g = 0; g < NS / 4; ++g) {
        f32x4 nxt = cur;
        if (g + 1 < NS / 4) nxt = ld4(a + 4 * (g + 1));
        __builtin_amdgcn_sched_barrier(0);
        acc = mfma32(cur[0], x[4 * g + 0], acc);
        acc = mfma32(cur[1], x[4 * g + 1], acc);
        acc = mfma32(cur[2], x[4 * g + 2], acc);
        acc = mfma32(cur[3], x[4 * g + 3], acc);
        cur = nxt;
    }
    return acc;
}

// S^T tile (32 keys x 32 queries) = K_tile (LDS, padded rows) x this wave's query rows (regs).
template <int D>
__device__ __forceinline__ f32x16 scores_t(const float *K, const float (&x)[Cfg<D>::NS], int col,
                                           int half) {
    using C = Cfg<D>;
    return chain_lds4<C::NS>(K + col * C::LD + C::NS * half, x, zero16());
}

// acc (D x 32 queries, transposed) += M_tile^T (D x 32 keys) * X (32 keys x 32 queries), with
// X the accumulator-layout tile in registers and M_tile the LDS tile [key][d].  Step st reads
// row acc_row(st, half); the reads of step st+1 are issued ahead of the MFMAs of step st.
template <int D>
__device__ __forceinline__ void accum_t(f32x16 (&acc)[Cfg<D>::ND], const float *M, const f32x16 &x,
                                        int col, int half) {
    using C = Cfg<D>;
    float cur[C::ND], nxt[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) cur[dd] = M[acc_row(0, half) * C::LD + dd * 32 + col];
#pragma unroll
    for (int st = 0; st < 16; ++st) {
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd)
            nxt[dd] = st + 1 < 16 ? M[acc_row(st + 1, half) * C::LD + dd * 32 + col] : cur[dd];
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd) acc[dd] = mfma32(cur[dd], x[st], acc[dd]);
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd) cur[dd] = nxt[dd];
    }
}

// Online-softmax step of one S^T tile (32 keys x this wave's 32 queries, keys from k0): masks
// keys after the query (position qpos) or past the end, moves the reference maximum m, rescaling
// l and O when it does, and turns s into the tile's probabilities.  p0: position of the wave's
// first query row.
template <int D, bool CAUSAL>
__device__ __forceinline__ void fwd_softmax(f32x16 &s, f32x16 (&acc)[Cfg<D>::ND], float &m,
                                            float &l, int k0, int p0, int qpos, int Tk, int half) {
    if ((CAUSAL && k0 + 31 > p0) || k0 + 32 > Tk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = k0 + acc_row(v, half);
            if ((CAUSAL && key > qpos) || key >= Tk) s[v] = -INFINITY;
        }
    }
    // Lazy rescale: the reference maximum m only moves when a score of this lane's row
    // exceeds it by more than 2^8 (probabilities up to 256 are exact enough in fp32 sums), so
    // most tiles skip the rescale of l and O.  The row maximum over both lane halves is only
    // formed when some lane needs it.
    const auto mx3 = [](float x, float y, float z) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
    };
    const float lmax = __builtin_elementwise_maximum(
        mx3(mx3(s[0], s[1], s[2]), mx3(s[3], s[4], s[5]), mx3(s[6], s[7], s[8])),
        mx3(mx3(s[9], s[10], s[11]), mx3(s[12], s[13], s[14]), s[15]));
    if (__builtin_amdgcn_ballot_w64(lmax > m + 8.0f) != 0) {
        // Only the rows that need it move (others keep m bit for bit, whatever the other rows
        // of the wave hold).
        const float rmax = fmaxf(lmax, swap_halves(lmax));
        if (rmax > m + 8.0f) {
            const float alpha = fast_exp2(m - rmax);
            m = rmax;
            l *= alpha;
#pragma unroll
            for (int dd = 0; dd < Cfg<D>::ND; ++dd) acc[dd] *= alpha;
        }
    }
    float ps = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        s[v] = fast_exp2(s[v] - m);
        ps += s[v];
    }
    l += ps;
}

// The forward's epilogue: O = acc / l and the natural-log LSE of the wave's rows.
template <int D>
__device__ __forceinline__ void fwd_store(const Args &a, int b, int h, int qrow, int half,
                                          const f32x16 (&acc)[Cfg<D>::ND], float m, float l) {
    l += swap_halves(l);
    if (qrow < a.T) {
        const float inv = 1.0f / l;
        float *orow = head_at(a.out_o, a.L.o, b, h) + qrow * a.L.o.st;
#pragma unroll
        for (int dd = 0; dd < Cfg<D>::ND; ++dd)
#pragma unroll
            for (int u = 0; u < 4; ++u)
                st4(orow + dd * 32 + 8 * u + 4 * half,
                    f32x4{acc[dd][4 * u] * inv, acc[dd][4 * u + 1] * inv, acc[dd][4 * u + 2] * inv,
                          acc[dd][4 * u + 3] * inv});
        if (half == 0) a.out_lse[((size_t)b * a.Hq + h) * a.T + qrow] = m * kLn2 + logf(l);
    }
}

template <int D, bool CAUSAL, bool ROPE>
__device__ __forceinline__ void fwd_tile(const Args &a, const QTile &c, float (&sK)[2][32 * Cfg<D>::LD],
                                         float (&sV)[2][32 * Cfg<D>::LD]) {
    using C = Cfg<D>;
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    // T query rows; Tk keys; query row r is at position r + qo (a prefill chunk; 0 usually).
    const int T = a.T, Tk = a.Tk, qo = a.qoff;
    const int qrow = c.r0 + col;
    const int p0 = c.r0 + qo;  // position of the wave's first row
    const float *kg = head_at(a.k, a.L.k, c.b, c.g);
    const float *vg = head_at(a.v, a.L.v, c.b, c.g);

    // The first K/V tile is requested before the query row, so the two latencies overlap.
    const int wg_rows = 32 * a.rb;
    const int wg_end = min(c.qt * wg_rows + wg_rows, T);
    const int ntiles = CAUSAL ? (wg_end - 1 + qo) / 32 + 1 : (Tk + 31) / 32;
    KVStager<D> stg;
    stg.load(kg, vg, a.L.k.st, a.L.v.st, 0, Tk, wave, nw, lane);

    float qr[C::NS];
    load_row_half<D, ROPE>(qr, head_at(a.q, a.L.q, c.b, c.h), a.L.q.st, qrow, T, half, a.qscale,
                           a.rope);

    f32x16 acc[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) acc[dd] = zero16();
    float m = kNegBig, l = 0.f;

    stg.store(sK[0], sV[0], 0, Tk, wave, nw, lane);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = j + 1 < ntiles;
        if (more) stg.load(kg, vg, a.L.k.st, a.L.v.st, j + 1, Tk, wave, nw, lane);
        const int k0 = j * 32;
        if (c.r0 < T && (!CAUSAL || k0 <= p0 + 31)) {
            f32x16 s = scores_t<D>(sK[buf], qr, col, half);
            fwd_softmax<D, CAUSAL>(s, acc, m, l, k0, p0, qrow + qo, Tk, half);
            accum_t<D>(acc, sV[buf], s, col, half);
        }
        if (more) stg.store(sK[buf ^ 1], sV[buf ^ 1], j + 1, Tk, wave, nw, lane);
        __syncthreads();
    }
    fwd_store<D>(a, c.b, c.h, qrow, half, acc, m, l);
}

// At D = 128 the forward without RoPE fits two waves per SIMD without spilling (the rotation's
// registers push the RoPE variant to one).
template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(D == 128 ? 256 : 512) __attribute__((amdgpu_waves_per_eu(D == 128 && ROPE ? 1 : NE_FWD_WAVES_PER_EU)))
fwd_f32(Args a) {
    __shared__ __attribute__((aligned(16))) float sK[2][32 * Cfg<D>::LD];
    __shared__ __attribute__((aligned(16))) float sV[2][32 * Cfg<D>::LD];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const QTileWork w = decode_qwork(a);
    fwd_tile<D, CAUSAL, ROPE>(a, qtile_of(a, w, w.qt0, wave), sK, sV);
    if (w.qt1 >= 0) {
        __syncthreads();
        fwd_tile<D, CAUSAL, ROPE>(a, qtile_of(a, w, w.qt1, wave), sK, sV);
    }
}

// The dQ pass's row set-up for this lane's query row: q (rotated with RoPE, the rotation kept in
// qrot for the dK/dV pass, then scaled) and dO in registers, delta_i = dO_i . o_i (written once
// per row for the dK/dV pass) and lse * log2(e).  Rows past the end get P = 0.  The caller may
// request other reads first: every read here is issued before any is used.
template <int D, bool ROPE>
__device__ __forceinline__ void dq_rows(const Args &a, int b, int h, int qrow, int half,
                                        float (&qr)[Cfg<D>::NS], float (&dor)[Cfg<D>::NS],
                                        float &lse2, float &delta) {
    using C = Cfg<D>;
    const int T = a.T;
    const size_t bh = (size_t)b * a.Hq + h;
    float orow[C::NS];
    load_row_half<D, false>(qr, head_at(a.q, a.L.q, b, h), a.L.q.st, qrow, T, half, 1.0f, a.rope);
    load_row_half<D, false>(dor, head_at(a.dO, a.L.dO, b, h), a.L.dO.st, qrow, T, half, 1.0f,
                            a.rope);
    load_row_half<D, false>(orow, head_at(a.o, a.L.o, b, h), a.L.o.st, qrow, T, half, 1.0f,
                            a.rope);
    const float lse_row = a.lse[bh * T + min(qrow, T - 1)];
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE) rotate_row_half<D>(qr, qrow, half, 1.0f, a.rope);
    else {
#pragma unroll
        for (int i = 0; i < C::NS; ++i) qr[i] *= a.qscale;
    }
    if (ROPE) {  // each query row is loaded by exactly one wave: keep its rotation, then scale
        if (qrow < T) {
#pragma unroll
            for (int c = 0; c < C::NS / 4; ++c)
                st4(a.qrot + (bh * T + qrow) * D + C::NS * half + 4 * c,
                    f32x4{qr[4 * c], qr[4 * c + 1], qr[4 * c + 2], qr[4 * c + 3]});
        }
#pragma unroll
        for (int i = 0; i < C::NS; ++i) qr[i] *= a.qscale;
    }
    {
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < C::NS; ++i) part += dor[i] * orow[i];
        delta = part + swap_halves(part);
    }
    if (qrow < T) {
        lse2 = lse_row * kLog2e;
        if (half == 0) a.delta[bh * T + qrow] = delta;
    } else {
        lse2 = INFINITY;  // padding row: P = 0
        delta = 0.f;
    }
}

// One key tile of the dQ pass, from its S^T (p) and dP^T (ds): P^T = exp2(S^T - lse2), zero
// for keys after the query or past the end, then dS^T = P^T (dP^T - delta).
template <bool CAUSAL>
__device__ __forceinline__ void dq_dscores(f32x16 &p, f32x16 &ds, float lse2, float delta, int k0,
                                           int r0, int qrow, int T, int half) {
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = fast_exp2(p[v] - lse2);
    if ((CAUSAL && k0 + 31 > r0) || k0 + 32 > T) {  // a block on the diagonal or the end
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = k0 + acc_row(v, half);
            if ((CAUSAL && key > qrow) || key >= T) p[v] = 0.f;
        }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) ds[v] = p[v] * (ds[v] - delta);
}

// dQ = scale * acc (rotated back with RoPE) for the wave's rows.
template <int D, bool ROPE>
__device__ __forceinline__ void dq_store(const Args &a, int b, int h, int qrow, int half,
                                         const f32x16 (&acc)[Cfg<D>::ND]) {
    if (qrow < a.T) {
        float *drow = head_at(a.dq, a.L.dq, b, h) + qrow * a.L.dq.st;
#pragma unroll
        for (int dd = 0; dd < Cfg<D>::ND; ++dd)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int d = dd * 32 + 8 * u + 4 * half;
                f32x4 x{acc[dd][4 * u] * a.scale, acc[dd][4 * u + 1] * a.scale,
                        acc[dd][4 * u + 2] * a.scale, acc[dd][4 * u + 3] * a.scale};
                if (ROPE) x = rope4<D>(x, qrow, d, a.rope, true);
                st4(drow + d, x);
            }
    }
}

template <int D, bool CAUSAL, bool ROPE>
__device__ __forceinline__ void dq_tile(const Args &a, const QTile &c, float (&sK)[2][32 * Cfg<D>::LD],
                                        float (&sV)[2][32 * Cfg<D>::LD]) {
    using C = Cfg<D>;
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const int T = a.T;
    const int qrow = c.r0 + col;
    const float *kg = head_at(a.k, a.L.k, c.b, c.g);
    const float *vg = head_at(a.v, a.L.v, c.b, c.g);

    // The first K/V tile, the row's q, dO and o and its lse are all requested before any is
    // used, so their latencies overlap.
    const int wg_rows = 32 * a.rb;
    const int wg_end = min(c.qt * wg_rows + wg_rows, T);
    const int ntiles = CAUSAL ? (wg_end - 1) / 32 + 1 : (T + 31) / 32;
    KVStager<D> stg;
    stg.load(kg, vg, a.L.k.st, a.L.v.st, 0, T, wave, nw, lane);
    float qr[C::NS], dor[C::NS], lse2, delta;
    dq_rows<D, ROPE>(a, c.b, c.h, qrow, half, qr, dor, lse2, delta);

    f32x16 acc[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) acc[dd] = zero16();

    stg.store(sK[0], sV[0], 0, T, wave, nw, lane);
    __syncthreads();
    for (int j = 0; j < ntiles; ++j) {
        const int buf = j & 1;
        const bool more = j + 1 < ntiles;
        if (more) stg.load(kg, vg, a.L.k.st, a.L.v.st, j + 1, T, wave, nw, lane);
        const int k0 = j * 32;
        if (c.r0 < T && (!CAUSAL || k0 <= c.r0 + 31)) {
            f32x16 p = scores_t<D>(sK[buf], qr, col, half);
            f32x16 ds = scores_t<D>(sV[buf], dor, col, half);  // dP^T = V dO^T
            dq_dscores<CAUSAL>(p, ds, lse2, delta, k0, c.r0, qrow, T, half);
            accum_t<D>(acc, sK[buf], ds, col, half);  // dQ^T += K^T dS^T
        }
        if (more) stg.store(sK[buf ^ 1], sV[buf ^ 1], j + 1, T, wave, nw, lane);
        __syncthreads();
    }
    dq_store<D, ROPE>(a, c.b, c.h, qrow, half, acc);
}

template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(D == 128 ? 256 : 512) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : NE_DQ_WAVES_PER_EU)))
dq_f32(Args a) {
    __shared__ __attribute__((aligned(16))) float sK[2][32 * Cfg<D>::LD];
    __shared__ __attribute__((aligned(16))) float sV[2][32 * Cfg<D>::LD];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const QTileWork w = decode_qwork(a);
    dq_tile<D, CAUSAL, ROPE>(a, qtile_of(a, w, w.qt0, wave), sK, sV);
    if (w.qt1 >= 0) {
        __syncthreads();
        dq_tile<D, CAUSAL, ROPE>(a, qtile_of(a, w, w.qt1, wave), sK, sV);
    }
}

// Single-wave query-tile launches.  With a group of G query heads per kv head, the multi-wave
// work-groups above put G waves on the 4 SIMDs of a compute unit; when G is not a multiple of 4
// the SIMDs end up with unequal work (at G = 3 the paired dQ launch leaves half of them with one
// wave and half with two).  Here every work-group is one wave, which the dispatcher spreads
// evenly over the SIMDs, longest tiles first; each wave stages its own K/V tiles through a
// single padded LDS buffer, the next tile's rows travelling in registers meanwhile.

// One 32-row K or V tile of a single wave: all chunks into registers, then into LDS (padded
// rows; rows past the end as zeros).
template <int D>
struct TileRegs {
    using C = Cfg<D>;
    f32x4 r[C::CH];
    __device__ __forceinline__ void load(const float *gp, int rs, int tile, int T, int lane) {
        const int c4 = 4 * (lane % C::C4);
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            const int row = min(tile * 32 + i * C::RPC + lane / C::C4, T - 1);
            r[i] = ld4(gp + row * rs + c4);
        }
    }
    __device__ __forceinline__ void store(float *sX, int tile, int T, int lane) const {
        const int c4 = 4 * (lane % C::C4);
        const f32x4 zero{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < C::CH; ++i) {
            const int rr = i * C::RPC + lane / C::C4;
            st4(sX + rr * C::LD + c4, tile * 32 + rr < T ? r[i] : zero);
        }
    }
};

// Keeps the compiler from moving this wave's LDS reads and writes across this point (the
// hardware executes one wave's LDS instructions in order).
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct Work1 {
    int b, g, h, qt;
};

// Work-group -> (batch, kv head, query head, 32-row tile), longest tiles first.  Work-groups go
// round-robin over the 8 XCDs (XCD = blockIdx % 8); when the (batch, kv head) pairs divide
// evenly, each XCD takes its own set of them, so the K/V rows its waves stream are shared
// through its L2.
__device__ __forceinline__ Work1 decode_1w(const Args &a) {
    const int nbg = a.B * a.Hkv;
    int bg, hl, t;
    if (nbg % 8 == 0) {
        const int x = blockIdx.x % 8, y = blockIdx.x / 8;
        const int per = (nbg / 8) * a.G;
        t = y / per;
        const int r = y % per;
        hl = r % a.G;
        bg = x * (nbg / 8) + r / a.G;
    } else {
        const int per = nbg * a.G;
        t = blockIdx.x / per;
        const int r = blockIdx.x % per;
        hl = r % a.G;
        bg = r / a.G;
    }
    Work1 w;
    w.b = bg / a.Hkv;
    w.g = bg % a.Hkv;
    w.h = w.g * a.G + hl;
    w.qt = a.nqt - 1 - t;
    return w;
}

template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
fwd_f32_1w(Args a) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) float sK[32 * Cfg<D>::LD];
    __shared__ __attribute__((aligned(16))) float sV[32 * Cfg<D>::LD];
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const Work1 w = decode_1w(a);
    const int T = a.T, Tk = a.Tk, qo = a.qoff;
    const int r0 = w.qt * 32, qrow = r0 + col, p0 = r0 + qo;
    const float *kg = head_at(a.k, a.L.k, w.b, w.g);
    const float *vg = head_at(a.v, a.L.v, w.b, w.g);
    const int ntiles = CAUSAL ? (min(r0 + 32, T) - 1 + qo) / 32 + 1 : (Tk + 31) / 32;
    // The first K/V tile is requested before the query row, so the two latencies overlap.
    TileRegs<D> tk, tv;
    tk.load(kg, a.L.k.st, 0, Tk, lane);
    tv.load(vg, a.L.v.st, 0, Tk, lane);
    float qr[C::NS];
    load_row_half<D, ROPE>(qr, head_at(a.q, a.L.q, w.b, w.h), a.L.q.st, qrow, T, half, a.qscale,
                           a.rope);
    f32x16 acc[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) acc[dd] = zero16();
    float m = kNegBig, l = 0.f;
    tk.store(sK, 0, Tk, lane);
    tv.store(sV, 0, Tk, lane);
    wave_lds_order();
    for (int j = 0; j < ntiles; ++j) {
        const bool more = j + 1 < ntiles;
        if (more) {  // the next tile's rows travel in registers while this one is used
            tk.load(kg, a.L.k.st, j + 1, Tk, lane);
            tv.load(vg, a.L.v.st, j + 1, Tk, lane);
        }
        f32x16 s = scores_t<D>(sK, qr, col, half);
        fwd_softmax<D, CAUSAL>(s, acc, m, l, j * 32, p0, qrow + qo, Tk, half);
        accum_t<D>(acc, sV, s, col, half);
        if (more) {
            wave_lds_order();
            tk.store(sK, j + 1, Tk, lane);
            tv.store(sV, j + 1, Tk, lane);
            wave_lds_order();
        }
    }
    fwd_store<D>(a, w.b, w.h, qrow, half, acc, m, l);
}

// The dQ pass in single-wave work-groups.  One register tile carries the next rows: V's after
// this tile's two score products (the last reads of V), then K's after dQ's (the last of K).
template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
dq_f32_1w(Args a) {
    using C = Cfg<D>;
    __shared__ __attribute__((aligned(16))) float sK[32 * Cfg<D>::LD];
    __shared__ __attribute__((aligned(16))) float sV[32 * Cfg<D>::LD];
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const Work1 w = decode_1w(a);
    const int T = a.T;
    const int r0 = w.qt * 32, qrow = r0 + col;
    const float *kg = head_at(a.k, a.L.k, w.b, w.g);
    const float *vg = head_at(a.v, a.L.v, w.b, w.g);
    const int ntiles = CAUSAL ? (min(r0 + 32, T) - 1) / 32 + 1 : (T + 31) / 32;
    TileRegs<D> tr;
    tr.load(kg, a.L.k.st, 0, T, lane);
    float qr[C::NS], dor[C::NS], lse2, delta;
    dq_rows<D, ROPE>(a, w.b, w.h, qrow, half, qr, dor, lse2, delta);
    tr.store(sK, 0, T, lane);
    tr.load(vg, a.L.v.st, 0, T, lane);
    f32x16 acc[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) acc[dd] = zero16();
    tr.store(sV, 0, T, lane);
    wave_lds_order();
    for (int j = 0; j < ntiles; ++j) {
        const bool more = j + 1 < ntiles;
        if (more) tr.load(vg, a.L.v.st, j + 1, T, lane);
        f32x16 p = scores_t<D>(sK, qr, col, half);
        f32x16 ds = scores_t<D>(sV, dor, col, half);  // dP^T = V dO^T
        if (more) {
            wave_lds_order();
            tr.store(sV, j + 1, T, lane);
            tr.load(kg, a.L.k.st, j + 1, T, lane);
        }
        dq_dscores<CAUSAL>(p, ds, lse2, delta, j * 32, r0, qrow, T, half);
        accum_t<D>(acc, sK, ds, col, half);  // dQ^T += K^T dS^T
        if (more) {
            wave_lds_order();
            tr.store(sK, j + 1, T, lane);
        }
        wave_lds_order();
    }
    dq_store<D, ROPE>(a, w.b, w.h, qrow, half, acc);
}

// Floats of LDS per dK/dV wave: a query tile and a dO tile (32 padded rows each), lse2, delta.
template <int D>
constexpr int dkdv_wave_floats() { return 2 * 32 * Cfg<D>::LD + 64; }

// Single-pass backward: each wave writes its transposed dS tile ([key][query], rows of kLDT
// floats) over its dO tile, free once the item's dK product has read its last operand; the
// work-group keeps the block's 32 key rows, unscaled, after the waves' areas.
constexpr int kLDT = 36;
static_assert(32 * kLDT <= 32 * Cfg<32>::LD, "the dS^T tile fits in a dO tile");
static_assert(4 * 4 * (2 * 32 * Cfg<128>::LD + 64) + 4 * 32 * Cfg<128>::LD <= 160 * 1024,
              "four D = 128 waves and the key rows fit in 160 KB of LDS");
template <int D>
constexpr int dkdvq_lds_floats(int nw) { return nw * dkdv_wave_floats<D>() + 32 * Cfg<D>::LD; }

// FUSED: the single-pass backward.  Besides dK and dV, every item adds its share of dQ,
// dS K (32 queries x D), into dq with fp32 atomics (dq zeroed beforehand): dS goes through LDS
// as [key][query] so that the product puts the head dimension on the lanes, and each atomic
// instruction then touches two 128-byte lines.  The order of the additions into dq varies from
// run to run, so dq is not bitwise reproducible (dk and dv still are).
template <int D, bool CAUSAL, bool ROPE, bool FUSED = false>
__device__ __forceinline__ void dkdv_block(const Args &a, int b, int g, int kb, float *smem) {
    using C = Cfg<D>;
    constexpr int WF = dkdv_wave_floats<D>();
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const int T = a.T;
    const size_t bg = (size_t)b * a.Hkv + g;
    const int krow = kb * 32 + col;
    // The single-pass backward only runs on contiguous tensors: its layouts follow from the
    // shape, which spares the scalar registers strides would hold through its loop.
    const TLay Lq = FUSED ? contiguous_lay(a.Hq, T, D) : a.L.q;
    const TLay Lk = FUSED ? contiguous_lay(a.Hkv, T, D) : a.L.k;
    const TLay Lv = FUSED ? contiguous_lay(a.Hkv, T, D) : a.L.v;
    const TLay LdO = FUSED ? contiguous_lay(a.Hq, T, D) : a.L.dO;
    const TLay Ldq = FUSED ? contiguous_lay(a.Hq, T, D) : a.L.dq;
    const TLay Ldk = FUSED ? contiguous_lay(a.Hkv, T, D) : a.L.dk;
    const TLay Ldv = FUSED ? contiguous_lay(a.Hkv, T, D) : a.L.dv;

    float kr[C::NS], vr[C::NS];
    load_row_half<D, false>(kr, head_at(a.k, Lk, b, g), Lk.st, krow, T, half, a.qscale,
                            a.rope);
    load_row_half<D, false>(vr, head_at(a.v, Lv, b, g), Lv.st, krow, T, half, 1.0f, a.rope);

    f32x16 dk[C::ND], dv[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) {
        dk[dd] = zero16();
        dv[dd] = zero16();
    }

    float *sQ = smem + wave * WF;
    float *sO = sQ + 32 * C::LD;  // dO tile
    float *sL = sO + 32 * C::LD;  // lse * log2(e) of the tile's rows
    float *sDl = sL + 32;         // delta of the tile's rows
    const int nqb = (T + 31) / 32;
    const int i0 = CAUSAL ? kb : 0;
    const int c4 = 4 * (lane % C::C4);
    float *sT = sO;                          // FUSED: this wave's dS^T tile
    float *sKt = smem + nw * WF;             // FUSED: the block's key rows
    if constexpr (FUSED) {
        for (int idx = threadIdx.x; idx < 32 * C::C4; idx += blockDim.x) {
            const int r = idx / C::C4, cc = 4 * (idx % C::C4);
            const int row = kb * 32 + r;
            st4(sKt + r * C::LD + cc,
                row < T ? ld4(head_at(a.k, Lk, b, g) + row * Lk.st + cc)
                        : f32x4{0.f, 0.f, 0.f, 0.f});
        }
        __syncthreads();
    }

    // The group's (query head, query block) items are dealt round-robin to the waves; each
    // wave stages its own query block and keeps private dK, dV partial sums.
    const int per_head = nqb - i0;
    const int nitems = a.G * per_head;
    for (int it = wave; it < nitems; it += nw) {
        const int hh = it / per_head;
        const int i = i0 + it % per_head;
        const size_t bh = (size_t)b * a.Hq + (size_t)g * a.G + hh;
        const float *qh = head_at(a.q, Lq, b, g * a.G + hh);
        const float *doh = head_at(a.dO, LdO, b, g * a.G + hh);
        // Only this wave reads its staging area, so ordering within the wave is all that is
        // needed between the previous item's reads and these writes.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        {
            f32x4 tq[C::CH], td[C::CH];
#pragma unroll
            for (int ch = 0; ch < C::CH; ++ch) {
                const int row = min(i * 32 + ch * C::RPC + lane / C::C4, T - 1);
                tq[ch] = ld4(qh + row * Lq.st + c4);
                td[ch] = ld4(doh + row * LdO.st + c4);
            }
            float lsev = 0.f, dlv = 0.f;
            const int lrow = i * 32 + (lane & 31);
            if (lrow < T) {
                lsev = a.lse[bh * T + lrow];
                dlv = a.delta[bh * T + lrow];
            }
            const f32x4 zero{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ch = 0; ch < C::CH; ++ch) {
                const int r = ch * C::RPC + lane / C::C4;
                const int row = i * 32 + r;
                st4(sQ + r * C::LD + c4, row < T ? tq[ch] : zero);
                st4(sO + r * C::LD + c4, row < T ? td[ch] : zero);
            }
            if (lane < 32) {
                sL[lane] = lrow < T ? lsev * kLog2e : INFINITY;  // padding rows get P = 0
                sDl[lane] = dlv;
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        __builtin_amdgcn_wave_barrier();

        // S = Q K'^T (rows: queries acc_row(v, half) of the block; column: this lane's key)
        f32x16 p = chain_lds4<C::NS>(sQ + col * C::LD + C::NS * half, kr, zero16());
        // P = exp2(S - lse2): independent of the dP chain below, so the two can overlap.
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 L = ld4(sL + 8 * u + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[4 * u + e] = fast_exp2(p[4 * u + e] - L[e]);
        }
        if (CAUSAL && i == kb) {  // the diagonal block: keys after the query get P = 0
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (col > acc_row(v, half)) p[v] = 0.f;
        }
        // dP = dO V^T
        f32x16 ds = chain_lds4<C::NS>(sO + col * C::LD + C::NS * half, vr, zero16());
        // dV^T += dO^T P  (needs only P, so it can run while dS is formed)
        accum_t<D>(dv, sO, p, col, half);
        // dS = P (dP - delta)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 Dl = ld4(sDl + 8 * u + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) ds[4 * u + e] = p[4 * u + e] * (ds[4 * u + e] - Dl[e]);
        }
        // dK^T += Q^T dS
        accum_t<D>(dk, sQ, ds, col, half);
        if constexpr (FUSED) {
            // dS^T into LDS: lane (key col) writes its 16 queries, four runs of four.
#pragma unroll
            for (int u = 0; u < 4; ++u)
                st4(sT + col * kLDT + 8 * u + 4 * half,
                    f32x4{ds[4 * u], ds[4 * u + 1], ds[4 * u + 2], ds[4 * u + 3]});
            // dQ (32 queries x D) = dS K: step st contracts keys 2 st + half; lane col takes
            // query col of A and head column col (+ 32 dd) of B.
            f32x16 aq[C::ND];
#pragma unroll
            for (int dd = 0; dd < C::ND; ++dd) aq[dd] = zero16();
#pragma unroll
            for (int st = 0; st < 16; ++st) {
                const int key = 2 * st + half;
                const float av = sT[key * kLDT + col];
#pragma unroll
                for (int dd = 0; dd < C::ND; ++dd)
                    aq[dd] = mfma32(av, sKt[key * C::LD + dd * 32 + col], aq[dd]);
            }
            // Register v holds query acc_row(v, half), head column dd * 32 + col.
            float *dqh = head_at(a.dq, Ldq, b, g * a.G + hh);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int qrow = i * 32 + acc_row(v, half);
                if (qrow < T)
#pragma unroll
                    for (int dd = 0; dd < C::ND; ++dd)
                        unsafeAtomicAdd(dqh + qrow * Ldq.st + dd * 32 + col, aq[dd][v] * a.scale);
            }
        }
    }

    // Add the waves' partial dK, dV in LDS (wave order fixed) and write them out.
    __syncthreads();
    {
        float *R = smem + wave * WF;
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int d = dd * 32 + 8 * u + 4 * half;
                st4(R + col * C::LD + d,
                    f32x4{dk[dd][4 * u] * a.scale, dk[dd][4 * u + 1] * a.scale,
                          dk[dd][4 * u + 2] * a.scale, dk[dd][4 * u + 3] * a.scale});
                st4(R + 32 * C::LD + col * C::LD + d,
                    f32x4{dv[dd][4 * u], dv[dd][4 * u + 1], dv[dd][4 * u + 2], dv[dd][4 * u + 3]});
            }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 2 * 32 * C::C4; idx += blockDim.x) {
        const int t = idx / (32 * C::C4);
        const int r = (idx / C::C4) % 32;
        const int cc = 4 * (idx % C::C4);
        f32x4 sum{0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w) sum += ld4(smem + w * WF + t * 32 * C::LD + r * C::LD + cc);
        const int row = kb * 32 + r;
        if (row < T) {
            if (t == 0) {
                if (ROPE) sum = rope4<D>(sum, row, cc, a.rope, true);
                st4(head_at(a.dk, Ldk, b, g) + row * Ldk.st + cc, sum);
            } else {
                st4(head_at(a.dv, Ldv, b, g) + row * Ldv.st + cc, sum);
            }
        }
    }
}

template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : NE_DKDV_WAVES_PER_EU)))
dkdv_f32(Args a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int per = a.B * a.Hkv;
    const int p = blockIdx.x / per;
    const int g = (blockIdx.x % per) % a.Hkv;
    const int b = (blockIdx.x % per) / a.Hkv;
    // Causal: key blocks p and nkb-1-p (the first sees the most queries, the second the fewest).
    dkdv_block<D, CAUSAL, ROPE>(a, b, g, p, smem);
    if (a.paired && a.nkb - 1 - p > p) {
        __syncthreads();
        dkdv_block<D, CAUSAL, ROPE>(a, b, g, a.nkb - 1 - p, smem);
    }
}

// Single-pass backward: as dkdv_f32, plus dQ by atomics.  With RoPE, q and k
// arrive rotated and dq is accumulated in the rotated frame (rotated back afterwards).
template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : NE_DKDVQ_WAVES_PER_EU)))
dkdvq_f32(Args a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int per = a.B * a.Hkv;
    const int p = blockIdx.x / per;
    const int g = (blockIdx.x % per) % a.Hkv;
    const int b = (blockIdx.x % per) / a.Hkv;
    dkdv_block<D, CAUSAL, ROPE, true>(a, b, g, p, smem);
    if (a.paired && a.nkb - 1 - p > p) {
        __syncthreads();
        dkdv_block<D, CAUSAL, ROPE, true>(a, b, g, a.nkb - 1 - p, smem);
    }
}

// delta_i = dO_i . o_i for every row, and dq zeroed, for the single-pass backward.  L = D / 4
// lanes per row, each with 4 columns; the rows' partial sums are added over their L lanes.
template <int D>
__global__ void __launch_bounds__(256) delta_zero_f32(const float *o, const float *dO,
                                                      float *delta, float *dq, long long rows) {
    constexpr int L = D / 4;
    const long long n = rows * L;
    for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx - threadIdx.x < n;
         idx += (long long)gridDim.x * 256) {
        const bool in = idx < n;
        const long long row = idx / L;
        const int c = 4 * (int)(idx % L);
        float x = 0.f;
        if (in) {
            const f32x4 u = ld4(o + row * D + c), w = ld4(dO + row * D + c);
            x = (u[0] * w[0] + u[1] * w[1]) + (u[2] * w[2] + u[3] * w[3]);
        }
#pragma unroll
        for (int m = 1; m < L; m <<= 1) x += __shfl_xor(x, m, 64);
        if (in) {
            if (c == 0) delta[row] = x;
            st4(dq + row * D + c, f32x4{0.f, 0.f, 0.f, 0.f});
        }
    }
}

// RoPE applied once to a whole tensor [BH][T][D] (the position of a row is its t), the angle
// reduced modulo one turn in double precision.  Each thread owns one (position, 4-column chunk):
// it evaluates the two sines and cosines once and applies them to the rows of every (batch,
// head) it visits.  The attention kernels that stream a tensor through LDS many times read this
// rotated copy instead of rotating every staged tile again.
// INV: the transpose R^T (a gradient rotated back), in place when x == y.
// x: rows of head h of batch b at x + b xl.sb + h xl.sh + t xl.st (H heads per batch).
template <int D, bool INV>
__global__ void __launch_bounds__(256) rope_rows_f32(const float *x, float *y, long long nbh, int T,
                                                     RopeTurns rt, TLay xl, int H) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * (D / 4)) return;
    const int t = idx / (D / 4);
    const int c = 4 * (idx % (D / 4));
    float sn[2], cs[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const double turns = (double)t * rt.per_pos[c / 2 + p];
        sincospif(2.0f * (float)(turns - rint(turns)), &sn[p], &cs[p]);
    }
    for (long long bh = blockIdx.y; bh < nbh; bh += gridDim.y) {
        const size_t off = ((size_t)bh * T + t) * D + c;
        const f32x4 v = ld4(x + (bh / H) * xl.sb + (size_t)(bh % H) * xl.sh + t * xl.st + c);
        if (INV)
            st4(y + off, f32x4{v[0] * cs[0] + v[1] * sn[0], v[1] * cs[0] - v[0] * sn[0],
                               v[2] * cs[1] + v[3] * sn[1], v[3] * cs[1] - v[2] * sn[1]});
        else
            st4(y + off, f32x4{v[0] * cs[0] - v[1] * sn[0], v[0] * sn[0] + v[1] * cs[0],
                               v[2] * cs[1] - v[3] * sn[1], v[2] * sn[1] + v[3] * cs[1]});
    }
}

Args make_args(const Shape &s) {
    Args a{};
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.T = s.T;
    a.Tk = s.Tk > 0 ? s.Tk : s.T;
    a.qoff = a.Tk - s.T;
    a.G = s.G;
    a.scale = (float)(1.0 / sqrt((double)s.D));
    a.qscale = (float)(1.4426950408889634 / sqrt((double)s.D));
    a.rope.on = s.rope_base > 0.f;
    a.rope.log2_base = a.rope.on ? log2((double)s.rope_base) : 0.0;
    if (s.lay) {
        a.L = *s.lay;
    } else {
        const TLay lq = contiguous_lay(s.Hq, s.T, s.D), lk = contiguous_lay(s.Hkv, a.Tk, s.D);
        const TLay lkb = contiguous_lay(s.Hkv, s.T, s.D);
        a.L = TLays{lq, lk, lk, lq, lq, lq, lkb, lkb};
    }
    return a;
}

#define NE_PICK(KERNEL)                                                                      \
    template <int D>                                                                         \
    const void *pick_##KERNEL(bool causal, bool rope) {                                      \
        if (causal) return rope ? (const void *)KERNEL<D, true, true> : (const void *)KERNEL<D, true, false>; \
        return rope ? (const void *)KERNEL<D, false, true> : (const void *)KERNEL<D, false, false>; \
    }
NE_PICK(fwd_f32)
NE_PICK(dq_f32)
NE_PICK(dkdv_f32)
NE_PICK(dkdvq_f32)
NE_PICK(fwd_f32_1w)
NE_PICK(dq_f32_1w)
#undef NE_PICK

hipError_t launch(const void *fn, long long blocks, int threads, size_t lds, hipStream_t st, Args &a) {
    void *params[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), params, lds, st);
}

// Launch-order distance of mirrored tiles for an unpaired causal launch of `fn` (see
// decode_qwork): compute units / work-groups per tile index, when every work-group of the
// launch is resident at once (then the order decides which work shares a unit) and the shape
// divides evenly; otherwise 0, longest tile first, which suits launches of several rounds.
// Compute units of the current device and resident work-groups of `fn` per compute unit,
// queried once per (device, kernel, work-group size) and kept for the process.
bool residency(const void *fn, int threads, int &cus, int &per_cu) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, int>, std::pair<int, int>> seen;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    const auto key = std::make_tuple(dev, fn, threads);
    {
        std::lock_guard<std::mutex> lk(mu);
        const auto it = seen.find(key);
        if (it != seen.end()) {
            cus = it->second.first;
            per_cu = it->second.second;
            return true;
        }
    }
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, 0) != hipSuccess)
        return false;
    std::lock_guard<std::mutex> lk(mu);
    seen[key] = {cus, per_cu};
    return true;
}

int mirror_step(const Shape &s, const QTileGeom &g, const void *fn) {
    if (!s.causal || g.paired) return 0;
    int cus = 0, per_cu = 0;
    if (!residency(fn, 64 * g.nwaves, cus, per_cu)) return 0;
    if (g.nblocks > (long long)per_cu * cus) return 0;
    const long long per = (long long)s.B * s.Hkv * (s.G / g.hpw);
    if (per <= 0 || cus % per != 0) return 0;
    const int ms = (int)(cus / per);
    return g.nqt % (2 * ms) == 0 ? ms : 0;
}

}  // namespace

QTileGeom qtile_geometry(const Shape &s, bool pair) {
    QTileGeom g{};
    g.hpw = 1;
    // At D = 128 a wave needs more than 256 registers, so a work-group holds at most 4 waves
    // (one per SIMD of a compute unit).
    for (int d = s.D == 128 ? 4 : 8; d >= 1; --d)
        if (s.G % d == 0) {
            g.hpw = d;
            break;
        }
    g.rb = g.hpw == 1 ? 2 : 1;
    g.nwaves = g.hpw * g.rb;
    g.rows = 32 * g.rb;
    g.nqt = (s.T + g.rows - 1) / g.rows;
    g.paired = pair ? 1 : 0;
    g.nblocks = (long long)s.B * s.Hkv * (s.G / g.hpw) * (g.paired ? (g.nqt + 1) / 2 : g.nqt);
    return g;
}

KBlockGeom kblock_geometry(const Shape &s, bool pair) {
    KBlockGeom g{};
    g.nwaves = 4;
    g.nkb = (s.T + 31) / 32;
    g.paired = pair ? 1 : 0;
    g.nblocks = (long long)s.B * s.Hkv * (g.paired ? (g.nkb + 1) / 2 : g.nkb);
    return g;
}

// Single-wave query-tile work-groups (fwd_f32_1w, dq_f32_1w) for causal attention over the
// sequence itself (tiles of unequal length) at head sizes up to 64, when the group of query
// heads sharing a kv head does not fill the 4 SIMDs of a compute unit evenly.  A prefill chunk's
// tiles all see the whole history, and there the multi-wave groups, which share each K/V tile
// between the group's heads, measured faster.
long long single_wave_blocks(const Shape &s) {
    if (!s.causal || (s.Tk != 0 && s.Tk != s.T) || s.D > 64 || s.G % 4 == 0) return 0;
    const long long n = (long long)s.B * s.Hq * ((s.T + 31) / 32);
    return n <= 0x7fffffffLL ? n : 0;
}

hipError_t launch_fwd_f32(const Shape &s, const float *q, const float *k, const float *v, float *o,
                          float *lse, hipStream_t st) {
    Args a = make_args(s);
    a.q = q;
    a.k = k;
    a.v = v;
    a.out_o = o;
    a.out_lse = lse;
    const QTileGeom g = qtile_geometry(s, s.causal && kPairF32.fwd != 0 ? 1 : 0);
    a.hpw = g.hpw;
    a.rb = g.rb;
    a.nqt = g.nqt;
    a.paired = g.paired;
    const bool causal = s.causal != 0, rope = a.rope.on != 0;
    if (const long long n1 = single_wave_blocks(s)) {
        a.nqt = (s.T + 31) / 32;
        const void *f1 = s.D == 64 ? pick_fwd_f32_1w<64>(causal, rope) : pick_fwd_f32_1w<32>(causal, rope);
        return launch(f1, n1, 64, 0, st, a);
    }
    const void *fn = s.D == 128  ? pick_fwd_f32<128>(causal, rope)
                     : s.D == 64 ? pick_fwd_f32<64>(causal, rope)
                                 : pick_fwd_f32<32>(causal, rope);
    a.mstep = mirror_step(s, g, fn);
    return launch(fn, g.nblocks, 64 * g.nwaves, 0, st, a);
}

hipError_t launch_dq_f32(const Shape &s, const float *q, const float *k, const float *v,
                         const float *o, const float *lse, const float *dO, float *dq,
                         float *delta, float *qrot, hipStream_t st) {
    Args a = make_args(s);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.dO = dO;
    a.dq = dq;
    a.delta = delta;
    a.qrot = qrot;
    const QTileGeom g = qtile_geometry(s, s.causal && kPairF32.dq != 0);
    a.hpw = g.hpw;
    a.rb = g.rb;
    a.nqt = g.nqt;
    a.paired = g.paired;
    const bool causal = s.causal != 0, rope = a.rope.on != 0;
    if (const long long n1 = single_wave_blocks(s)) {
        a.nqt = (s.T + 31) / 32;
        const void *f1 = s.D == 64 ? pick_dq_f32_1w<64>(causal, rope) : pick_dq_f32_1w<32>(causal, rope);
        return launch(f1, n1, 64, 0, st, a);
    }
    const void *fn = s.D == 128  ? pick_dq_f32<128>(causal, rope)
                     : s.D == 64 ? pick_dq_f32<64>(causal, rope)
                                 : pick_dq_f32<32>(causal, rope);
    return launch(fn, g.nblocks, 64 * g.nwaves, 0, st, a);
}

hipError_t launch_dkdv_f32(const Shape &s, const float *q, const float *k, const float *v,
                           const float *lse, const float *dO, const float *delta, float *dk,
                           float *dv, hipStream_t st) {
    Args a = make_args(s);
    a.q = q;
    a.k = k;
    a.v = v;
    a.lse = lse;
    a.dO = dO;
    a.dk = dk;
    a.dv = dv;
    a.delta = const_cast<float *>(delta);  // read only in this pass
    const KBlockGeom g = kblock_geometry(s, s.causal && kPairF32.dkdv != 0);
    a.paired = g.paired;
    a.nkb = g.nkb;
    const bool causal = s.causal != 0, rope = a.rope.on != 0;
    const int wf = s.D == 128 ? dkdv_wave_floats<128>()
                   : s.D == 64 ? dkdv_wave_floats<64>()
                               : dkdv_wave_floats<32>();
    const size_t lds = (size_t)g.nwaves * wf * sizeof(float);
    const void *fn = s.D == 128  ? pick_dkdv_f32<128>(causal, rope)
                     : s.D == 64 ? pick_dkdv_f32<64>(causal, rope)
                                 : pick_dkdv_f32<32>(causal, rope);
    return launch(fn, g.nblocks, 64 * g.nwaves, lds, st, a);
}

hipError_t launch_bwd_fused_f32(const Shape &s, const float *q, const float *k, const float *v,
                                const float *o, const float *lse, const float *dO, float *dq,
                                float *dk, float *dv, float *delta, float *qrot, float *krot,
                                hipStream_t st) {
    // D = 128: 153 KB of LDS per work-group, one per compute unit.
    if (s.D != 32 && s.D != 64 && s.D != 128) return hipErrorInvalidValue;
    const bool rope = s.rope_base > 0.f;
    const long long rows = (long long)s.B * s.Hq * s.T;
    if (rope) {  // q and k rotated once into the workspace
        if (!qrot || !krot) return hipErrorInvalidValue;
        hipError_t e = launch_rope_f32(s, q, qrot, rows, st, false);
        if (e == hipSuccess) e = launch_rope_f32(s, k, krot, (long long)s.B * s.Hkv * s.T, st, false);
        if (e != hipSuccess) return e;
        q = qrot;
        k = krot;
    }
    {
        const long long thr = rows * (s.D / 4);
        const unsigned grid = (unsigned)std::min<long long>((thr + 255) / 256, 1LL << 20);
        const void *fn = s.D == 128  ? (const void *)delta_zero_f32<128>
                         : s.D == 64 ? (const void *)delta_zero_f32<64>
                                     : (const void *)delta_zero_f32<32>;
        long long r = rows;
        void *params[] = {&o, &dO, &delta, &dq, &r};
        const hipError_t e = hipLaunchKernel(fn, dim3(grid), dim3(256), params, 0, st);
        if (e != hipSuccess) return e;
    }
    Args a = make_args(s);
    a.q = q;
    a.k = k;
    a.v = v;
    a.lse = lse;
    a.dO = dO;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    const KBlockGeom g = kblock_geometry(s, s.causal && kPairF32.dkdv != 0);
    a.paired = g.paired;
    a.nkb = g.nkb;
    const bool causal = s.causal != 0;
    const int lf = s.D == 128  ? dkdvq_lds_floats<128>(g.nwaves)
                   : s.D == 64 ? dkdvq_lds_floats<64>(g.nwaves)
                               : dkdvq_lds_floats<32>(g.nwaves);
    const void *fn = s.D == 128  ? pick_dkdvq_f32<128>(causal, rope)
                     : s.D == 64 ? pick_dkdvq_f32<64>(causal, rope)
                                 : pick_dkdvq_f32<32>(causal, rope);
    hipError_t e = launch(fn, g.nblocks, 64 * g.nwaves, (size_t)lf * sizeof(float), st, a);
    if (e == hipSuccess && rope) e = launch_rope_f32(s, dq, dq, rows, st, true);  // dq = R^T dq'
    return e;
}

hipError_t launch_rope_f32(const Shape &s, const float *x, float *y, long long rows,
                           hipStream_t st, bool inv, const TLay *xl_, int H) {
    RopeTurns rt = rope_turns(s);
    long long nbh = rows / s.T;
    int T = s.T;
    TLay xl = xl_ ? *xl_ : contiguous_lay(1, T, s.D);
    if (!xl_) H = 1;
    const long long per_pos = (long long)T * (s.D / 4);
    const unsigned gx = (unsigned)((per_pos + 255) / 256);
    const long long gy = std::max(1LL, std::min(nbh, std::max(nbh / 8, 2048LL / (long long)gx)));
    const void *fn = inv ? (s.D == 128  ? (const void *)rope_rows_f32<128, true>
                            : s.D == 64 ? (const void *)rope_rows_f32<64, true>
                                        : (const void *)rope_rows_f32<32, true>)
                         : (s.D == 128  ? (const void *)rope_rows_f32<128, false>
                            : s.D == 64 ? (const void *)rope_rows_f32<64, false>
                                        : (const void *)rope_rows_f32<32, false>);
    void *params[] = {&x, &y, &nbh, &T, &rt, &xl, &H};
    return hipLaunchKernel(fn, dim3(gx, (unsigned)std::min(gy, 65535LL)), dim3(256), params, 0, st);
}

}  // namespace ne
