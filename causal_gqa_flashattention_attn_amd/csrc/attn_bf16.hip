// attn_bf16.hip -- bfloat16 causal grouped-query FlashAttention for gfx950 with an optional fused
// RoPE prologue, forward and backward.  Inputs and outputs are bf16; lse and delta are fp32; all
// accumulation is fp32 (v_mfma_f32_32x32x16_bf16).
//
// Same method and decomposition as the fp32 kernels (exact softmax attention, online softmax,
// no T x T matrix: "nanoeuler: un LLM estilo GPT-2 construido desde cero en C y CUDA", second
// paragraph; causal upper triangle skipped: "NanoEuler: a GPT-2 hand-built in pure C/CUDA"
// (openai-hub), implementation details; grouped-query heads and RoPE on queries and keys:
// README translations, section "Architecture").
//
// RoPE: the pair (x[2i], x[2i+1]) at position t is rotated by t * base^(-2i/D) in fp32: q when a
// wave loads its rows (the dQ pass keeps its rotated rows in the workspace for the dK/dV pass),
// k once by a pre-pass into the workspace (rope_rows_bf16), since the K/V tiles reach LDS by
// direct copies; the rotated values are rounded to bf16 before they enter the matrix cores.
// The angle is formed and reduced modulo one turn in double precision (per-pair turn rates are
// evaluated on the host in double), so it is exact to float rounding at every position.  dq and
// dk are rotated back (transpose) in fp32 before rounding, so they are gradients with respect to
// the caller's un-rotated q and k.
//
// Layout in LDS: K, V, Q and dO tiles stay row-major as in HBM (16-byte chunks XOR-swizzled per
// row).  Products that contract over the tile's rows (P V, dS K, dO^T P, Q^T dS) read their
// operand with the transposing LDS load, so no tile is ever transposed in memory.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "attn_device.hpp"
#include "attn_kernels.hpp"

#ifndef NE_BF16_FWD_WAVES_PER_EU
#define NE_BF16_FWD_WAVES_PER_EU 3
#endif
#ifndef NE_BF16_DQ_WAVES_PER_EU
#define NE_BF16_DQ_WAVES_PER_EU 3
#endif
// Keys per K/V tile at D = 64.  32 (a 24 KB ring, room for a fourth wave per SIMD in the
// forward) measured no faster than 64 at T = 1024, and the dQ pass slower.
#ifndef NE_BF16_BN_D64
#define NE_BF16_BN_D64 64
#endif
#ifndef NE_BF16_DKDV_WAVES_PER_EU
#define NE_BF16_DKDV_WAVES_PER_EU 2
#endif
// Stages of the forward's K/V ring at D <= 64.  Two (32 KB at D = 64) let four work-groups of
// four waves share a compute unit, which the forward's registers allow; with each tile's copies
// issued as soon as the barrier frees its stage, they still overlap a whole tile of work.  This
// measured 5-7 % faster than three stages (48 KB, three work-groups) at B 16, Hq 16, T 1024.
#ifndef NE_BF16_FWD_NST
#define NE_BF16_FWD_NST 2
#endif

namespace ne {

namespace {

template <int D>
struct CfgB {
    static constexpr int KS = D / 16;   // MFMA k-steps of a contraction over D
    static constexpr int ND = D / 32;   // 32-wide blocks of D
    static constexpr int NCH = D / 8;   // 16-byte chunks per row
    static constexpr int RB = 2 * D;    // bytes per tile row
    // Keys per staged K/V tile: two 32-key sub-blocks, one at D = 128 (so that the three-stage
    // ring, 48 KB, leaves room for two work-groups per compute unit).
    static constexpr int BN = D == 128 ? 32 : D == 64 ? NE_BF16_BN_D64 : 64;
    static constexpr int NSB = BN / 32;  // 32-key sub-blocks per tile
};

struct ArgsB {
    const __bf16 *q, *k, *v, *o, *dO;
    const float *lse;
    __bf16 *out_o, *dq, *dk, *dv;
    __bf16 *qrot;   // dQ pass with RoPE: rotated query rows, written for the dK/dV pass
    float *out_lse, *delta;
    int B, Hq, Hkv, T, G;
    int hpw, rb, nqt;
    int paired;     // work-groups take mirrored pairs of tiles or key blocks
    int nkb;        // key blocks per head (dK/dV)
    int Tk, qoff;   // forward: key length and position of query row 0 (Tk = T, 0 usually)
    float qscale;   // scale * log2(e)
    float scale;    // 1 / sqrt(D)
    RopeTurns rt;        // turns per position of each RoPE pair (double)
    double rope_shift4;  // base^(-8/D): per_pos[i + 4] / per_pos[i]
    double rope_shift2;  // base^(-4/D): per_pos[i + 2] / per_pos[i]
    double rope_lb;      // log2(base)
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf2f(__bf16 x) { return (float)x; }

// RoPE angles in turns.  Pair i of a row at position t turns by t * per_pos[i], per_pos[i] =
// base^(-2i/D) / (2 pi) evaluated on the host in double.  A lane's pairs are i0 + p for a
// compile-time i0, offset by a whole number of pairs j on the second half-wave; since
// per_pos[i0 + j + p] = per_pos[i0 + p] * base^(-2j/D), the lane folds that factor into its
// position once (tpos, double) and every angle is tpos times a scalar rate, formed and reduced
// modulo one turn in double, then rounded once to float: exact to float rounding at any position.
__device__ __forceinline__ float rope_frac(double tpos, double rate) {
    const double turns = tpos * rate;
    return (float)(turns - rint(turns));
}

// Rotates the pairs (x[2p], x[2p+1]), p < N/2, by tpos * rt.per_pos[i0 + p] turns (the
// transpose when inv).  The reduced angle goes to the hardware sine/cosine (input in turns).
template <int N>
__device__ __forceinline__ void rope_rotate(float (&x)[N], double tpos, const RopeTurns &rt,
                                            int i0, bool inv) {
#pragma unroll
    for (int p = 0; p < N / 2; ++p) {
        const float fr = rope_frac(tpos, rt.per_pos[i0 + p]);
        const float sn = __builtin_amdgcn_sinf(fr), cs = __builtin_amdgcn_cosf(fr);
        const float a = x[2 * p], b = x[2 * p + 1];
        if (!inv) {
            x[2 * p] = a * cs - b * sn;
            x[2 * p + 1] = a * sn + b * cs;
        } else {
            x[2 * p] = a * cs + b * sn;
            x[2 * p + 1] = b * cs - a * sn;
        }
    }
}

__device__ __forceinline__ void unpack8(const bf16x8 &v, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = bf2f(v[i]);
}
__device__ __forceinline__ bf16x8 round8(const float (&x)[8]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[i];
    return r;
}

// 8 elements (row, c0 .. c0+7) from HBM, rotated when ROPE (rates of the 4 pairs given).
// (With ROPE: tpos, rt and i0 give the angles of its four pairs, as for rope_rotate.)
template <int D, bool ROPE>
__device__ __forceinline__ bf16x8 load_row8(const __bf16 *base, int row, int T, int c0,
                                            double tpos, const RopeTurns &rt, int i0) {
    const int r = min(row, T - 1);
    bf16x8 v = *reinterpret_cast<const bf16x8 *>(base + (size_t)r * D + c0);
    if (ROPE) {
        float x[8];
        unpack8(v, x);
        rope_rotate<8>(x, tpos, rt, i0, false);
        v = round8(x);
    }
    return v;
}

// Stores four fp32 values (row, c0 .. c0+3) as bf16, optionally rotating them back first (the
// two pairs' angles from tpos, rt and i0, as for rope_rotate).
template <int D, bool ROPE_INV>
__device__ __forceinline__ void store_row4(__bf16 *base, int row, int c0, float (&x)[4],
                                           double tpos, const RopeTurns &rt, int i0) {
    if (ROPE_INV) rope_rotate<4>(x, tpos, rt, i0, true);
    bf16x4 r{(__bf16)x[0], (__bf16)x[1], (__bf16)x[2], (__bf16)x[3]};
    *reinterpret_cast<bf16x4 *>(base + (size_t)row * D + c0) = r;
}

struct QTileB {
    int b, g, h, qt, r0;
};

// Work-group -> (batch, kv head, head chunk) and its query tiles (mirrored pairs when causal).
struct QWorkB {
    int b, g, hc, qt0, qt1;  // qt1 < 0: a single tile
};

__device__ __forceinline__ QWorkB decode_qwork_b(const ArgsB &a) {
    const int nhc = a.G / a.hpw;
    const int per = a.B * a.Hkv * nhc;
    const int t = blockIdx.x / per;
    int r = blockIdx.x % per;
    QWorkB w;
    w.hc = r % nhc;
    r /= nhc;
    w.g = r % a.Hkv;
    w.b = r / a.Hkv;
    // Longest tile first under a causal mask (the order is immaterial otherwise).
    w.qt0 = a.nqt - 1 - t;
    w.qt1 = a.paired && t < w.qt0 ? t : -1;
    return w;
}

__device__ __forceinline__ QTileB qtile_of_b(const ArgsB &a, const QWorkB &w, int qt, int wave) {
    QTileB c;
    c.b = w.b;
    c.g = w.g;
    c.qt = qt;
    c.h = w.g * a.G + w.hc * a.hpw + wave / a.rb;
    c.r0 = qt * 32 * a.rb + (wave % a.rb) * 32;
    return c;
}

// K and V tiles of BN rows staged by direct global -> LDS copies into a ring of NST stages
// (stage = K tile then V tile, rows in the swizzled layout of tile_off).  A stage is NPC 1 KB
// pieces; one wave-wide copy fills one piece, and lane l fills the 16-byte slot l of it, so a
// lane loads the logical chunk that the swizzle places in its slot (the swizzle is an XOR, its
// own inverse).  Within a tensor tile, piece q covers rows q * RPP .. + RPP - 1 and the lane's
// row is q * RPP + lane / NCH; the lane's column offset only depends on the parity of q.  The
// copies go through buffer resources on the head's K and V, so the address of a whole tile's
// piece is a per-lane offset plus a uniform one.  Wave w copies pieces w, w + nw, ...; a wave with a
// shorter share copies its first piece again, so every wave issues lpw copies per tile and can
// wait on a fixed count.  Rows past the end read row T - 1: those keys are masked, so only
// finiteness matters.
template <int D, int NSTAGES = 3>
struct KVRingB {
    using C = CfgB<D>;
    static constexpr int NST = NSTAGES;           // stages
    static constexpr int PD = NST - 1;            // tiles requested ahead of the one in use
    static constexpr int TB = C::BN * C::RB;      // bytes of one K (or V) tile
    static constexpr int SB = 2 * TB;             // bytes of one stage
    static constexpr int PPT = TB / 1024;         // pieces per tensor tile
    static constexpr int NPC = 2 * PPT;           // pieces per stage
    static constexpr int RPP = 1024 / C::RB;      // tile rows per piece
    static constexpr int MAXL = NPC / 2;          // pieces per wave (query-tile groups: >= 2 waves)
    int wave, nw, lpw;  // wave-uniform
    int lrow;           // lane / NCH: the lane's row within a piece
    int chb;            // byte offset of the lane's 16 bytes within its row, even pieces
    int off0, off1;     // the lane's offset within an even / odd piece (D <= 64)
    int offw;           // ... within piece number `wave`
    static constexpr int PX = 16 * swizzle_piece_xor<D>(1);  // D <= 64, odd pieces: offset ^ PX
    static_assert(PPT <= 4 || PPT % 4 == 0, "piece runs are whole groups of four pieces");
    static constexpr int MAXRUN = D == 128 ? 8 : 4;  // longest run of pieces per wave and tile

    __device__ __forceinline__ void init(int wave_, int nw_, int lane) {
        wave = wave_;
        nw = nw_;
        lpw = (NPC + nw - 1) / nw;
        lrow = lane / C::NCH;
        chb = 16 * chunk_swizzle<D>(lrow, lane % C::NCH);
        off0 = lrow * C::RB + chb;
        off1 = off0 ^ PX;
        if constexpr (D == 128) {
            // Run of ppw pieces from p0 = wave ppw: piece p0 + j permutes by (p0 & 3) ^ (j & 3)
            // (ppw is 2, 4 or 8, so p0 & 3 is 0 or 2 and never carries into j).
            const int ppw = PPT % nw_ == 0 ? PPT / nw_ : 1;
            offw = off0 ^ (16 * swizzle_piece_xor<D>(wave * ppw));
        } else {
            offw = (wave & 1) ? off1 : off0;
        }
    }
    // Starts the copies of tile `tile` into `stage`.  Addresses are offsets within the head
    // (kg, vg), split into a per-lane part and a wave-uniform part.
    __device__ __forceinline__ void issue(const __bf16 *kg, const __bf16 *vg, int tile, int T,
                                          unsigned char *stage) const {
        const unsigned bytes = (unsigned)T * C::RB;
        const buf_rsrc_t rk = raw_rsrc(kg, bytes), rv = raw_rsrc(vg, bytes);
        const uint32_t sa = opaque_lds_addr(stage);
        if ((tile + 1) * C::BN <= T && PPT % nw == 0 && PPT / nw <= MAXRUN) {
            // No row past the end, and nw divides the pieces of a tensor tile: wave w copies
            // the ppw consecutive pieces w ppw .. of K and of V (the same count, lpw, as below).
            // Consecutive pieces are 1 KB apart in the tensor and in the stage alike: an
            // instruction offset (below 4 KB; groups of four pieces step the uniform offsets).
            // D <= 64: with ppw even, piece parity is that of j; with ppw = 1, of w.  D = 128:
            // the run's first piece sets offw (init).
            const int ppw = PPT / nw;
            const int p0 = wave * ppw;
            const unsigned soff = (unsigned)(tile * TB + p0 * 1024);
            const uint32_t dk = sa + p0 * 1024, dv = sa + TB + p0 * 1024;
            // All K pieces, then all V pieces: a run shares one LDS base (the M0 register),
            // and the scores need K first.
            static_for<2>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                static_for<(PPT < MAXRUN ? PPT : MAXRUN)>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    if (j < ppw) {
                        unsigned vo;
                        if constexpr (D == 128)
                            vo = (unsigned)(offw ^ (16 * swizzle_piece_xor<D>(j)));
                        else
                            vo = (unsigned)(j == 0 ? (ppw == 1 ? offw : off0) : (j & 1) ? off1 : off0);
                        constexpr unsigned hi = (unsigned)(j / 4) * 4096u;
                        dma16_buf_imm_at<(j % 4) * 1024>(t ? rv : rk, vo, soff + hi, (t ? dv : dk) + hi);
                    }
                });
            });
            return;
        }
        // Rows past the end read row T - 1 instead.
#pragma unroll
        for (int i = 0; i < MAXL; ++i)
            if (i < lpw) {
                int pc = wave + i * nw;
                if (pc >= NPC) pc = wave;
                const bool isv = pc >= PPT;
                const int q = isv ? pc - PPT : pc;
                const int r = min(tile * C::BN + q * RPP + lrow, T - 1);
                dma16_buf_at(isv ? rv : rk,
                             (unsigned)((r * C::RB + chb) ^ (16 * swizzle_piece_xor<D>(q))), 0u,
                             sa + pc * 1024);
            }
    }
};

// This lane's query (or key) row as KS operand chunks: chunk s holds columns 16 s + 8 half ..+7.
// With ROPE the row is rotated: chunk s holds pairs 8 s + 4 half + p (p < 4), so the second
// half-wave's pairs are 4 further on (rope_shift4 = base^(-8/D) folded into its position).
template <int D, bool ROPE>
__device__ __forceinline__ void load_operand_row(bf16x8 (&dst)[CfgB<D>::KS], const __bf16 *base,
                                                 int row, int T, int half, const ArgsB &a) {
    const double tpos = ROPE ? (double)row * (half ? a.rope_shift4 : 1.0) : 0.0;
#pragma unroll
    for (int s = 0; s < CfgB<D>::KS; ++s)
        dst[s] = load_row8<D, ROPE>(base, row, T, 16 * s + 8 * half, tpos, a.rt, 8 * s);
}

// The rotation of a row loaded raw by load_operand_row<D, false> (chunks as there), for callers
// that request other reads before the rotation waits for these.
template <int D>
__device__ __forceinline__ void rotate_operand_row(bf16x8 (&v)[CfgB<D>::KS], int row, int half,
                                                   const ArgsB &a) {
    const double tpos = (double)row * (half ? a.rope_shift4 : 1.0);
#pragma unroll
    for (int s = 0; s < CfgB<D>::KS; ++s) {
        float x[8];
        unpack8(v[s], x);
        rope_rotate<8>(x, tpos, a.rt, 8 * s, false);
        v[s] = round8(x);
    }
}

// S^T block (32 keys of the tile from row r0 x this wave's 32 rows) = M_tile x X^T.
template <int D>
__device__ __forceinline__ f32x16 block_scores(const unsigned char *tile, int r0,
                                               const bf16x8 (&x)[CfgB<D>::KS], int col, int half) {
    f32x16 s = zero16();
#pragma unroll
    for (int st = 0; st < CfgB<D>::KS; ++st)
        s = mfma32_bf16(tile_read8<D>(tile, r0 + col, 16 * st + 8 * half), x[st], s);
    return s;
}

// A transposed operand M_tile[r0 .. r0+31]^T (D x 32) in flight: read with lds_read_tr4 for
// tiles that LDS copies may be filling concurrently, so it can be requested well before use.
template <int D>
struct TrOperand {
    bf16x4 lo[2][CfgB<D>::ND], hi[2][CfgB<D>::ND];
    static constexpr int NREAD = 4 * CfgB<D>::ND;  // LDS reads per operand
};

// Lane addresses of a TrOperand read from a tile at offset 0 of a region: [h][dd] for the rows
// 8 h .. of each 16-row group and the columns 32 dd ..
template <int D>
struct TrAddr {
    uint32_t a[2][CfgB<D>::ND];
    __device__ __forceinline__ void init(const unsigned char *region, int lane) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int dd = 0; dd < CfgB<D>::ND; ++dd) a[h][dd] = tr4_lane_addr<D>(region, 8 * h, 32 * dd, lane);
    }
};

// Issues the reads of the operand M^T for the 32-row tile at byte offset OFF of the region, in
// the order accum_tr's waits count on: for s2 = 0 then 1, for each 32-column block dd, the
// reads of rows 8 h .. (h = 0, 1) of the 16-row group s2.
template <int D, int OFF>
__device__ __forceinline__ void issue_tr_at(TrOperand<D> &op, const TrAddr<D> &ad) {
    constexpr int G16 = 16 * CfgB<D>::RB;  // bytes of 16 rows
#pragma unroll
    for (int dd = 0; dd < CfgB<D>::ND; ++dd) {
        op.lo[0][dd] = lds_read_tr4<OFF>(ad.a[0][dd]);
        op.hi[0][dd] = lds_read_tr4<OFF>(ad.a[1][dd]);
    }
#pragma unroll
    for (int dd = 0; dd < CfgB<D>::ND; ++dd) {
        op.lo[1][dd] = lds_read_tr4<OFF + G16>(ad.a[0][dd]);
        op.hi[1][dd] = lds_read_tr4<OFF + G16>(ad.a[1][dd]);
    }
}

// acc (D x 32, transposed) += op x X, X given as its two bf16 operand halves.  LATER: how many
// transposed reads were issued after op's; each product waits only for its own two reads.
template <int D, int LATER>
__device__ __forceinline__ void accum_tr(f32x16 (&acc)[CfgB<D>::ND], TrOperand<D> &op,
                                         const bf16x8 (&xb)[2]) {
    // The reads were issued in the order (s2, dd), lo then hi: after the pair (s2, dd) came
    // 2 (ND - 1 - dd) reads of the same s2, and 2 ND more when s2 = 0.
    constexpr int ND = CfgB<D>::ND;
    static_for<2>([&](auto s2c) {
        constexpr int s2 = decltype(s2c)::value;
        static_for<ND>([&](auto ddc) {
            constexpr int dd = decltype(ddc)::value;
            lds_wait_n<LATER + 2 * (ND - 1 - dd) + (s2 == 0 ? 2 * ND : 0)>(op.lo[s2][dd], op.hi[s2][dd]);
            acc[dd] = mfma32_bf16(join8(op.lo[s2][dd], op.hi[s2][dd]), xb[s2], acc[dd]);
        });
    });
}

// Online-softmax state of a wave's 32 query rows in the forward: O^T accumulator, reference
// maximum m (base 2, scaled) and four partial sums of the bf16 probabilities.
template <int D>
struct FwdState {
    f32x16 acc[CfgB<D>::ND];
    float m;
    float mthr;  // (m + 8) / qscale: raw scores above it make m move
    float l4[4];
};

// One 32-key half of a tile in the forward (keys kb0 .. kb0 + 31, tile rows rt .. rt + 31).  The
// halves are processed one after the other, each with its own online-softmax update, so only
// one 32 x 32 score block is live: that keeps the kernel within the registers of two waves per
// SIMD with room to spare, which measured faster than one wider update per 64 keys.
// OFFV: byte offset of the half's V rows from the ring base, for which `tra` holds the lane
// addresses.  The transposed V reads are issued as soon as the scores are requested, and in a
// form the compiler does not track, so it neither waits for the copies of later tiles still in
// flight into other stages before them nor delays them behind the exponentials.
template <int D, bool CAUSAL, int OFFV>
__device__ __forceinline__ void fwd_half(const ArgsB &a, FwdState<D> &st, const unsigned char *sK,
                                         const TrAddr<D> &tra, int rt, int kb0, int r0, int T,
                                         const bf16x8 (&qv)[CfgB<D>::KS], int lane, int li) {
    const int half = lane >> 5, col = lane & 31;
    const int qrow = r0 + col;
    f32x16 s = block_scores<D>(sK, rt, qv, col, half);
    TrOperand<D> tv;
    issue_tr_at<D, OFFV>(tv, tra);
    if ((CAUSAL && kb0 + 31 > r0) || kb0 + 32 > T) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int key = kb0 + acc_row(v, half);
            if ((CAUSAL && key > qrow) || key >= T) s[v] = -INFINITY;
        }
    }
    // Maximum of this lane's 16 scores, a tree of three-input maxima.  (IEEE maximum: unlike
    // fmaxf it needs no quieting of its inputs first, and -inf from the mask is neutral.)
    const auto mx3 = [](float x, float y, float z) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(x, y), z);
    };
    const float lmax = __builtin_elementwise_maximum(
        mx3(mx3(s[0], s[1], s[2]), mx3(s[3], s[4], s[5]), mx3(s[6], s[7], s[8])),
        mx3(mx3(s[9], s[10], s[11]), mx3(s[12], s[13], s[14]), s[15]));
    // The reference maximum m only moves when some row's maximum exceeds it by more than 2^8:
    // probabilities up to 256 are exact enough in fp32 sums and bf16 operands, and most steps
    // then skip the rescale of l and O entirely.  The test is per lane, on raw scores; the row
    // maximum over both lane halves is only formed when m moves.
    if (__builtin_amdgcn_ballot_w64(lmax > st.mthr) != 0) {
        // Only the rows whose maximum exceeds the threshold move: a row's m (and so its
        // rounding) never depends on the other rows of the wave.
        const float rmax = max_halves(lmax);
        if (rmax > st.mthr) {
            const float mnew = fmaxf(st.m, rmax * a.qscale);
            const float alpha = fast_exp2(st.m - mnew);
            st.m = mnew;
            st.mthr = (mnew + 8.0f) / a.qscale;
#pragma unroll
            for (int i = 0; i < 4; ++i) st.l4[i] *= alpha;
#pragma unroll
            for (int dd = 0; dd < CfgB<D>::ND; ++dd) st.acc[dd] *= alpha;
        }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) s[v] = fast_exp2(fmaf(s[v], a.qscale, -st.m));
    // P enters the matrix cores rounded to bf16; l sums exactly those values.
    const bf16x8 pb[2] = {pack8(s, 0), pack8(s, 1)};
    st.l4[li] = sum8_bf16(pb[0], st.l4[li]);
    st.l4[li + 1] = sum8_bf16(pb[1], st.l4[li + 1]);
    accum_tr<D, 0>(st.acc, tv, pb);  // O^T += V^T P^T
}

// One tile of the forward (BN keys): its 32-key halves one after the other (a half entirely
// above the diagonal or past the end is skipped, and then so is the second).  OFFV: byte offset
// of the tile's V rows from the ring base.
// (r0 is the position of the wave's first query row, T the number of keys.)
template <int D, bool CAUSAL, int OFFV>
__device__ __forceinline__ void fwd_step(const ArgsB &a, FwdState<D> &st, const unsigned char *sK,
                                         const TrAddr<D> &tra, int kt0, int r0, int T,
                                         const bf16x8 (&qv)[CfgB<D>::KS], int lane) {
    if (!(kt0 < T && (!CAUSAL || kt0 <= r0 + 31))) return;
    fwd_half<D, CAUSAL, OFFV>(a, st, sK, tra, 0, kt0, r0, T, qv, lane, 0);
    if constexpr (CfgB<D>::NSB == 2) {
        const int kb0 = kt0 + 32;
        if (!(kb0 < T && (!CAUSAL || kb0 <= r0 + 31))) return;
        fwd_half<D, CAUSAL, OFFV + 32 * CfgB<D>::RB>(a, st, sK, tra, 32, kb0, r0, T, qv, lane, 2);
    }
}

template <int D, bool CAUSAL, bool ROPE, int NWC>
__device__ __forceinline__ void fwd_tile_b(const ArgsB &a, const QTileB &c, unsigned char *ring) {
    using C = CfgB<D>;
    using R = KVRingB<D, D == 128 ? 3 : NE_BF16_FWD_NST>;
    const int nw = NWC ? NWC : blockDim.x >> 6;  // a compile-time count makes the waits immediates
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    // T query rows; Tk keys; query row r is at position r + qo (a prefill chunk; 0 usually).
    // The half-tile steps take positions and Tk.
    const int T = a.T, Tk = a.Tk, qo = a.qoff;
    const int r0 = __builtin_amdgcn_readfirstlane(c.r0);
    const int qrow = r0 + col;
    const size_t bh = (size_t)c.b * a.Hq + c.h, bg = (size_t)c.b * a.Hkv + c.g;
    const __bf16 *kg = a.k + bg * Tk * D;
    const __bf16 *vg = a.v + bg * Tk * D;

    const int wg_rows = 32 * a.rb;
    const int wg_end = min(c.qt * wg_rows + wg_rows, T);
    const int ntiles = CAUSAL ? (wg_end - 1 + qo) / C::BN + 1 : (Tk + C::BN - 1) / C::BN;
    const bool live = r0 < T;

    // The first two K/V tiles are requested before the query row, so the two latencies overlap
    // (the first use of the row then waits for all three).
    R kv;
    kv.init(wave, nw, lane);
#pragma unroll
    for (int t = 0; t < R::PD; ++t)
        if (t < ntiles) kv.issue(kg, vg, t, Tk, ring + t * R::SB);
    bf16x8 qv[C::KS];
    load_operand_row<D, ROPE>(qv, a.q + bh * T * D, qrow, T, half, a);

    FwdState<D> st;
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) st.acc[dd] = zero16();
    st.m = kNegBig;
    st.mthr = kNegBig;
#pragma unroll
    for (int i = 0; i < 4; ++i) st.l4[i] = 0.f;
    TrAddr<D> tra;  // lane addresses of transposed reads at the ring base; tiles are offsets
    tra.init(ring, lane);
    // Everything requested so far has landed before the loop, so the compiler places no wait
    // for the row inside it.
    wait_vm_lgkm0(0);

    // Tile j uses stage j % NST.  The loop is unrolled over the stages so that each stage's
    // address is a constant: LDS reads then carry it in their offset field instead of adding it.
    auto iter = [&](int j, auto stage) {
        constexpr int ST = decltype(stage)::value;
        // This wave's copies of tile j have landed (only the next PD - 1 tiles' may be in flight)
        // and its reads of tile j-1 are done; after the barrier every wave's are, so tile j is
        // complete and stage (j + PD) % NST, last read for tile j-1, is free.
        wait_vm_lgkm0(min(R::PD - 1, ntiles - 1 - j) * kv.lpw);
        __builtin_amdgcn_s_barrier();
        // Stage (j + PD) % NST held tile j - 1, which every wave has finished: with two stages
        // its copies start now, so that they overlap this tile's work.
        if (R::NST == 2 && j + R::PD < ntiles)
            kv.issue(kg, vg, j + R::PD, Tk, ring + ((ST + R::PD) % R::NST) * R::SB);
        const unsigned char *sK = ring + ST * R::SB;
        if (live) fwd_step<D, CAUSAL, ST * R::SB + R::TB>(a, st, sK, tra, j * C::BN, r0 + qo, Tk, qv, lane);
        // Issued after this tile's reads: the compiler makes transposed LDS reads wait for every
        // copy in flight, and by the next tile's reads these have landed.
        if (R::NST != 2 && j + R::PD < ntiles)
            kv.issue(kg, vg, j + R::PD, Tk, ring + ((ST + R::PD) % R::NST) * R::SB);
    };
    static_assert(R::NST == 2 || R::NST == 3, "the loop below is unrolled over two or three stages");
    for (int j = 0; j < ntiles; j += R::NST) {
        iter(j, std::integral_constant<int, 0>{});
        if (j + 1 < ntiles) iter(j + 1, std::integral_constant<int, 1>{});
        if constexpr (R::NST == 3)
            if (j + 2 < ntiles) iter(j + 2, std::integral_constant<int, 2>{});
    }

    const float l = sum_halves((st.l4[0] + st.l4[1]) + (st.l4[2] + st.l4[3]));
    if (qrow < T) {
        const float inv = 1.0f / l;
        __bf16 *orow = a.out_o + bh * T * D;
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float x[4] = {st.acc[dd][4 * u] * inv, st.acc[dd][4 * u + 1] * inv,
                              st.acc[dd][4 * u + 2] * inv, st.acc[dd][4 * u + 3] * inv};
                store_row4<D, false>(orow, qrow, 32 * dd + 8 * u + 4 * half, x, 0.0, a.rt, 0);
            }
        if (half == 0) a.out_lse[bh * T + qrow] = st.m * kLn2 + logf(l);
    }
}

// NWC: the waves per work-group when known at compile time (4: groups of four query heads),
// else 0.
template <int D, bool CAUSAL, bool ROPE, int NWC>
__global__ void __launch_bounds__(D == 128 ? 256 : 512)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : NE_BF16_FWD_WAVES_PER_EU)))
fwd_bf16(ArgsB a) {
    using R = KVRingB<D, D == 128 ? 3 : NE_BF16_FWD_NST>;
    __shared__ __attribute__((aligned(16))) unsigned char ring[R::NST * R::SB];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const QWorkB w = decode_qwork_b(a);
    fwd_tile_b<D, CAUSAL, ROPE, NWC>(a, qtile_of_b(a, w, w.qt0, wave), ring);
    if (w.qt1 >= 0) {
        __syncthreads();
        fwd_tile_b<D, CAUSAL, ROPE, NWC>(a, qtile_of_b(a, w, w.qt1, wave), ring);
    }
}

template <int D, bool CAUSAL, bool ROPE, int NWC>
__device__ __forceinline__ void dq_tile_b(const ArgsB &a, const QTileB &c, unsigned char *ring) {
    using C = CfgB<D>;
    using R = KVRingB<D>;
    const int nw = NWC ? NWC : blockDim.x >> 6;  // a compile-time count makes the waits immediates
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const int T = a.T;
    const int r0 = __builtin_amdgcn_readfirstlane(c.r0);
    const int qrow = r0 + col;
    const size_t bh = (size_t)c.b * a.Hq + c.h, bg = (size_t)c.b * a.Hkv + c.g;
    const __bf16 *kg = a.k + bg * T * D;
    const __bf16 *vg = a.v + bg * T * D;

    const int wg_rows = 32 * a.rb;
    const int wg_end = min(c.qt * wg_rows + wg_rows, T);
    const int ntiles = CAUSAL ? (wg_end - 1) / C::BN + 1 : (T + C::BN - 1) / C::BN;
    const bool live = r0 < T;

    // The first two K/V tiles are requested before the rows, so the latencies overlap.
    R kv;
    kv.init(wave, nw, lane);
#pragma unroll
    for (int t = 0; t < R::PD; ++t)
        if (t < ntiles) kv.issue(kg, vg, t, T, ring + t * R::SB);
    // Every global read of the row (q, dO, o, lse) is requested before any is used, so their
    // latencies overlap: the rotation of q and delta wait for one round trip, not several.
    bf16x8 qv[C::KS], dov[C::KS], ov[C::KS];
    load_operand_row<D, false>(qv, a.q + bh * T * D, qrow, T, half, a);
    load_operand_row<D, false>(dov, a.dO + bh * T * D, qrow, T, half, a);
    load_operand_row<D, false>(ov, a.o + bh * T * D, qrow, T, half, a);
    const float lse_row = a.lse[bh * T + min(qrow, T - 1)];
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE) rotate_operand_row<D>(qv, qrow, half, a);

    // delta_i = sum_d dO_id o_id over this row (fp32), written once for the dK/dV pass.
    float delta;
    {
        float part = 0.f;
#pragma unroll
        for (int s = 0; s < C::KS; ++s)
#pragma unroll
            for (int i = 0; i < 8; ++i) part += bf2f(dov[s][i]) * bf2f(ov[s][i]);
        delta = sum_halves(part);
    }
    float lse2;
    if (qrow < T) {
        lse2 = lse_row * kLog2e;
        if (half == 0) a.delta[bh * T + qrow] = delta;
    } else {
        lse2 = INFINITY;
        delta = 0.f;
    }
    if (ROPE && qrow < T) {  // each query row is loaded by exactly one wave: keep its rotation
#pragma unroll
        for (int st = 0; st < C::KS; ++st)
            *reinterpret_cast<bf16x8 *>(a.qrot + (bh * T + qrow) * D + 16 * st + 8 * half) = qv[st];
    }

    f32x16 acc[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) acc[dd] = zero16();
    TrAddr<D> tra;  // lane addresses of transposed reads at the ring base, as in the forward
    tra.init(ring, lane);
    wait_vm_lgkm0(0);  // as in the forward

    auto iter = [&](int j, auto stage) {  // unrolled over the stages, as in the forward
        constexpr int ST = decltype(stage)::value;
        wait_vm_lgkm0(min(R::PD - 1, ntiles - 1 - j) * kv.lpw);
        __builtin_amdgcn_s_barrier();
        const unsigned char *sK = ring + ST * R::SB;
        const unsigned char *sV = sK + R::TB;
        // One 32-key half (SB) of the tile; false when it lies above the diagonal or past the
        // end (and so does the next).  The transposed K reads for dQ are issued once both score
        // products are requested, untracked by the compiler (as in the forward).
        auto sub = [&](auto sbc) -> bool {
            constexpr int SB = decltype(sbc)::value;
            const int kb0 = j * C::BN + 32 * SB;
            if (!(live && kb0 < T && (!CAUSAL || kb0 <= r0 + 31))) return false;
            f32x16 p = block_scores<D>(sK, 32 * SB, qv, col, half);
            f32x16 ds = block_scores<D>(sV, 32 * SB, dov, col, half);  // dP^T = V dO^T
            TrOperand<D> tk;
            issue_tr_at<D, ST * R::SB + 32 * SB * C::RB>(tk, tra);
#pragma unroll
            for (int v = 0; v < 16; ++v) p[v] = fast_exp2(fmaf(p[v], a.qscale, -lse2));
            if ((CAUSAL && kb0 + 31 > r0) || kb0 + 32 > T) {  // a block on the diagonal or the end
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int key = kb0 + acc_row(v, half);
                    if ((CAUSAL && key > qrow) || key >= T) p[v] = 0.f;
                }
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) ds[v] = p[v] * (ds[v] - delta);
            const bf16x8 db[2] = {pack8(ds, 0), pack8(ds, 1)};
            accum_tr<D, 0>(acc, tk, db);  // dQ^T += K^T dS^T
            return true;
        };
        if (sub(std::integral_constant<int, 0>{}) && C::NSB == 2)
            sub(std::integral_constant<int, C::NSB - 1>{});
        if (j + R::PD < ntiles)
            kv.issue(kg, vg, j + R::PD, T, ring + ((ST + R::PD) % R::NST) * R::SB);
    };
    for (int j = 0; j < ntiles; j += 3) {
        iter(j, std::integral_constant<int, 0>{});
        if (j + 1 < ntiles) iter(j + 1, std::integral_constant<int, 1>{});
        if (j + 2 < ntiles) iter(j + 2, std::integral_constant<int, 2>{});
    }

    if (qrow < T) {
        __bf16 *drow = a.dq + bh * T * D;
        const double tpos2 = ROPE ? (double)qrow * (half ? a.rope_shift2 : 1.0) : 0.0;
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float x[4] = {acc[dd][4 * u] * a.scale, acc[dd][4 * u + 1] * a.scale,
                              acc[dd][4 * u + 2] * a.scale, acc[dd][4 * u + 3] * a.scale};
                // pairs 16 dd + 4 u + 2 half + p: the second half-wave's are 2 further on
                store_row4<D, ROPE>(drow, qrow, 32 * dd + 8 * u + 4 * half, x, tpos2, a.rt,
                                    16 * dd + 4 * u);
            }
    }
}

// NWC: the waves per work-group when known at compile time (4: groups of four query heads),
// else 0.
template <int D, bool CAUSAL, bool ROPE, int NWC>
__global__ void __launch_bounds__(D == 128 ? 256 : 512)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : NE_BF16_DQ_WAVES_PER_EU)))
dq_bf16(ArgsB a) {
    __shared__ __attribute__((aligned(16))) unsigned char ring[KVRingB<D>::NST * KVRingB<D>::SB];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const QWorkB w = decode_qwork_b(a);
    dq_tile_b<D, CAUSAL, ROPE, NWC>(a, qtile_of_b(a, w, w.qt0, wave), ring);
    if (w.qt1 >= 0) {
        __syncthreads();
        dq_tile_b<D, CAUSAL, ROPE, NWC>(a, qtile_of_b(a, w, w.qt1, wave), ring);
    }
}

// Row stride (floats) of the fp32 partial dK, dV rows in the final reduction: 16 bytes of
// padding put the rows that 16 lanes write at once in different banks.
template <int D>
constexpr int dkdv_red_ld() { return D + 4; }

// Staging of the dK/dV items.  Each wave copies its own (query head, 32-row query block) items
// straight into two private LDS stages, one item ahead: the query tile and the dO tile in the
// swizzled layout (NPQ 1 KB pieces each, laid out as in KVRingB), then the 32 lse and the 32
// delta values of the rows in one 256-byte copy.  Every wave issues NDMA copies per item.
template <int D>
struct ItemStageB {
    using C = CfgB<D>;
    static constexpr int TBQ = 32 * C::RB;      // bytes of a 32-row tile
    static constexpr int NPQ = TBQ / 1024;      // 1 KB pieces per tile
    static constexpr int RPP = 1024 / C::RB;    // tile rows per piece
    static constexpr int SB = 2 * TBQ + 256;    // bytes of a stage
    static constexpr int NDMA = 2 * NPQ + 1;    // copies per item
};

// LDS bytes per dK/dV wave: the larger of its two item stages and the fp32 partial dK, dV it
// contributes to the final reduction.
template <int D>
constexpr int dkdv_wave_bytes_b() {
    constexpr int stage = 2 * ItemStageB<D>::SB;
    constexpr int red = 2 * 32 * dkdv_red_ld<D>() * 4;
    return stage > red ? stage : red;
}

template <int D, bool CAUSAL, bool ROPE>
__device__ __forceinline__ void dkdv_block_b(const ArgsB &a, int b, int g, int kb,
                                             unsigned char *smem_b) {
    using C = CfgB<D>;
    using S = ItemStageB<D>;
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const int T = a.T;
    const size_t bg = (size_t)b * a.Hkv + g;
    const int krow = kb * 32 + col;

    f32x16 dk[C::ND], dv[C::ND];
#pragma unroll
    for (int dd = 0; dd < C::ND; ++dd) {
        dk[dd] = zero16();
        dv[dd] = zero16();
    }

    const int nqb = (T + 31) / 32;
    const int i0 = CAUSAL ? kb : 0;
    const int per_head = nqb - i0;
    const int nitems = a.G * per_head;

    // This lane's 16 bytes of a piece: row lrow of the piece, swizzled chunk (piece pc: the
    // offset XOR 16 swizzle_piece_xor(pc)).
    const int lrow = lane / C::NCH;
    const int chb = 16 * chunk_swizzle<D>(lrow, lane % C::NCH);
    const int off0 = lrow * C::RB + chb;
    // A wave takes the items wave, wave + nw, ... in order, both when it copies them and when it
    // uses them: (head hh of the group, query block i0 + ii) of the next item to copy and of the
    // next to use are advanced by nw items at a time, so the loop divides nothing.
    struct ItemPos {
        int hh, ii;
        __device__ __forceinline__ void advance(int n, int per) {
            ii += n;
            while (ii >= per) {
                ii -= per;
                ++hh;
            }
        }
    };
    const size_t bh0 = (size_t)b * a.Hq + (size_t)g * a.G;  // the group's first query head
    ItemPos cp{(int)((unsigned)wave / (unsigned)per_head), (int)((unsigned)wave % (unsigned)per_head)};
    ItemPos up = cp;
    // Starts the copies of the next item (cp) into `st`, through buffer resources on the
    // head's q and dO.  Rows past the end read row T - 1; their lse is replaced by +inf once
    // the item has landed, so their probabilities are 0.
    auto issue = [&](unsigned char *st) {
        const int i = i0 + cp.ii;
        const size_t bh = bh0 + cp.hh;
        cp.advance(nw, per_head);
        const unsigned bytes = (unsigned)T * C::RB;
        const buf_rsrc_t rq = raw_rsrc(a.q + bh * T * D, bytes);
        const buf_rsrc_t ro = raw_rsrc(a.dO + bh * T * D, bytes);
        if (i * 32 + 32 <= T) {
            // Piece pc sits 1 KB further on in both the tensor and the stage: an instruction
            // offset (below 4 KB; each group of four pieces steps the uniform offsets), so the
            // destinations of a stage are two values per group.
            const unsigned soff = (unsigned)(i * 32 * C::RB);
            // All Q pieces, then all dO pieces: a run shares one LDS base (the M0 register).
            static_for<2>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                static_for<S::NPQ>([&](auto pcc) {
                    constexpr int pc = decltype(pcc)::value;
                    constexpr int hi = (pc / 4) * 4096;
                    const unsigned vo = (unsigned)(off0 ^ (16 * swizzle_piece_xor<D>(pc)));
                    dma16_buf_imm<(pc % 4) * 1024>(t ? ro : rq, vo, soff + hi, st + t * S::TBQ + hi);
                });
            });
        } else {
            // Rare (the last item of a head with T % 32 != 0): the stage address is made opaque
            // so that its per-piece destinations are formed here, not held across the loop.
            typedef __attribute__((address_space(3))) unsigned char lds_u8;
            uint32_t sto = (uint32_t)(uintptr_t)(lds_u8 *)st;
            asm volatile("" : "+s"(sto));
#pragma unroll
            for (int pc = 0; pc < S::NPQ; ++pc) {
                const int r = min(i * 32 + pc * S::RPP + lrow, T - 1);
                const unsigned vo = (unsigned)((r * C::RB + chb) ^ (16 * swizzle_piece_xor<D>(pc)));
                dma16_buf_at(rq, vo, 0u, sto + pc * 1024);
                dma16_buf_at(ro, vo, 0u, sto + S::TBQ + pc * 1024);
            }
        }
        const int r = min(i * 32 + col, T - 1);  // lanes 0..31: lse, lanes 32..63: delta
        dma4((half ? a.delta : a.lse) + bh * T + r, st + 2 * S::TBQ);
    };

    // The first two items are requested before the K, V rows, so the latencies overlap; all of
    // it has landed before the loop, so the compiler places no wait for the rows inside it.
    unsigned char *wbuf = smem_b + wave * dkdv_wave_bytes_b<D>();
    if (wave < nitems) issue(wbuf);
    if (wave + nw < nitems) issue(wbuf + S::SB);
    bf16x8 kv[C::KS], vv[C::KS];
    load_operand_row<D, false>(kv, a.k + bg * T * D, krow, T, half, a);
    load_operand_row<D, false>(vv, a.v + bg * T * D, krow, T, half, a);
    wait_vm_lgkm0(0);
    TrAddr<D> tra;  // transposed reads of the stage-0 Q tile; other tiles are immediate offsets
    tra.init(wbuf, lane);
    // One item in stage ST (compile-time, so that every LDS offset of the item is an immediate).
    auto item = [&](int it, auto stage) {
        constexpr int ST = decltype(stage)::value;
        const int i = i0 + up.ii;
        up.advance(nw, per_head);
        unsigned char *st = wbuf + ST * S::SB;
        const unsigned char *sQ = st;
        const unsigned char *sO = st + S::TBQ;
        float *sL = reinterpret_cast<float *>(st + 2 * S::TBQ);
        const float *sDl = sL + 32;
        // This item's copies have landed (the next item's may still be in flight); the stage
        // is private to the wave, so no barrier is needed.
        wait_vm_lgkm0(it + nw < nitems ? S::NDMA : 0);
        // lse of rows past the end -> +inf (P = 0); delta -> -delta, the start of dP - delta.
        sL[lane] = lane >= 32 ? -sL[lane] : i * 32 + lane < T ? sL[lane] * kLog2e : INFINITY;

        // S = Q K'^T (rows: queries acc_row(v, half) of the block; column: this lane's key)
        f32x16 p = zero16();
#pragma unroll
        for (int st2 = 0; st2 < C::KS; ++st2)
            p = mfma32_bf16(tile_read8<D>(sQ, col, 16 * st2 + 8 * half), kv[st2], p);
        // dP - delta = dO V^T - delta (rows of the accumulator: queries)
        f32x16 ds;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 Dl = ld4(sDl + 8 * u + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) ds[4 * u + e] = Dl[e];
        }
#pragma unroll
        for (int st2 = 0; st2 < C::KS; ++st2)
            ds = mfma32_bf16(tile_read8<D>(sO, col, 16 * st2 + 8 * half), vv[st2], ds);
        // The transposed operands of dV and dK are requested now, so their latency overlaps
        // the exponentials.
        TrOperand<D> tdo, tq;
        issue_tr_at<D, ST * S::SB + S::TBQ>(tdo, tra);
        issue_tr_at<D, ST * S::SB>(tq, tra);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 L = ld4(sL + 8 * u + 4 * half);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[4 * u + e] = fast_exp2(fmaf(p[4 * u + e], a.qscale, -L[e]));
        }
        if (CAUSAL && i == kb) {  // the diagonal block: keys after the query get P = 0
#pragma unroll
            for (int v = 0; v < 16; ++v)
                if (col > acc_row(v, half)) p[v] = 0.f;
        }
        // dV^T += dO^T P
        const bf16x8 pb[2] = {pack8(p, 0), pack8(p, 1)};
        accum_tr<D, TrOperand<D>::NREAD>(dv, tdo, pb);
        // dS = P (dP - delta)
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] *= p[v];
        // dK^T += Q^T dS
        const bf16x8 db[2] = {pack8(ds, 0), pack8(ds, 1)};
        accum_tr<D, 0>(dk, tq, db);
        // The stage is free once this item's reads are done: copy the item after next into it.
        if (it + 2 * nw < nitems) issue(st);
    };
    for (int it = wave; it < nitems; it += 2 * nw) {
        item(it, std::integral_constant<int, 0>{});
        if (it + nw < nitems) item(it + nw, std::integral_constant<int, 1>{});
    }

    // Add the waves' partial sums in LDS (fixed wave order), rotate dK back, round, store.
    __syncthreads();
    {
        float *R = reinterpret_cast<float *>(wbuf);
#pragma unroll
        for (int dd = 0; dd < C::ND; ++dd)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int d = 32 * dd + 8 * u + 4 * half;
                constexpr int LD = dkdv_red_ld<D>();
                st4(R + col * LD + d, f32x4{dk[dd][4 * u] * a.scale, dk[dd][4 * u + 1] * a.scale,
                                            dk[dd][4 * u + 2] * a.scale, dk[dd][4 * u + 3] * a.scale});
                st4(R + 32 * LD + col * LD + d,
                    f32x4{dv[dd][4 * u], dv[dd][4 * u + 1], dv[dd][4 * u + 2], dv[dd][4 * u + 3]});
            }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 2 * 32 * (D / 4); idx += blockDim.x) {
        const int t = idx / (32 * (D / 4));
        const int r = (idx / (D / 4)) % 32;
        const int cc = 4 * (idx % (D / 4));
        f32x4 sum{0.f, 0.f, 0.f, 0.f};
        for (int w = 0; w < nw; ++w)
            sum += ld4(reinterpret_cast<const float *>(smem_b + w * dkdv_wave_bytes_b<D>()) +
                       (t * 32 + r) * dkdv_red_ld<D>() + cc);
        const int row = kb * 32 + r;
        if (row < T) {
            float x[4] = {sum[0], sum[1], sum[2], sum[3]};
            if (t == 0) {
                // pairs cc / 2 + p: per_pos[cc / 2 + p] = per_pos[p] * base^(-cc/D)
                const double tpos = ROPE ? (double)row * exp2(-(double)cc / D * a.rope_lb) : 0.0;
                store_row4<D, ROPE>(a.dk + bg * T * D, row, cc, x, tpos, a.rt, 0);
            } else {
                store_row4<D, false>(a.dv + bg * T * D, row, cc, x, 0.0, a.rt, 0);
            }
        }
    }
}

template <int D, bool CAUSAL, bool ROPE>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : NE_BF16_DKDV_WAVES_PER_EU)))
dkdv_bf16(ArgsB a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_b[];
    const int per = a.B * a.Hkv;
    const int p = blockIdx.x / per;
    const int g = (blockIdx.x % per) % a.Hkv;
    const int b = (blockIdx.x % per) / a.Hkv;
    dkdv_block_b<D, CAUSAL, ROPE>(a, b, g, p, smem_b);
    if (a.paired && a.nkb - 1 - p > p) {
        __syncthreads();
        dkdv_block_b<D, CAUSAL, ROPE>(a, b, g, a.nkb - 1 - p, smem_b);
    }
}

// RoPE applied once to a whole bf16 tensor [BH][T][D] (the position of a row is its t), in fp32
// with the angle reduced modulo one turn in double precision, rounded once to bf16.  Each thread
// owns one (position, 8-column chunk): it evaluates the four sines and cosines once and applies
// them to the rows of every (batch, head) it visits.  The attention kernels that stream a tensor
// through LDS many times read this rotated copy.
template <int D>
__global__ void __launch_bounds__(256) rope_rows_bf16(const __bf16 *x, __bf16 *y, long long nbh, int T,
                                                      RopeTurns rt) {
    const int idx = blockIdx.x * 256 + threadIdx.x;
    if (idx >= T * (D / 8)) return;
    const int t = idx / (D / 8);
    const int c = 8 * (idx % (D / 8));
    float sn[4], cs[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const double turns = (double)t * rt.per_pos[c / 2 + p];
        sincospif(2.0f * (float)(turns - rint(turns)), &sn[p], &cs[p]);
    }
    for (long long bh = blockIdx.y; bh < nbh; bh += gridDim.y) {
        const size_t off = ((size_t)bh * T + t) * D + c;
        float f[8];
        unpack8(*reinterpret_cast<const bf16x8 *>(x + off), f);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const float u = f[2 * p], w = f[2 * p + 1];
            f[2 * p] = u * cs[p] - w * sn[p];
            f[2 * p + 1] = u * sn[p] + w * cs[p];
        }
        *reinterpret_cast<bf16x8 *>(y + off) = round8(f);
    }
}

ArgsB make_args_b(const Shape &s) {
    ArgsB a{};
    a.B = s.B;
    a.Hq = s.Hq;
    a.Hkv = s.Hkv;
    a.T = s.T;
    a.Tk = s.Tk > 0 ? s.Tk : s.T;
    a.qoff = a.Tk - s.T;
    a.G = s.G;
    a.scale = (float)(1.0 / sqrt((double)s.D));
    a.qscale = (float)(1.4426950408889634 / sqrt((double)s.D));
    a.rt = rope_turns(s);
    const double lb = s.rope_base > 0.f ? log2((double)s.rope_base) : 0.0;
    a.rope_shift4 = exp2(-8.0 / s.D * lb);
    a.rope_shift2 = exp2(-4.0 / s.D * lb);
    a.rope_lb = lb;
    const QTileGeom g = qtile_geometry(s, false);
    a.hpw = g.hpw;
    a.rb = g.rb;
    a.nqt = g.nqt;
    a.nkb = kblock_geometry(s, false).nkb;
    return a;
}

#define NE_PICK_B(KERNEL, TPARAMS, TARGS)                                                    \
    template <TPARAMS>                                                                       \
    const void *pick_##KERNEL(bool causal, bool rope) {                                      \
        if (causal)                                                                          \
            return rope ? (const void *)KERNEL<D, true, true TARGS>                          \
                        : (const void *)KERNEL<D, true, false TARGS>;                        \
        return rope ? (const void *)KERNEL<D, false, true TARGS>                             \
                    : (const void *)KERNEL<D, false, false TARGS>;                           \
    }
#define NE_COMMA ,
NE_PICK_B(fwd_bf16, int D NE_COMMA int NWC, NE_COMMA NWC)
NE_PICK_B(dq_bf16, int D NE_COMMA int NWC, NE_COMMA NWC)
NE_PICK_B(dkdv_bf16, int D, )
#undef NE_COMMA
#undef NE_PICK_B

// The query-tile kernel for this shape: four-wave groups get the variant with the count built in.
template <template <int, int> class P>
const void *pick_qtile(const Shape &s, int nwaves) {
    const bool causal = s.causal != 0, rope = s.rope_base > 0.f;
    if (s.D == 128) return nwaves == 4 ? P<128, 4>::get(causal, rope) : P<128, 0>::get(causal, rope);
    if (s.D == 64) return nwaves == 4 ? P<64, 4>::get(causal, rope) : P<64, 0>::get(causal, rope);
    return nwaves == 4 ? P<32, 4>::get(causal, rope) : P<32, 0>::get(causal, rope);
}
template <int D, int NWC>
struct PickFwd {
    static const void *get(bool causal, bool rope) { return pick_fwd_bf16<D, NWC>(causal, rope); }
};
template <int D, int NWC>
struct PickDq {
    static const void *get(bool causal, bool rope) { return pick_dq_bf16<D, NWC>(causal, rope); }
};

hipError_t launch_b(const void *fn, long long blocks, int threads, size_t lds, hipStream_t st,
                    ArgsB &a) {
    void *params[] = {&a};
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(threads), params, lds, st);
}

}  // namespace

hipError_t launch_fwd_bf16(const Shape &s, const void *q, const void *k, const void *v, void *o,
                           float *lse, hipStream_t st) {
    if (s.D != 32 && s.D != 64 && s.D != 128) return hipErrorInvalidValue;
    ArgsB a = make_args_b(s);
    a.q = static_cast<const __bf16 *>(q);
    a.k = static_cast<const __bf16 *>(k);
    a.v = static_cast<const __bf16 *>(v);
    a.out_o = static_cast<__bf16 *>(o);
    a.out_lse = lse;
    const QTileGeom g = qtile_geometry(s, s.causal && kPairBf16.fwd != 0);
    a.paired = g.paired;
    const void *fn = pick_qtile<PickFwd>(s, g.nwaves);
    return launch_b(fn, g.nblocks, 64 * g.nwaves, 0, st, a);
}

hipError_t launch_dq_bf16(const Shape &s, const void *q, const void *k, const void *v,
                          const void *o, const float *lse, const void *dO, void *dq, float *delta,
                          void *qrot, hipStream_t st) {
    if (s.D != 32 && s.D != 64 && s.D != 128) return hipErrorInvalidValue;
    ArgsB a = make_args_b(s);
    a.q = static_cast<const __bf16 *>(q);
    a.k = static_cast<const __bf16 *>(k);
    a.v = static_cast<const __bf16 *>(v);
    a.o = static_cast<const __bf16 *>(o);
    a.lse = lse;
    a.dO = static_cast<const __bf16 *>(dO);
    a.dq = static_cast<__bf16 *>(dq);
    a.delta = delta;
    a.qrot = static_cast<__bf16 *>(qrot);
    const QTileGeom g = qtile_geometry(s, s.causal && kPairBf16.dq != 0);
    a.paired = g.paired;
    const void *fn = pick_qtile<PickDq>(s, g.nwaves);
    return launch_b(fn, g.nblocks, 64 * g.nwaves, 0, st, a);
}

hipError_t launch_dkdv_bf16(const Shape &s, const void *q, const void *k, const void *v,
                            const float *lse, const void *dO, const float *delta, void *dk,
                            void *dv, hipStream_t st) {
    if (s.D != 32 && s.D != 64 && s.D != 128) return hipErrorInvalidValue;
    ArgsB a = make_args_b(s);
    a.q = static_cast<const __bf16 *>(q);
    a.k = static_cast<const __bf16 *>(k);
    a.v = static_cast<const __bf16 *>(v);
    a.lse = lse;
    a.dO = static_cast<const __bf16 *>(dO);
    a.delta = const_cast<float *>(delta);  // read only in this pass
    a.dk = static_cast<__bf16 *>(dk);
    a.dv = static_cast<__bf16 *>(dv);
    const KBlockGeom g = kblock_geometry(s, s.causal && kPairBf16.dkdv != 0);
    a.paired = g.paired;
    const bool causal = s.causal != 0, rope = s.rope_base > 0.f;
    const int wb = s.D == 128  ? dkdv_wave_bytes_b<128>()
                   : s.D == 64 ? dkdv_wave_bytes_b<64>()
                               : dkdv_wave_bytes_b<32>();
    const size_t lds = (size_t)g.nwaves * wb;
    const void *fn = s.D == 128  ? pick_dkdv_bf16<128>(causal, rope)
                     : s.D == 64 ? pick_dkdv_bf16<64>(causal, rope)
                                 : pick_dkdv_bf16<32>(causal, rope);
    return launch_b(fn, g.nblocks, 64 * g.nwaves, lds, st, a);
}

hipError_t launch_rope_bf16(const Shape &s, const void *x, void *y, long long rows,
                            hipStream_t st) {
    if (s.D != 32 && s.D != 64 && s.D != 128) return hipErrorInvalidValue;
    const __bf16 *xb = static_cast<const __bf16 *>(x);
    __bf16 *yb = static_cast<__bf16 *>(y);
    RopeTurns rt = rope_turns(s);
    long long nbh = rows / s.T;
    int T = s.T;
    const long long per_pos = (long long)T * (s.D / 8);
    const unsigned gx = (unsigned)((per_pos + 255) / 256);
    // About 8 (batch, head) rows per thread when that still leaves enough threads.
    const long long gy = std::max(1LL, std::min(nbh, std::max(nbh / 8, 2048LL / (long long)gx)));
    const void *fn = s.D == 128  ? (const void *)rope_rows_bf16<128>
                     : s.D == 64 ? (const void *)rope_rows_bf16<64>
                                 : (const void *)rope_rows_bf16<32>;
    void *params[] = {&xb, &yb, &nbh, &T, &rt};
    return hipLaunchKernel(fn, dim3(gx, (unsigned)std::min(gy, 65535LL)), dim3(256), params, 0, st);
}

}  // namespace ne
