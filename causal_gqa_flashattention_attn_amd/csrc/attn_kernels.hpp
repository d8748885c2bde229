// attn_kernels.hpp -- launch descriptions shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>

namespace ne {

// Where the rows of a [B][H][T][D] tensor live: element (b, h, t, d) at b sb + h sh + t st + d
// (elements).  Contiguous: sb = H T D, sh = T D, st = D.  The attention sub-block reads q, k, v
// straight from the rows of its projection ([B T][W]: sb = T W, sh = D, st = W) and writes o,
// dq, dk, dv as rows.
// Element (b, h, t, d) of a tensor sits at b sb + h sh + t st + d (d contiguous).  sh is at most
// T D <= 2^31 (contiguous heads), st at most the width of a row of the attention sub-block's
// projections, so both fit 32 bits; they are kept narrow to spare scalar registers.
struct TLay {
    long long sb;
    unsigned sh;
    int st;
};
// Layouts of every tensor the float32 kernels read or write (lse and delta are always
// contiguous [B][Hq][T]).
struct TLays {
    TLay q, k, v, o, dO, dq, dk, dv;
};

__host__ __device__ inline TLay contiguous_lay(int H, int T, int D) {
    return TLay{(long long)H * T * D, (unsigned)T * (unsigned)D, D};
}

// One problem instance.  Element offsets are computed in 64-bit inside the kernels.
struct Shape {
    int B, Hq, Hkv, T, D, G;  // G = Hq / Hkv
    int causal;
    float rope_base;          // 0: no RoPE
    // Forward only: keys/values of length Tk >= T, query row i at position i + Tk - T (a chunk
    // of T new queries against a cache).  0: Tk = T.
    int Tk = 0;
    // float32 kernels: tensor layouts; null: all contiguous.
    const TLays *lay = nullptr;
};

// Work-group composition of the query-tile kernels (forward and dQ): each work-group serves
// `hpw` query heads of one key/value head and `rb` 32-row blocks per head, i.e. hpw * rb waves,
// all sharing each K/V tile staged in LDS.
//
// With a causal mask the work of a query tile grows with its position.  With `pair` set,
// work-groups take a mirrored pair of tiles (qt and nqt-1-qt, one after the other), so every
// work-group does the same work and a single round of work-groups fills the GPU evenly.
struct QTileGeom {
    int hpw, rb, nwaves, rows;  // rows = 32 * rb query rows per head
    int nqt;                    // query tiles per head
    int paired;                 // work-groups take mirrored tile pairs
    long long nblocks;
};

QTileGeom qtile_geometry(const Shape &s, bool pair);

// Key-block kernel (dK/dV): one work-group per (b, kv head, 32-key block) -- per mirrored pair
// of key blocks with `pair` set -- with `nwaves` waves that split the group's (query head, query
// block) items between them and add their partial sums in LDS.
struct KBlockGeom {
    int nwaves, nkb;
    int paired;
    long long nblocks;
};

KBlockGeom kblock_geometry(const Shape &s, bool pair);

// Which passes take mirrored pairs under a causal mask (measured per pass and dtype).  Pairing
// evens out the work per work-group, but a compute unit favours its oldest waves, so equal
// work-groups still finish at staggered times; once none is left to dispatch the unit drains
// at low occupancy.  Unpaired launches, longest tile first, keep more work-groups in flight and
// win where the grid is several times the resident capacity (the fp32 forward at long
// sequences, and the bf16 passes); pairing wins for the fp32 backward passes.
#ifndef NE_PAIR_F32
#define NE_PAIR_F32 0, 1, 1  // forward, dQ, dK/dV
#endif
#ifndef NE_PAIR_BF16
#define NE_PAIR_BF16 0, 0, 0
#endif
struct PairPolicy {
    int fwd, dq, dkdv;
};
constexpr PairPolicy kPairF32{NE_PAIR_F32};
constexpr PairPolicy kPairBf16{NE_PAIR_BF16};

// With RoPE (s.rope_base > 0) the kernels take rotated k, since they stream it through LDS.
// The forward and the dQ pass rotate each query row as they load it; the dQ pass also writes
// the rotated rows to `qrot`, which the dK/dV pass then takes as q (it streams q through LDS).
// dq and dk are rotated back before they are stored.
hipError_t launch_fwd_f32(const Shape &s, const float *q, const float *k, const float *v,
                          float *o, float *lse, hipStream_t st);
// dQ pass: writes dq, delta (= rowsum(dO * o)) and, with RoPE, the rotated q to qrot.
hipError_t launch_dq_f32(const Shape &s, const float *q, const float *k, const float *v,
                         const float *o, const float *lse, const float *dO, float *dq,
                         float *delta, float *qrot, hipStream_t st);
// dK/dV pass: reads delta written by the dQ pass.
hipError_t launch_dkdv_f32(const Shape &s, const float *q, const float *k, const float *v,
                           const float *lse, const float *dO, const float *delta, float *dk,
                           float *dv, hipStream_t st);

// Single-pass backward (float32): a pre-pass writes delta and zeroes dq, then one key-block
// pass forms dk, dv and adds dq with fp32 atomics (dq not bitwise reproducible).  With RoPE,
// q and k are first rotated into qrot, krot ([B][Hq][T][D], [B][Hkv][T][D]) and dq is rotated
// back at the end.
hipError_t launch_bwd_fused_f32(const Shape &s, const float *q, const float *k, const float *v,
                                const float *o, const float *lse, const float *dO, float *dq,
                                float *dk, float *dv, float *delta, float *qrot, float *krot,
                                hipStream_t st);

// Attention sub-block helpers (attn_block.hip), float32, row-major.
// rocBLAS workspace of the sub-block's products: a region of the caller's block workspace.
constexpr size_t kBlasWorkspaceBytes = (size_t)32 << 20;
hipError_t gemm_rm(hipStream_t st, void *ws, size_t ws_bytes, bool ta, bool tb, int M, int N,
                   int K, const float *A, const float *Bm, float *Cm, float beta);
hipError_t launch_rmsnorm_fwd(const float *x, const float *gamma, float *xn, float *rstd,
                              long long rows, int C, float eps, hipStream_t st);
int rmsnorm_bwd_blocks(long long rows);
hipError_t launch_rmsnorm_bwd(const float *x, const float *gamma, const float *rstd,
                              const float *dxn, const float *dy, float *dx, float *part,
                              float *dgamma, long long rows, int C, hipStream_t st);

// bfloat16 variants: tensors are bf16 (passed untyped), lse and delta fp32.
hipError_t launch_fwd_bf16(const Shape &s, const void *q, const void *k, const void *v, void *o,
                           float *lse, hipStream_t st);
hipError_t launch_dq_bf16(const Shape &s, const void *q, const void *k, const void *v,
                          const void *o, const float *lse, const void *dO, void *dq, float *delta,
                          void *qrot, hipStream_t st);
hipError_t launch_dkdv_bf16(const Shape &s, const void *q, const void *k, const void *v,
                            const float *lse, const void *dO, const float *delta, void *dk,
                            void *dv, hipStream_t st);

// Turns per position of each RoPE pair, base^(-2i/D) / (2 pi), evaluated on the host in double.
struct RopeTurns {
    double per_pos[64];
};

inline RopeTurns rope_turns(const Shape &s) {
    RopeTurns r{};
    const double lb = s.rope_base > 0.f ? log2((double)s.rope_base) : 0.0;
    for (int i = 0; i < s.D / 2 && i < 64; ++i)
        r.per_pos[i] = exp2(-(2.0 * i / s.D) * lb) * 0.15915494309189535;
    return r;
}

// RoPE applied to a whole tensor [rows / T][T][D] (s.rope_base > 0), x -> y; y contiguous, x
// in layout xl over H heads (null: contiguous).
hipError_t launch_rope_f32(const Shape &s, const float *x, float *y, long long rows,
                           hipStream_t st, bool inv = false, const TLay *xl = nullptr, int H = 1);
hipError_t launch_rope_bf16(const Shape &s, const void *x, void *y, long long rows,
                            hipStream_t st);

// Decode step against a key/value cache (s.T = cache length Tc): one query per (batch, query
// head), keys 0 .. lens[b] - 1.  q, o: [B][Hq][D]; k, v: [B][Hkv][Tc][D] (bf16 when bf16 != 0,
// else fp32); lse [B][Hq] fp32; part_o, part_lse: workspace of decode_splits(Tc) splits,
// [split][B][Hq][D] and [split][B][Hq] fp32.
int decode_splits(int Tc);
hipError_t launch_decode(const Shape &s, int bf16, const void *q, const void *k, const void *v,
                         const int *lens, void *o, float *lse, float *part_o, float *part_lse,
                         hipStream_t st);

}  // namespace ne
