// attn_kernels.hpp -- launch descriptions shared by the host entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace ne {

// One problem instance.  Element offsets are computed in 64-bit inside the kernels.
struct Shape {
    int B, Hq, Hkv, T, D, G;  // G = Hq / Hkv
    int causal;
    float rope_base;          // 0: no RoPE
};

// Work-group composition of the query-tile kernels (forward and dQ): each work-group serves
// `hpw` query heads of one key/value head and `rb` 32-row blocks per head, i.e. hpw * rb waves,
// all sharing each K/V tile staged in LDS.
struct QTileGeom {
    int hpw, rb, nwaves, rows;  // rows = 32 * rb query rows per head
    int nqt;                    // query tiles per head
    long long nblocks;
};

QTileGeom qtile_geometry(const Shape &s);

// Key-block kernel (dK/dV): one work-group per (b, kv head, 32-key block), `nwaves` waves that
// split the group's query heads between them and reduce their partial sums in LDS.
struct KBlockGeom {
    int nwaves, nkb;
    long long nblocks;
};

KBlockGeom kblock_geometry(const Shape &s);

hipError_t launch_fwd_f32(const Shape &s, const float *q, const float *k, const float *v,
                          float *o, float *lse, hipStream_t st);
// dQ pass: writes dq and delta (= rowsum(dO * o)).
hipError_t launch_dq_f32(const Shape &s, const float *q, const float *k, const float *v,
                         const float *o, const float *lse, const float *dO, float *dq,
                         float *delta, hipStream_t st);
// dK/dV pass: reads delta written by the dQ pass.
hipError_t launch_dkdv_f32(const Shape &s, const float *q, const float *k, const float *v,
                           const float *lse, const float *dO, const float *delta, float *dk,
                           float *dv, hipStream_t st);

// bfloat16 variants: tensors are bf16 (passed untyped), lse and delta fp32.
hipError_t launch_fwd_bf16(const Shape &s, const void *q, const void *k, const void *v, void *o,
                           float *lse, hipStream_t st);
hipError_t launch_dq_bf16(const Shape &s, const void *q, const void *k, const void *v,
                          const void *o, const float *lse, const void *dO, void *dq, float *delta,
                          hipStream_t st);
hipError_t launch_dkdv_bf16(const Shape &s, const void *q, const void *k, const void *v,
                            const float *lse, const void *dO, const float *delta, void *dk,
                            void *dv, hipStream_t st);

}  // namespace ne
