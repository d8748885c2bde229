// ne_attn_api.hip -- the C ABI declared in include/ne_attn.h: argument checks, then dispatch to
// the gfx950 kernels on the caller's stream.  Nothing here allocates, synchronises or keeps
// state.
#include <math.h>
#include <stdint.h>

#include <initializer_list>
#include <mutex>

#include "../../include/ne_attn.h"
#include "attn_kernels.hpp"

namespace {

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

// The bf16 kernels address one head's T x D tensor through buffer resources, whose byte count
// and offsets are 32-bit: a head must span at most 2^31 bytes (T <= 2^23 at D = 128).
bool bf16_head_fits(long long T, int D) { return T * D * 2 <= (1LL << 31); }

// Checks shared by every entry point; fills `s` on success.
int check_shape(int B, int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
                ne::Shape &s) {
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1) return NE_ERR_SHAPE;
    if (Hq % Hkv != 0) return NE_ERR_SHAPE;
    if (D != 32 && D != 64 && D != 128) return NE_ERR_UNSUPPORTED;
    if (dtype != NE_F32 && dtype != NE_BF16) return NE_ERR_UNSUPPORTED;
    if (!(rope_base >= 0.f) || !isfinite(rope_base)) return NE_ERR_UNSUPPORTED;
    // Element counts and grid sizes must stay far from 64-bit and 31-bit limits.
    const double rows = (double)B * (double)Hq * (double)T;
    if (rows * D > 9.0e15 || T > (1 << 24)) return NE_ERR_SHAPE;
    if (dtype == NE_BF16 && !bf16_head_fits(T, D)) return NE_ERR_SHAPE;
    s.B = B;
    s.Hq = Hq;
    s.Hkv = Hkv;
    s.T = T;
    s.D = D;
    s.G = Hq / Hkv;
    s.causal = causal != 0;
    s.rope_base = rope_base;
    // Unpaired launches have the most work-groups.
    const ne::QTileGeom gq = ne::qtile_geometry(s, false);
    const ne::KBlockGeom gk = ne::kblock_geometry(s, false);
    if (gq.nblocks > 0x7fffffffLL || gk.nblocks > 0x7fffffffLL) return NE_ERR_SHAPE;
    return NE_OK;
}

bool any_misaligned(std::initializer_list<const void *> ptrs) {
    for (const void *p : ptrs)
        if (misaligned(p)) return true;
    return false;
}

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace of the _ex entry points: delta (fp32 [B][Hq][T]) first, then -- with RoPE -- the
// rotated keys [B][Hkv][T][D] and the rotated queries [B][Hq][T][D] in the tensors' dtype, each
// region starting on a 256-byte boundary.
struct WsLayout {
    size_t delta, kr, qr, total;
};

WsLayout ws_layout(const ne::Shape &s, int dtype) {
    const size_t es = dtype == NE_BF16 ? 2 : 4;
    const size_t bt = (size_t)s.B * (size_t)s.T;
    WsLayout w{};
    size_t off = up256(4 * bt * (size_t)s.Hq);
    if (s.rope_base > 0.f) {
        w.kr = off;
        off += up256(es * bt * (size_t)s.Hkv * (size_t)s.D);
        w.qr = off;
        off += up256(es * bt * (size_t)s.Hq * (size_t)s.D);
    }
    w.total = off;
    return w;
}

// Rotates the keys (or queries) x of H heads into the contiguous copy y; xl: x's layout (fp32
// only; null: contiguous).
hipError_t launch_rope(const ne::Shape &s, int dtype, const void *x, void *y, long long rows,
                       hipStream_t stream, const ne::TLay *xl = nullptr, int H = 1) {
    return dtype == NE_BF16 ? ne::launch_rope_bf16(s, x, y, rows, stream)
                            : ne::launch_rope_f32(s, static_cast<const float *>(x),
                                                  static_cast<float *>(y), rows, stream, false,
                                                  xl, H);
}

// The entry points below take an optional `lay` (float32 only): the layouts of the caller's
// tensors, for the attention sub-block, which keeps q, k, v, o and the gradients as rows of its
// projections (null: every tensor contiguous).  Copies the kernels make in the workspace
// (rotated k and q) are contiguous, and `lay` is adjusted to say so.
int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, void *ws, int B,
             int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
             hipStream_t stream, const ne::TLays *lay = nullptr) {
    if (!q || !k || !v || !o || !lse) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    const bool rope = s.rope_base > 0.f;
    if (rope && !ws) return NE_ERR_NULL;
    if (any_misaligned({q, k, v, o, lse}) || (rope && misaligned(ws))) return NE_ERR_ALIGN;
    ne::TLays L{};
    if (lay) {
        L = *lay;
        s.lay = &L;
    }
    const void *kk = k;
    if (rope) {
        // Keys rotated once into the workspace; each query row is rotated as it is loaded.
        void *kr = static_cast<char *>(ws) + ws_layout(s, dtype).kr;
        if (launch_rope(s, dtype, k, kr, (long long)B * Hkv * T, stream, lay ? &lay->k : nullptr,
                        Hkv) != hipSuccess)
            return NE_ERR_HIP;
        kk = kr;
        L.k = ne::contiguous_lay(Hkv, T, D);
    }
    const hipError_t e =
        dtype == NE_BF16
            ? ne::launch_fwd_bf16(s, q, kk, v, o, lse, stream)
            : ne::launch_fwd_f32(s, static_cast<const float *>(q), static_cast<const float *>(kk),
                                 static_cast<const float *>(v), static_cast<float *>(o), lse,
                                 stream);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

int dq_impl(const void *q, const void *k, const void *v, const void *o, const float *lse,
            const void *dO, void *dq, void *ws, int B, int Hq, int Hkv, int T, int D, int causal,
            int dtype, float rope_base, hipStream_t stream, const ne::TLays *lay = nullptr) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !ws) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k, v, o, lse, dO, dq, ws})) return NE_ERR_ALIGN;
    const WsLayout L = ws_layout(s, dtype);
    ne::TLays TL{};
    if (lay) {
        TL = *lay;
        s.lay = &TL;
    }
    float *delta = static_cast<float *>(ws);
    const void *kk = k;
    void *qr = nullptr;
    if (s.rope_base > 0.f) {
        // Keys rotated once into the workspace for both passes; the dQ pass rotates each query
        // row as it loads it and leaves the rotated rows in the workspace for the dK/dV pass.
        void *kr = static_cast<char *>(ws) + L.kr;
        if (launch_rope(s, dtype, k, kr, (long long)B * Hkv * T, stream, lay ? &lay->k : nullptr,
                        Hkv) != hipSuccess)
            return NE_ERR_HIP;
        kk = kr;
        TL.k = ne::contiguous_lay(Hkv, T, D);
        qr = static_cast<char *>(ws) + L.qr;
    }
    const hipError_t e =
        dtype == NE_BF16
            ? ne::launch_dq_bf16(s, q, kk, v, o, lse, dO, dq, delta, qr, stream)
            : ne::launch_dq_f32(s, static_cast<const float *>(q), static_cast<const float *>(kk),
                                static_cast<const float *>(v), static_cast<const float *>(o), lse,
                                static_cast<const float *>(dO), static_cast<float *>(dq), delta,
                                static_cast<float *>(qr), stream);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

int dkdv_impl(const void *q, const void *k, const void *v, const float *lse, const void *dO,
              const void *ws, void *dk, void *dv, int B, int Hq, int Hkv, int T, int D,
              int causal, int dtype, float rope_base, hipStream_t stream,
              const ne::TLays *lay = nullptr) {
    if (!q || !k || !v || !lse || !dO || !ws || !dk || !dv) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k, v, lse, dO, ws, dk, dv})) return NE_ERR_ALIGN;
    const WsLayout L = ws_layout(s, dtype);
    ne::TLays TL{};
    if (lay) {
        TL = *lay;
        s.lay = &TL;
    }
    const float *delta = static_cast<const float *>(ws);
    const void *qq = q, *kk = k;
    if (s.rope_base > 0.f) {  // rotated by the dQ pass
        qq = static_cast<const char *>(ws) + L.qr;
        kk = static_cast<const char *>(ws) + L.kr;
        TL.q = ne::contiguous_lay(Hq, T, D);
        TL.k = ne::contiguous_lay(Hkv, T, D);
    }
    const hipError_t e =
        dtype == NE_BF16
            ? ne::launch_dkdv_bf16(s, qq, kk, v, lse, dO, delta, dk, dv, stream)
            : ne::launch_dkdv_f32(s, static_cast<const float *>(qq), static_cast<const float *>(kk),
                                  static_cast<const float *>(v), lse,
                                  static_cast<const float *>(dO), delta,
                                  static_cast<float *>(dk), static_cast<float *>(dv), stream);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

int bwd_impl(const void *q, const void *k, const void *v, const void *o, const float *lse,
             const void *dO, void *dq, void *dk, void *dv, void *ws, int B, int Hq, int Hkv,
             int T, int D, int causal, int dtype, float rope_base, hipStream_t stream,
             const ne::TLays *lay = nullptr) {
    // Check everything (including dk, dv) before the first pass is enqueued.
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !ws) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k, v, o, lse, dO, dq, dk, dv, ws})) return NE_ERR_ALIGN;
    const int r1 = dq_impl(q, k, v, o, lse, dO, dq, ws, B, Hq, Hkv, T, D, causal, dtype,
                           rope_base, stream, lay);
    if (r1 != NE_OK) return r1;
    return dkdv_impl(q, k, v, lse, dO, ws, dk, dv, B, Hq, Hkv, T, D, causal, dtype, rope_base,
                     stream, lay);
}

int bwd_fused_impl(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, void *dq, void *dk, void *dv, void *ws, int B, int Hq, int Hkv,
                   int T, int D, int causal, int dtype, float rope_base, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !ws) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (dtype != NE_F32) return NE_ERR_UNSUPPORTED;
    if (any_misaligned({q, k, v, o, lse, dO, dq, dk, dv, ws})) return NE_ERR_ALIGN;
    const WsLayout L = ws_layout(s, dtype);  // delta; with RoPE the rotated k and q
    char *w = static_cast<char *>(ws);
    const bool rope = s.rope_base > 0.f;
    const hipError_t e = ne::launch_bwd_fused_f32(
        s, static_cast<const float *>(q), static_cast<const float *>(k),
        static_cast<const float *>(v), static_cast<const float *>(o), lse,
        static_cast<const float *>(dO), static_cast<float *>(dq), static_cast<float *>(dk),
        static_cast<float *>(dv), reinterpret_cast<float *>(w + L.delta),
        rope ? reinterpret_cast<float *>(w + L.qr) : nullptr,
        rope ? reinterpret_cast<float *>(w + L.kr) : nullptr, stream);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

// Scratch of ne_attn_bwd_noalloc: a file-scope device array (each device that runs it holds its
// own copy until the process ends) standing in for the workspace of ne_attn_bwd_ex.  In host
// code `scratch` names a host-side stand-in, never the device memory: kernels get the address
// hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex scratch_mu;
void *scratch_dev[64] = {};

// Device address of the current device's copy of `scratch`, looked up once per device (with
// that device current) and kept; nullptr if the lookup fails.
void *scratch_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_dev[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        scratch_dev[dev] = p;
    }
    return scratch_dev[dev];
}

int bwd_noalloc_impl(const void *q, const void *k, const void *v, const void *o,
                     const float *lse, const void *dO, void *dq, void *dk, void *dv, int B, int Hq,
                     int Hkv, int T, int D, int causal, int dtype, float rope_base,
                     hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (ws_layout(s, dtype).total > kNoAllocScratchBytes) return NE_ERR_SCRATCH;
    if (any_misaligned({q, k, v, o, lse, dO, dq, dk, dv})) return NE_ERR_ALIGN;
    void *ws = scratch_ptr();
    if (!ws) return NE_ERR_HIP;
    // Every byte of the scratch that the passes read is written first by the dQ pass (delta,
    // rotated q) or the RoPE pre-pass before it (rotated k): nothing needs clearing.
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, ws, B, Hq, Hkv, T, D, causal, dtype,
                    rope_base, stream);
}

// Attention sub-block workspace (float32): what the forward saves for the backward (the
// normalised rows, the projection rows [B T][(Hq + 2 Hkv) D] that hold q, k, v, the attention
// output rows [B T][Hq D] and lse), the attention workspace, then the backward's scratch (the
// gradient of the projection rows, one [B T][Hq D] buffer for d(o rows) then dxn, the RMSNorm
// partial sums) and the rocBLAS scratch; each region 256-aligned.  The attention kernels read
// and write these rows in place (strided), so no tensor is repacked into heads.
struct BlkLayout {
    size_t xn, rstd, qkv, o, lse, attn, dqkv, rows_b, part, blas, total;
};

BlkLayout blk_layout(const ne::Shape &s) {
    const size_t N = (size_t)s.B * s.T, C = (size_t)s.Hq * s.D;
    const size_t W = (size_t)(s.Hq + 2 * s.Hkv) * s.D;
    BlkLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t at = off; off += up256(bytes); return at; };
    L.xn = take(4 * N * C);
    L.rstd = take(4 * N);
    L.qkv = take(4 * N * W);
    L.o = take(4 * N * C);
    L.lse = take(4 * N * s.Hq);
    L.attn = take(ws_layout(s, NE_F32).total);
    L.dqkv = take(4 * N * W);
    L.rows_b = take(4 * N * C);
    L.part = take(4 * (size_t)ne::rmsnorm_bwd_blocks((long long)N) * C);
    L.blas = take(ne::kBlasWorkspaceBytes);  // rocBLAS workspace of the projections
    L.total = off;
    return L;
}

// Layout of H heads of D columns inside rows of `width` elements: (b, h, t, d) at
// (b T + t) width + h D + d (the head's first column is added to the tensor's pointer).
ne::TLay rows_lay(int T, int width, int D) {
    return ne::TLay{(long long)T * width, (unsigned)D, width};
}

int blk_check(int B, int T, int Hq, int Hkv, int D, float eps, float rope_base, ne::Shape &s) {
    const int rc = check_shape(B, Hq, Hkv, T, D, 1, NE_F32, rope_base, s);
    if (rc != NE_OK) return rc;
    if (!(eps > 0.f) || !isfinite(eps)) return NE_ERR_UNSUPPORTED;
    const long long C = (long long)Hq * D, W = (long long)(Hq + 2 * Hkv) * D;
    const long long N = (long long)B * T;
    // C <= 8192: the RMSNorm backward keeps four rows of C floats in LDS (128 KB).  The
    // attention kernels index a batch element's projection rows in 32 bits: T W < 2^31.
    if (C > 8192 || W > 0x7fffffffLL / 4 || N > 0x7fffffffLL || N * W > (1LL << 40) ||
        (long long)T * W > 0x7fffffffLL)
        return NE_ERR_SHAPE;
    return NE_OK;
}

// Decode workspace: the splits' outputs then their lse, each region 256-aligned.
struct DecLayout {
    size_t part_lse, total;
};

DecLayout dec_layout(int B, int Hq, int Tc, int D) {
    const size_t ns = (size_t)ne::decode_splits(Tc);
    DecLayout L{};
    L.part_lse = up256(4 * ns * (size_t)B * (size_t)Hq * (size_t)D);
    L.total = L.part_lse + up256(4 * ns * (size_t)B * (size_t)Hq);
    return L;
}

int decode_check(int B, int Hq, int Hkv, int Tc, int D, int dtype, ne::Shape &s) {
    const int rc = check_shape(B, Hq, Hkv, Tc, D, 0, dtype, 0.f, s);
    if (rc != NE_OK) return rc;
    // Work-groups per split: (batch, key/value head, chunk of up to 8 query heads).
    const long long gy = (long long)B * Hkv * ((s.G + 7) / 8);
    if (gy > 65535) return NE_ERR_SHAPE;
    if ((long long)B * Hq > 0x7fffffffLL) return NE_ERR_SHAPE;  // merge: a work-group per row
    return NE_OK;
}

}  // namespace

extern "C" {

int ne_attn_fwd(const float *q, const float *k, const float *v, float *o, float *lse, int B,
                int Hq, int Hkv, int T, int D, int causal, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, nullptr, B, Hq, Hkv, T, D, causal, NE_F32, 0.f, stream);
}

int ne_attn_bwd(const float *q, const float *k, const float *v, const float *o, const float *lse,
                const float *dO, float *dq, float *dk, float *dv, float *delta_ws, int B, int Hq,
                int Hkv, int T, int D, int causal, hipStream_t stream) {
    // Without RoPE the workspace is the delta region alone.
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, delta_ws, B, Hq, Hkv, T, D, causal, NE_F32,
                    0.f, stream);
}

int ne_attn_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                   void *workspace, int B, int Hq, int Hkv, int T, int D, int causal, int dtype,
                   float rope_base, hipStream_t stream) {
    return fwd_impl(q, k, v, o, lse, workspace, B, Hq, Hkv, T, D, causal, dtype, rope_base,
                    stream);
}

int ne_attn_bwd_ex(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dO, void *dq, void *dk, void *dv, void *workspace, int B, int Hq,
                   int Hkv, int T, int D, int causal, int dtype, float rope_base,
                   hipStream_t stream) {
    return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, workspace, B, Hq, Hkv, T, D, causal, dtype,
                    rope_base, stream);
}

int ne_attn_bwd_dq_ex(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dO, void *dq, void *workspace, int B, int Hq,
                      int Hkv, int T, int D, int causal, int dtype, float rope_base,
                      hipStream_t stream) {
    return dq_impl(q, k, v, o, lse, dO, dq, workspace, B, Hq, Hkv, T, D, causal, dtype,
                   rope_base, stream);
}

int ne_attn_bwd_dkdv_ex(const void *q, const void *k, const void *v, const float *lse,
                        const void *dO, const void *workspace, void *dk, void *dv, int B, int Hq,
                        int Hkv, int T, int D, int causal, int dtype, float rope_base,
                        hipStream_t stream) {
    return dkdv_impl(q, k, v, lse, dO, workspace, dk, dv, B, Hq, Hkv, T, D, causal, dtype,
                     rope_base, stream);
}

int ne_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                        const float *lse, const void *dO, void *dq, void *dk, void *dv, int B,
                        int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
                        hipStream_t stream) {
    return bwd_noalloc_impl(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, T, D, causal, dtype,
                            rope_base, stream);
}

int ne_attn_bwd_fused(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dO, void *dq, void *dk, void *dv,
                      void *workspace, int B, int Hq, int Hkv, int T, int D, int causal,
                      int dtype, float rope_base, hipStream_t stream) {
    return bwd_fused_impl(q, k, v, o, lse, dO, dq, dk, dv, workspace, B, Hq, Hkv, T, D, causal,
                          dtype, rope_base, stream);
}

size_t ne_attn_block_workspace_bytes(int B, int T, int Hq, int Hkv, int D, float rope_base) {
    ne::Shape s;
    if (blk_check(B, T, Hq, Hkv, D, 1e-5f, rope_base, s) != NE_OK) return 0;
    return blk_layout(s).total;
}

int ne_attn_block_fwd(const float *x, const float *gamma, const float *w_qkv, const float *w_o,
                      float *y, void *workspace, int B, int T, int Hq, int Hkv, int D, float eps,
                      float rope_base, hipStream_t stream) {
    if (!x || !gamma || !w_qkv || !w_o || !y || !workspace) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = blk_check(B, T, Hq, Hkv, D, eps, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({x, gamma, w_qkv, w_o, y, workspace})) return NE_ERR_ALIGN;
    const BlkLayout L = blk_layout(s);
    char *w = static_cast<char *>(workspace);
    auto F = [&](size_t off) { return reinterpret_cast<float *>(w + off); };
    const long long N = (long long)B * T;
    const int C = Hq * D, W = (Hq + 2 * Hkv) * D;
    void *bw = w + L.blas;
    const size_t bn = ne::kBlasWorkspaceBytes;
    // xn = rmsnorm(x); [q | k | v] rows = xn w_qkv
    hipError_t e = ne::launch_rmsnorm_fwd(x, gamma, F(L.xn), F(L.rstd), N, C, eps, stream);
    if (e == hipSuccess) e = ne::gemm_rm(stream, bw, bn, false, false, (int)N, W, C, F(L.xn), w_qkv, F(L.qkv), 0.f);
    if (e != hipSuccess) return NE_ERR_HIP;
    // attention straight on the projection rows, o written as rows
    const ne::TLay lq = rows_lay(T, W, D), lo = rows_lay(T, C, D);
    const ne::TLays lay{lq, lq, lq, lo, lo, lq, lq, lq};
    const float *q = F(L.qkv), *k = q + (size_t)Hq * D, *v = k + (size_t)Hkv * D;
    const int ra = fwd_impl(q, k, v, F(L.o), F(L.lse), w + L.attn, B, Hq, Hkv, T, D, 1, NE_F32,
                            rope_base, stream, &lay);
    if (ra != NE_OK) return ra;
    // y = x + (o rows) w_o
    e = hipMemcpyAsync(y, x, sizeof(float) * (size_t)N * C, hipMemcpyDeviceToDevice, stream);
    if (e == hipSuccess) e = ne::gemm_rm(stream, bw, bn, false, false, (int)N, C, C, F(L.o), w_o, y, 1.f);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

int ne_attn_block_bwd(const float *x, const float *gamma, const float *w_qkv, const float *w_o,
                      const float *dy, float *dx, float *dgamma, float *dw_qkv, float *dw_o,
                      void *workspace, int B, int T, int Hq, int Hkv, int D, float eps,
                      float rope_base, hipStream_t stream) {
    if (!x || !gamma || !w_qkv || !w_o || !dy || !dx || !dgamma || !dw_qkv || !dw_o || !workspace)
        return NE_ERR_NULL;
    ne::Shape s;
    const int rc = blk_check(B, T, Hq, Hkv, D, eps, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({x, gamma, w_qkv, w_o, dy, dx, dgamma, dw_qkv, dw_o, workspace}))
        return NE_ERR_ALIGN;
    const BlkLayout L = blk_layout(s);
    char *w = static_cast<char *>(workspace);
    auto F = [&](size_t off) { return reinterpret_cast<float *>(w + off); };
    const long long N = (long long)B * T;
    const int C = Hq * D, W = (Hq + 2 * Hkv) * D;
    void *bw = w + L.blas;
    const size_t bn = ne::kBlasWorkspaceBytes;
    // d(o rows) = dy w_o^T;  dw_o = (o rows)^T dy
    hipError_t e = ne::gemm_rm(stream, bw, bn, false, true, (int)N, C, C, dy, w_o, F(L.rows_b), 0.f);
    if (e == hipSuccess) e = ne::gemm_rm(stream, bw, bn, true, false, C, C, (int)N, F(L.o), dy, dw_o, 0.f);
    if (e != hipSuccess) return NE_ERR_HIP;
    // the attention backward on the rows: q, k, v and o as the forward left them, dO = d(o rows),
    // dq, dk, dv written as the rows of d[q | k | v]
    const ne::TLay lq = rows_lay(T, W, D), lo = rows_lay(T, C, D);
    const ne::TLays lay{lq, lq, lq, lo, lo, lq, lq, lq};
    const float *q = F(L.qkv), *k = q + (size_t)Hq * D, *v = k + (size_t)Hkv * D;
    float *dq = F(L.dqkv), *dk = dq + (size_t)Hq * D, *dv = dk + (size_t)Hkv * D;
    const int ra = bwd_impl(q, k, v, F(L.o), F(L.lse), F(L.rows_b), dq, dk, dv, w + L.attn, B, Hq,
                            Hkv, T, D, 1, NE_F32, rope_base, stream, &lay);
    if (ra != NE_OK) return ra;
    // dw_qkv = xn^T d[q | k | v];  dxn = d[q | k | v] w_qkv^T;  RMSNorm backward
    e = ne::gemm_rm(stream, bw, bn, true, false, C, W, (int)N, F(L.xn), F(L.dqkv), dw_qkv, 0.f);
    if (e == hipSuccess) e = ne::gemm_rm(stream, bw, bn, false, true, (int)N, C, W, F(L.dqkv), w_qkv, F(L.rows_b), 0.f);
    if (e == hipSuccess)
        e = ne::launch_rmsnorm_bwd(x, gamma, F(L.rstd), F(L.rows_b), dy, dx, F(L.part), dgamma, N, C, stream);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

size_t ne_attn_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int dtype,
                               float rope_base) {
    ne::Shape s;
    if (check_shape(B, Hq, Hkv, T, D, 1, dtype, rope_base, s) != NE_OK) return 0;
    return ws_layout(s, dtype).total;
}

int ne_attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *lens,
                   void *o, float *lse, void *workspace, int B, int Hq, int Hkv, int Tc, int D,
                   int dtype, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !lens || !o || !lse || !workspace) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = decode_check(B, Hq, Hkv, Tc, D, dtype, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k_cache, v_cache, lens, o, lse, workspace})) return NE_ERR_ALIGN;
    const DecLayout L = dec_layout(B, Hq, Tc, D);
    float *part_o = static_cast<float *>(workspace);
    float *part_lse = reinterpret_cast<float *>(static_cast<char *>(workspace) + L.part_lse);
    return ne::launch_decode(s, dtype == NE_BF16, q, k_cache, v_cache, lens, o, lse, part_o,
                             part_lse, stream) == hipSuccess
               ? NE_OK
               : NE_ERR_HIP;
}

int ne_attn_prefill(const void *q, const void *k_cache, const void *v_cache, void *o, float *lse,
                    int B, int Hq, int Hkv, int Tq, int Tk, int D, int dtype, hipStream_t stream) {
    if (!q || !k_cache || !v_cache || !o || !lse) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, Tq, D, 1, dtype, 0.f, s);
    if (rc != NE_OK) return rc;
    if (Tk < Tq || Tk > (1 << 24) || (double)B * Hkv * Tk * D > 9.0e15) return NE_ERR_SHAPE;
    if (dtype == NE_BF16 && !bf16_head_fits(Tk, D)) return NE_ERR_SHAPE;
    if (any_misaligned({q, k_cache, v_cache, o, lse})) return NE_ERR_ALIGN;
    s.Tk = Tk;
    const hipError_t e =
        dtype == NE_BF16
            ? ne::launch_fwd_bf16(s, q, k_cache, v_cache, o, lse, stream)
            : ne::launch_fwd_f32(s, static_cast<const float *>(q),
                                 static_cast<const float *>(k_cache),
                                 static_cast<const float *>(v_cache), static_cast<float *>(o), lse,
                                 stream);
    return e == hipSuccess ? NE_OK : NE_ERR_HIP;
}

size_t ne_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Tc, int D, int dtype) {
    ne::Shape s;
    if (decode_check(B, Hq, Hkv, Tc, D, dtype, s) != NE_OK) return 0;
    return dec_layout(B, Hq, Tc, D).total;
}

size_t ne_attn_bwd_workspace_bytes(int B, int Hq, int T) {
    if (B < 1 || Hq < 1 || T < 1) return 0;
    return (size_t)4 * (size_t)B * (size_t)Hq * (size_t)T;
}

const char *ne_attn_strerror(int status) {
    switch (status) {
        case NE_OK: return "success";
        case NE_ERR_NULL: return "null pointer argument";
        case NE_ERR_SHAPE: return "invalid shape (B, Hq, Hkv, T must be >= 1, Hq a multiple of Hkv, sizes in range)";
        case NE_ERR_UNSUPPORTED: return "unsupported configuration (D must be 32, 64 or 128, dtype NE_F32 or NE_BF16, rope_base finite and >= 0)";
        case NE_ERR_ALIGN: return "pointer not 16-byte aligned";
        case NE_ERR_HIP: return "HIP kernel launch failed";
        case NE_ERR_SCRATCH: return "the shape needs more scratch than the library's static buffer holds (64 MiB)";
        default: return "unknown status";
    }
}

}  // extern "C"
