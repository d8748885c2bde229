// ne_attn_api.hip -- the C ABI declared in include/ne_attn.h: argument checks, then dispatch to
// the gfx950 kernels on the caller's stream.  Nothing here allocates, synchronises or keeps
// state.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/ne_attn.h"
#include "attn_kernels.hpp"

namespace {

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

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

hipError_t launch_rope(const ne::Shape &s, int dtype, const void *x, void *y, long long rows,
                       hipStream_t stream) {
    return dtype == NE_BF16 ? ne::launch_rope_bf16(s, x, y, rows, stream)
                            : ne::launch_rope_f32(s, static_cast<const float *>(x),
                                                  static_cast<float *>(y), rows, stream);
}

int fwd_impl(const void *q, const void *k, const void *v, void *o, float *lse, void *ws, int B,
             int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
             hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    const bool rope = s.rope_base > 0.f;
    if (rope && !ws) return NE_ERR_NULL;
    if (any_misaligned({q, k, v, o, lse}) || (rope && misaligned(ws))) return NE_ERR_ALIGN;
    const void *kk = k;
    if (rope) {
        // Keys rotated once into the workspace; each query row is rotated as it is loaded.
        void *kr = static_cast<char *>(ws) + ws_layout(s, dtype).kr;
        if (launch_rope(s, dtype, k, kr, (long long)B * Hkv * T, stream) != hipSuccess)
            return NE_ERR_HIP;
        kk = kr;
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
            int dtype, float rope_base, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse || !dO || !dq || !ws) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k, v, o, lse, dO, dq, ws})) return NE_ERR_ALIGN;
    const WsLayout L = ws_layout(s, dtype);
    float *delta = static_cast<float *>(ws);
    const void *kk = k;
    void *qr = nullptr;
    if (s.rope_base > 0.f) {
        // Keys rotated once into the workspace for both passes; the dQ pass rotates each query
        // row as it loads it and leaves the rotated rows in the workspace for the dK/dV pass.
        void *kr = static_cast<char *>(ws) + L.kr;
        if (launch_rope(s, dtype, k, kr, (long long)B * Hkv * T, stream) != hipSuccess)
            return NE_ERR_HIP;
        kk = kr;
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
              int causal, int dtype, float rope_base, hipStream_t stream) {
    if (!q || !k || !v || !lse || !dO || !ws || !dk || !dv) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k, v, lse, dO, ws, dk, dv})) return NE_ERR_ALIGN;
    const WsLayout L = ws_layout(s, dtype);
    const float *delta = static_cast<const float *>(ws);
    const void *qq = q, *kk = k;
    if (s.rope_base > 0.f) {  // rotated by the dQ pass
        qq = static_cast<const char *>(ws) + L.qr;
        kk = static_cast<const char *>(ws) + L.kr;
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
             int T, int D, int causal, int dtype, float rope_base, hipStream_t stream) {
    // Check everything (including dk, dv) before the first pass is enqueued.
    if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv || !ws) return NE_ERR_NULL;
    ne::Shape s;
    const int rc = check_shape(B, Hq, Hkv, T, D, causal, dtype, rope_base, s);
    if (rc != NE_OK) return rc;
    if (any_misaligned({q, k, v, o, lse, dO, dq, dk, dv, ws})) return NE_ERR_ALIGN;
    const int r1 = dq_impl(q, k, v, o, lse, dO, dq, ws, B, Hq, Hkv, T, D, causal, dtype,
                           rope_base, stream);
    if (r1 != NE_OK) return r1;
    return dkdv_impl(q, k, v, lse, dO, ws, dk, dv, B, Hq, Hkv, T, D, causal, dtype, rope_base,
                     stream);
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

int ne_attn_bwd_fused(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dO, void *dq, void *dk, void *dv,
                      void *workspace, int B, int Hq, int Hkv, int T, int D, int causal,
                      int dtype, float rope_base, hipStream_t stream) {
    return bwd_fused_impl(q, k, v, o, lse, dO, dq, dk, dv, workspace, B, Hq, Hkv, T, D, causal,
                          dtype, rope_base, stream);
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
        default: return "unknown status";
    }
}

}  // extern "C"
