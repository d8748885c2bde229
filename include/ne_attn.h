/*
 * ne_attn.h -- C ABI of the causal grouped-query FlashAttention library for MI355X (gfx950).
 *
 * What the operation is.  Exact softmax attention of queries against keys and values, computed
 * tile by tile with an online softmax so that the T x T score matrix is never stored, forward
 * and backward, as NanoEuler's hand-written training kernel does ("nanoeuler: un LLM estilo
 * GPT-2 construido desde cero en C y CUDA", second paragraph; "NanoEuler -- Show HN" Japanese
 * README translation, section "Kernels and acceleration").  Queries see only keys at their own
 * and earlier positions when causal, and the upper triangle is skipped, not masked after the
 * fact ("NanoEuler: a GPT-2 hand-built in pure C/CUDA" (openai-hub), implementation details,
 * item "causal mask in attention").  Query heads share a smaller set of key/value heads
 * (grouped-query attention) and RoPE is applied to queries and keys (README translations,
 * section "Architecture").
 *
 *   s_ij   = (R_i q_i) . (R_j k_j) / sqrt(D)        (R = identity without RoPE)
 *   P_ij   = exp(s_ij - lse_i) over keys j <= i (causal) or all j,  lse_i = log sum_j exp(s_ij)
 *   o_i    = sum_j P_ij v_j
 *   backward: gradients of sum(dO * o) with respect to the caller's q, k, v.
 *
 * Layout (all tensors contiguous, row-major, no strides):
 *   q, o, dO, dq : [B][Hq][T][D]        k, v, dk, dv : [B][Hkv][T][D]
 *   lse, delta   : [B][Hq][T]  float32 (natural-log log-sum-exp of the scaled scores)
 *   Query head h reads key/value head h / (Hq / Hkv).  scale = 1 / sqrt(D).
 *   RoPE (rope_base > 0): the pair (x[2i], x[2i+1]) of the row at position t (0..T-1) is rotated
 *   by the angle t * rope_base^(-2i/D).
 *
 * Ownership and memory.  Every pointer is a device pointer owned by the caller; the library
 * allocates and frees nothing, keeps no state and is thread-safe (calls that share a workspace
 * must be ordered).  The one exception is the sub-block, whose products keep a rocBLAS handle
 * per device (see ne_attn_block_fwd).  Outputs (o, lse, dq, dk, dv,
 * delta) are fully overwritten; inputs are never written.  Inputs and outputs must not alias.
 * Pointers must be 16-byte aligned.
 *
 * Streams.  Work is enqueued on `stream` (NULL = the null stream) and the call returns without
 * synchronising.  A fault during execution surfaces at the caller's next synchronisation.
 *
 * Errors.  Every entry point returns an ne_status.  Argument errors are detected before any
 * launch and nothing is enqueued: NE_ERR_NULL (a null pointer), NE_ERR_SHAPE (B, Hq, Hkv or T
 * below 1, Hq not a multiple of Hkv, sizes whose element count overflows, a bf16 head -- T x D
 * elements of one (batch, head) -- of more than 2^31 bytes), NE_ERR_UNSUPPORTED
 * (D not 32, 64 or 128, unknown dtype, negative or non-finite rope_base), NE_ERR_ALIGN (a pointer
 * not 16-byte aligned).  NE_ERR_HIP reports a failed kernel launch.  No C++ exception crosses
 * this interface.
 */
#ifndef NE_ATTN_H
#define NE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own stream handle. */
typedef struct ihipStream_t *hipStream_t;

enum ne_status {
    NE_OK = 0,
    NE_ERR_NULL = 1,
    NE_ERR_SHAPE = 2,
    NE_ERR_UNSUPPORTED = 3,
    NE_ERR_ALIGN = 4,
    NE_ERR_HIP = 5,
    NE_ERR_SCRATCH = 6  /* ne_attn_bwd_noalloc: the shape needs more than its static scratch */
};

enum ne_dtype {
    NE_F32 = 0,  /* float32 tensors, float32 arithmetic (fp32 MFMA) */
    NE_BF16 = 1  /* bfloat16 q, k, v, o, dO, dq, dk, dv; float32 lse/delta; fp32 accumulate */
};

/*
 * Forward, float32, no RoPE.  Writes o [B][Hq][T][D] and lse [B][Hq][T].
 * causal != 0 restricts query i to keys j <= i.
 */
int ne_attn_fwd(const float *q, const float *k, const float *v, float *o, float *lse,
                int B, int Hq, int Hkv, int T, int D, int causal, hipStream_t stream);

/*
 * Backward, float32, no RoPE.  Takes the o and lse written by ne_attn_fwd for the same inputs
 * and causal flag, and the incoming gradient dO.  Writes dq, dk, dv, and uses delta_ws as a
 * caller-owned workspace of ne_attn_bwd_workspace_bytes(B, Hq, T) bytes, into which it writes
 * delta_i = sum_d dO_id * o_id, float32 [B][Hq][T].  No atomics: results are bitwise
 * reproducible run to run.
 */
int ne_attn_bwd(const float *q, const float *k, const float *v, const float *o,
                const float *lse, const float *dO, float *dq, float *dk, float *dv,
                float *delta_ws, int B, int Hq, int Hkv, int T, int D, int causal,
                hipStream_t stream);

/*
 * Forward with a dtype (NE_F32 or NE_BF16) and an optional RoPE prologue on q and k
 * (rope_base > 0; 0 disables it).  Tensors are float* for NE_F32 and bfloat16 (uint16 bit
 * patterns) for NE_BF16; lse is float32 in both.
 *
 * workspace: caller-owned device memory of ne_attn_workspace_bytes(B, Hq, Hkv, T, D, dtype,
 * rope_base) bytes, 16-byte aligned, not aliasing any tensor.  With RoPE the keys are rotated
 * once into it (each query row is rotated as the kernel loads it); without RoPE it is not used
 * and may be NULL.  Its contents on return are unspecified.
 *
 * The workspace argument is the one difference from a forward that takes only tensors: with
 * RoPE, every key is staged into LDS by each of the T / 32 query-tile work-groups of its head
 * group (the bf16 kernels copy tiles from global memory straight into LDS, with no register
 * step where a rotation could happen), so the keys are rotated once per call by a
 * bandwidth-bound pre-pass instead of once per staging: about 6 us at B 16, Hq 16, Hkv 4,
 * T 1024, D 64 in bf16.  Rotating while staging cost about 90 vector instructions per tile and
 * wave; moving the backward's rotation to the same kind of pre-pass took its dK/dV pass at that
 * shape from 180 to 143 us.
 */
int ne_attn_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
                   void *workspace, int B, int Hq, int Hkv, int T, int D, int causal, int dtype,
                   float rope_base, hipStream_t stream);

/*
 * Backward with a dtype and the same RoPE setting as the forward call.  With RoPE, dq and dk
 * are gradients with respect to the un-rotated q and k the caller passed.
 *
 * workspace: caller-owned device memory of ne_attn_workspace_bytes(...) bytes (never NULL),
 * 16-byte aligned, not aliasing any tensor.  It receives delta_i = sum_d dO_id o_id (float32
 * [B][Hq][T], at offset 0) and, with RoPE, the rotated q and k used by both passes.  No
 * atomics: results are bitwise reproducible run to run.
 */
int ne_attn_bwd_ex(const void *q, const void *k, const void *v, const void *o,
                   const float *lse, const void *dO, void *dq, void *dk, void *dv,
                   void *workspace, int B, int Hq, int Hkv, int T, int D, int causal,
                   int dtype, float rope_base, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * or training loops, harnesses that forbid allocation): ne_attn_bwd_ex without the workspace
 * argument.  Its scratch (delta and, with RoPE, the rotated q and k: ne_attn_workspace_bytes(...)
 * bytes) is a static device array of 64 MiB inside the library; each GPU the call runs on
 * holds its own copy until the process ends.  The call allocates nothing.  Its first call on a
 * device looks up that device's copy once (hipGetSymbolAddress, which may make the runtime load
 * the library's device code there): make that first call outside graph capture.
 * A shape whose scratch exceeds 64 MiB returns NE_ERR_SCRATCH before any launch (bf16 with RoPE
 * at B 16, Hq 16, Hkv 4, T 1024, D 64 needs 41 MiB).  All calls on one GPU share its array and
 * nothing in it survives a call that matters to the next: calls that overlap on one GPU (other
 * streams, other host threads) race on it and must be ordered by the caller.  Results are
 * bitwise those of ne_attn_bwd_ex.  Other arguments and errors as for ne_attn_bwd_ex.
 */
int ne_attn_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                        const float *lse, const void *dO, void *dq, void *dk, void *dv, int B,
                        int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
                        hipStream_t stream);

/*
 * The two passes that ne_attn_bwd_ex runs back to back, as separate calls for callers that
 * schedule them themselves or need only dq.  ne_attn_bwd_dq_ex writes dq and fills the
 * workspace (delta and, with RoPE, the rotated q and k); ne_attn_bwd_dkdv_ex reads the
 * workspace and writes dk, dv, and must be ordered after the dq pass that filled it (same
 * stream, or an event), with the same inputs and settings.  Arguments mean what they mean for
 * ne_attn_bwd_ex.
 */
int ne_attn_bwd_dq_ex(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dO, void *dq, void *workspace, int B,
                      int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
                      hipStream_t stream);
int ne_attn_bwd_dkdv_ex(const void *q, const void *k, const void *v, const float *lse,
                        const void *dO, const void *workspace, void *dk, void *dv, int B,
                        int Hq, int Hkv, int T, int D, int causal, int dtype, float rope_base,
                        hipStream_t stream);

/*
 * Single-pass backward, the alternative to the two passes of ne_attn_bwd_ex.  The pages give no
 * backward algorithm ("NanoEuler: a GPT-2 hand-built in pure C/CUDA" (openai-hub),
 * implementation details, and the README translations, section "Verified backward pass",
 * only require that it be exact); this variant
 * computes the same gradients without recomputing the scores and dP in a separate dq pass: the
 * pass over key blocks also forms dS K for dq and adds it with float32 atomics.  A pre-pass
 * writes delta to the workspace and zeroes dq.  Because the additions into dq happen in an
 * order that varies from run to run, dq is not bitwise reproducible (dk and dv are); it agrees
 * with ne_attn_bwd_ex to rounding.
 *
 * Arguments, layouts, ownership and errors as for ne_attn_bwd_ex, with these limits:
 * dtype NE_F32 only (NE_BF16: NE_ERR_UNSUPPORTED).  The workspace is that of
 * ne_attn_bwd_ex, ne_attn_workspace_bytes(B, Hq, Hkv, T, D, NE_F32, rope_base) bytes: delta and,
 * with RoPE, the rotated q and k (dq is summed in the rotated frame and rotated back).
 */
int ne_attn_bwd_fused(const void *q, const void *k, const void *v, const void *o,
                      const float *lse, const void *dO, void *dq, void *dk, void *dv,
                      void *workspace, int B, int Hq, int Hkv, int T, int D, int causal,
                      int dtype, float rope_base, hipStream_t stream);

/*
 * Bytes of the workspace of the _ex entry points: the delta region (4 * B * Hq * T) and, when
 * rope_base > 0, room for rotated copies of q and k in the given dtype, each region rounded up
 * to 256 bytes.  0 if the arguments are invalid (the checks of the entry points).
 */
size_t ne_attn_workspace_bytes(int B, int Hq, int Hkv, int T, int D, int dtype,
                               float rope_base);

/*
 * One decode step against a key/value cache, for autoregressive generation (the pages say the
 * attention supports a KV cache for it: "NanoEuler" article on ainews.cool, section "technical
 * deep dive", attention item).  Each (batch b, query head h) has one new query q[b][h]; it
 * attends to the cached keys j = 0 .. lens[b] - 1 of key/value head h / (Hq / Hkv), which
 * include its own position, so no further mask applies:
 *   s_j = q . k_j / sqrt(D),  lse = log sum_j exp(s_j),  o = sum_j exp(s_j - lse) v_j.
 * Any RoPE must already be applied to q and to the cached keys.
 *
 * q, o: [B][Hq][D]; k_cache, v_cache: [B][Hkv][Tc][D] (Tc = cache capacity); dtype NE_F32 or
 * NE_BF16 for these four (arithmetic in fp32); lse: [B][Hq] float32; lens: [B] int32, in device
 * memory, read by the kernels (a value outside 0 .. Tc is clamped to it; lens[b] = 0 gives
 * o = 0, lse = -inf).  workspace: caller-owned device memory of
 * ne_attn_decode_workspace_bytes(...) bytes (partial results of the splits of the cache; its
 * contents on return are unspecified).  Errors as above; NE_ERR_SHAPE also when
 * B * Hkv * ceil(Hq / Hkv / 8) exceeds 65535.
 */
int ne_attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *lens,
                   void *o, float *lse, void *workspace, int B, int Hq, int Hkv, int Tc, int D,
                   int dtype, hipStream_t stream);

/*
 * Prefill of a chunk of Tq new queries against a key/value cache of Tk positions (Tq <= Tk) that
 * already holds the chunk's own keys and values at its end: query row i is at position
 * i + Tk - Tq and sees keys 0 .. i + Tk - Tq (causal).  With Tq = Tk this is ne_attn_fwd_ex
 * without RoPE; the chunked form serves generation (the KV cache of the pages, as for
 * ne_attn_decode).  Any RoPE must already be applied to q and to the cached keys.
 *
 * q, o: [B][Hq][Tq][D]; k_cache, v_cache: [B][Hkv][Tk][D]; dtype NE_F32 or NE_BF16 for these
 * four; lse: [B][Hq][Tq] float32.  No workspace.  Errors as above; NE_ERR_SHAPE also when
 * Tk < Tq.
 */
int ne_attn_prefill(const void *q, const void *k_cache, const void *v_cache, void *o, float *lse,
                    int B, int Hq, int Hkv, int Tq, int Tk, int D, int dtype, hipStream_t stream);

/*
 * The attention sub-block around the kernel, float32: the pre-norm residual branch of a
 * NanoEuler block, y = x + attn(rmsnorm(x)) ("NanoEuler -- Show HN" Japanese README translation,
 * section "Architecture": RMSNorm pre-normalisation without bias, RoPE on queries and keys,
 * grouped-query attention, x = x + attn(rmsnorm(x))):
 *   r = (mean_c x^2 + eps)^(-1/2),  xn = x r gamma,  [q | k | v] = xn w_qkv,
 *   o = causal GQA attention (RoPE when rope_base > 0),  y = x + o w_o.
 * x, y: [B][T][C] with C = Hq * D; gamma: [C]; w_qkv: [C][(Hq + 2 Hkv) D], columns ordered
 * q heads, then k heads, then v heads, D per head; w_o: [Hq D][C]; all float32, row-major,
 * device memory, 16-byte aligned.  The products run in rocBLAS (a handle per device, created on
 * the first call and kept); the rest in the library's kernels.  Each product binds the shared
 * handle to the caller's stream and to a 32 MiB region of the caller's workspace as rocBLAS
 * scratch, and is enqueued under one lock, so host threads may call these entry points at once,
 * on streams of their own, each with its own workspace.
 *
 * workspace: caller-owned, ne_attn_block_workspace_bytes(...) bytes.  ne_attn_block_fwd leaves
 * in it what ne_attn_block_bwd needs, so the backward must follow a forward with the same
 * inputs and workspace (same stream, or an event).  ne_attn_block_bwd writes dx (including the
 * residual dy), dgamma, dw_qkv and dw_o, all overwritten; results are bitwise reproducible
 * given rocBLAS's own determinism.  Errors as above; NE_ERR_UNSUPPORTED also for eps <= 0,
 * NE_ERR_SHAPE for C above 8192.
 */
size_t ne_attn_block_workspace_bytes(int B, int T, int Hq, int Hkv, int D, float rope_base);
int ne_attn_block_fwd(const float *x, const float *gamma, const float *w_qkv, const float *w_o,
                      float *y, void *workspace, int B, int T, int Hq, int Hkv, int D, float eps,
                      float rope_base, hipStream_t stream);
int ne_attn_block_bwd(const float *x, const float *gamma, const float *w_qkv, const float *w_o,
                      const float *dy, float *dx, float *dgamma, float *dw_qkv, float *dw_o,
                      void *workspace, int B, int T, int Hq, int Hkv, int D, float eps,
                      float rope_base, hipStream_t stream);

/* Bytes of the decode workspace: 4 * S * B * Hq * (D + 1) with S = ceil(Tc / 256), in two
 * regions each rounded up to 256 bytes; 0 if the arguments are invalid. */
size_t ne_attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Tc, int D, int dtype);

/* Bytes of the workspace of ne_attn_bwd: 4 * B * Hq * T (0 if an argument is below 1). */
size_t ne_attn_bwd_workspace_bytes(int B, int Hq, int T);

/* Static, NUL-terminated description of a status code ("unknown status" otherwise). */
const char *ne_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* NE_ATTN_H */
