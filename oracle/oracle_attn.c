/*
 * oracle_attn.c -- plain, slow, fp64 CPU oracle for causal grouped-query softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load this file;
 * only the test-suite, the smoke check and the CPU-baseline leg of the benchmark use it.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes, and where that is stated:
 *   - The attention kernel of NanoEuler is an exact softmax attention computed tile by tile
 *     with an online softmax and without ever holding the T x T score matrix
 *     ("nanoeuler: un LLM estilo GPT-2 construido desde cero en C y CUDA", second paragraph;
 *     "NanoEuler -- Show HN" Japanese README translation, section "Kernels and acceleration").
 *     Tiling and the online softmax only reorder the arithmetic, so the oracle is the plain
 *     definition: s = q.k / sqrt(D), P = softmax over the allowed keys, O = P V.
 *   - Causal: a query sees keys at its own and earlier positions; the upper triangle is
 *     skipped ("NanoEuler: a GPT-2 hand-built in pure C/CUDA" (openai-hub), section on
 *     implementation details, item "causal mask in attention").
 *   - Grouped-query attention: query heads share a smaller set of key/value heads; the GPU
 *     model has 12 query and 4 key/value heads, the CPU model 4 and 2 (README translations,
 *     sections "Architecture" and the configuration table).  Reading: contiguous groups,
 *     query head h uses key/value head h / (Hq/Hkv).
 *   - RoPE is applied to queries and keys (README translations, section "Architecture").
 *     Reading: rotation of pairs by angle t * base^(-2i/D), t the position; pairs are
 *     (2i, 2i+1) ("interleaved", pairing 0) or (i, i + D/2) ("half split", pairing 1).
 *     The pages fix neither the pairing nor the base; the base is an argument.
 *   - The saved per-row statistic is the natural-log log-sum-exp of the scaled scores,
 *     lse_i = log sum_j exp(s_ij), so that P_ij = exp(s_ij - lse_i).
 *   - Backward: the textbook softmax Jacobian.  dP_ij = dO_i . v_j,
 *     delta_i = sum_j P_ij dP_ij, dS_ij = P_ij (dP_ij - delta_i), dq_i = sum_j dS_ij k_j / sqrt(D),
 *     dk_j = sum over the query heads of the group and over i of dS_ij q_i / sqrt(D),
 *     dv_j = sum over the group and over i of P_ij dO_i.  With RoPE, the gradients of the
 *     rotated vectors are rotated back (transpose of the rotation), so they are gradients with
 *     respect to the caller's un-rotated q and k.  The pages state that every hand-written
 *     backward pass is checked against central finite differences in double precision
 *     (README translations, section "Verifying the backward pass"); the test-suite does the
 *     same to this file.
 *
 * Layout: every tensor is contiguous row-major, q,o,dO,dq: [B][Hq][T][D];
 * k,v,dk,dv: [B][Hkv][T][D]; lse: [B][Hq][T].  All values are double.
 *
 * Return value of every entry point: 0 on success, -1 on an invalid argument, -2 when out of
 * host memory.  Outputs are fully overwritten.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

#define IDX4(a, b, c, d, B_, C_, D_) ((((size_t)(a) * (B_) + (b)) * (C_) + (c)) * (D_) + (d))

static int check_args(int B, int Hq, int Hkv, int T, int D, int rope, int pairing)
{
    if (B < 1 || Hq < 1 || Hkv < 1 || T < 1 || D < 1) return -1;
    if (Hq % Hkv != 0) return -1;
    if (rope && (D % 2 != 0 || (pairing != 0 && pairing != 1))) return -1;
    return 0;
}

/* Rotation of one head's [T][D] block in place.  inverse != 0 applies the transpose. */
static void rope_head(double *x, int T, int D, double base, int pairing, int inverse)
{
    int half = D / 2;
    for (int t = 0; t < T; ++t) {
        double *row = x + (size_t)t * D;
        for (int i = 0; i < half; ++i) {
            double theta = pow(base, -2.0 * (double)i / (double)D);
            double phi = (double)t * theta;
            double c = cos(phi), s = sin(phi);
            int ia = pairing == 0 ? 2 * i : i;
            int ib = pairing == 0 ? 2 * i + 1 : i + half;
            double a = row[ia], b = row[ib];
            if (!inverse) {
                row[ia] = a * c - b * s;
                row[ib] = a * s + b * c;
            } else {
                row[ia] = a * c + b * s;
                row[ib] = -a * s + b * c;
            }
        }
    }
}

/* Applies the rotation to every head of a [B][H][T][D] tensor in place. */
int oracle_rope(double *x, int B, int H, int T, int D, double base, int pairing, int inverse)
{
    if (check_args(B, H, H, T, D, 1, pairing)) return -1;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            rope_head(x + IDX4(b, h, 0, 0, H, T, D), T, D, base, pairing, inverse);
    return 0;
}

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int d = 0; d < n; ++d) s += a[d] * b[d];
    return s;
}

/* Copies q and k, rotating them when rope_base > 0.  Returns 0 or -2. */
static int rotated_copies(const double *q, const double *k, int B, int Hq, int Hkv, int T, int D,
                          double rope_base, int pairing, double **qr, double **kr)
{
    size_t nq = (size_t)B * Hq * T * D, nk = (size_t)B * Hkv * T * D;
    *qr = (double *)malloc(nq * sizeof(double));
    *kr = (double *)malloc(nk * sizeof(double));
    if (!*qr || !*kr) { free(*qr); free(*kr); return -2; }
    memcpy(*qr, q, nq * sizeof(double));
    memcpy(*kr, k, nk * sizeof(double));
    if (rope_base > 0.0) {
        oracle_rope(*qr, B, Hq, T, D, rope_base, pairing, 0);
        oracle_rope(*kr, B, Hkv, T, D, rope_base, pairing, 0);
    }
    return 0;
}

/*
 * Forward.  For every (b, h, i): s_ij = q_i . k_j / sqrt(D) over the allowed keys j
 * (j <= i when causal), m = max_j s_ij, l = sum_j exp(s_ij - m), P_ij = exp(s_ij - m) / l,
 * lse_i = m + log l, o_i = sum_j P_ij v_j.  lse may be NULL.
 */
int oracle_attn_fwd(const double *q, const double *k, const double *v, double *o, double *lse,
                    int B, int Hq, int Hkv, int T, int D, int causal, double rope_base,
                    int rope_pairing)
{
    int rope = rope_base > 0.0;
    if (check_args(B, Hq, Hkv, T, D, rope, rope_pairing)) return -1;
    if (!q || !k || !v || !o) return -1;
    double *qr, *kr;
    if (rotated_copies(q, k, B, Hq, Hkv, T, D, rope_base, rope_pairing, &qr, &kr)) return -2;
    int G = Hq / Hkv;
    double scale = 1.0 / sqrt((double)D);
    int failed = 0;

    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)T * sizeof(double));
        if (!s) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for collapse(3) schedule(dynamic, 16)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < Hq; ++h)
                for (int i = 0; i < T; ++i) {
                    if (!s) continue;
                    int g = h / G;
                    const double *qi = qr + IDX4(b, h, i, 0, Hq, T, D);
                    int n = causal ? i + 1 : T;
                    double m = -INFINITY;
                    for (int j = 0; j < n; ++j) {
                        s[j] = dot(qi, kr + IDX4(b, g, j, 0, Hkv, T, D), D) * scale;
                        if (s[j] > m) m = s[j];
                    }
                    double l = 0.0;
                    for (int j = 0; j < n; ++j) l += exp(s[j] - m);
                    double *oi = o + IDX4(b, h, i, 0, Hq, T, D);
                    for (int d = 0; d < D; ++d) oi[d] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        double p = exp(s[j] - m) / l;
                        const double *vj = v + IDX4(b, g, j, 0, Hkv, T, D);
                        for (int d = 0; d < D; ++d) oi[d] += p * vj[d];
                    }
                    if (lse) lse[((size_t)b * Hq + h) * T + i] = m + log(l);
                }
        free(s);
    }
    free(qr);
    free(kr);
    return failed ? -2 : 0;
}

/*
 * Backward of o with respect to q, k, v for an incoming gradient dO (no gradient flows into
 * lse).  Two plain passes, both straight from the definition:
 *   pass 1, per query row (b, h, i): P_i. (softmax of the row), dP_ij = dO_i . v_j,
 *           delta_i = sum_j P_ij dP_ij, dS_ij = P_ij (dP_ij - delta_i),
 *           dq_i = sum_j dS_ij k_j / sqrt(D); lse_i and delta_i are kept (O(T) per head);
 *   pass 2, per key row (b, g, j): for each query head h of group g and each query i that
 *           sees key j: P_ij = exp(s_ij - lse_i), dS_ij as above,
 *           dk_j += dS_ij q_i / sqrt(D), dv_j += P_ij dO_i.
 * With RoPE the rows of dq and dk are finally rotated back.
 */
int oracle_attn_bwd(const double *q, const double *k, const double *v, const double *dO,
                    double *dq, double *dk, double *dv, int B, int Hq, int Hkv, int T, int D,
                    int causal, double rope_base, int rope_pairing)
{
    int rope = rope_base > 0.0;
    if (check_args(B, Hq, Hkv, T, D, rope, rope_pairing)) return -1;
    if (!q || !k || !v || !dO || !dq || !dk || !dv) return -1;
    double *qr, *kr;
    if (rotated_copies(q, k, B, Hq, Hkv, T, D, rope_base, rope_pairing, &qr, &kr)) return -2;
    size_t nl = (size_t)B * Hq * T;
    double *lse = (double *)malloc(nl * sizeof(double));
    double *delta = (double *)malloc(nl * sizeof(double));
    if (!lse || !delta) {
        free(qr); free(kr); free(lse); free(delta);
        return -2;
    }
    int G = Hq / Hkv;
    double scale = 1.0 / sqrt((double)D);
    int failed = 0;

    /* pass 1: rows */
    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)T * sizeof(double));
        double *dp = (double *)malloc((size_t)T * sizeof(double));
        if (!s || !dp) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for collapse(3) schedule(dynamic, 16)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < Hq; ++h)
                for (int i = 0; i < T; ++i) {
                    if (!s || !dp) continue;
                    int g = h / G;
                    const double *qi = qr + IDX4(b, h, i, 0, Hq, T, D);
                    const double *doi = dO + IDX4(b, h, i, 0, Hq, T, D);
                    int n = causal ? i + 1 : T;
                    double m = -INFINITY;
                    for (int j = 0; j < n; ++j) {
                        s[j] = dot(qi, kr + IDX4(b, g, j, 0, Hkv, T, D), D) * scale;
                        if (s[j] > m) m = s[j];
                    }
                    double l = 0.0;
                    for (int j = 0; j < n; ++j) l += exp(s[j] - m);
                    double dl = 0.0; /* delta_i = sum_j P_ij dP_ij */
                    for (int j = 0; j < n; ++j) {
                        s[j] = exp(s[j] - m) / l; /* s now holds P_ij */
                        dp[j] = dot(doi, v + IDX4(b, g, j, 0, Hkv, T, D), D);
                        dl += s[j] * dp[j];
                    }
                    double *dqi = dq + IDX4(b, h, i, 0, Hq, T, D);
                    for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        double ds = s[j] * (dp[j] - dl);
                        const double *kj = kr + IDX4(b, g, j, 0, Hkv, T, D);
                        for (int d = 0; d < D; ++d) dqi[d] += ds * kj[d] * scale;
                    }
                    size_t r = ((size_t)b * Hq + h) * T + i;
                    lse[r] = m + log(l);
                    delta[r] = dl;
                }
        free(s);
        free(dp);
    }

    /* pass 2: key rows */
    #pragma omp parallel for collapse(3) schedule(dynamic, 16)
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < Hkv; ++g)
            for (int j = 0; j < T; ++j) {
                const double *kj = kr + IDX4(b, g, j, 0, Hkv, T, D);
                const double *vj = v + IDX4(b, g, j, 0, Hkv, T, D);
                double *dkj = dk + IDX4(b, g, j, 0, Hkv, T, D);
                double *dvj = dv + IDX4(b, g, j, 0, Hkv, T, D);
                for (int d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
                for (int h = g * G; h < (g + 1) * G; ++h)
                    for (int i = causal ? j : 0; i < T; ++i) {
                        const double *qi = qr + IDX4(b, h, i, 0, Hq, T, D);
                        const double *doi = dO + IDX4(b, h, i, 0, Hq, T, D);
                        size_t r = ((size_t)b * Hq + h) * T + i;
                        double p = exp(dot(qi, kj, D) * scale - lse[r]);
                        double ds = p * (dot(doi, vj, D) - delta[r]);
                        for (int d = 0; d < D; ++d) {
                            dkj[d] += ds * qi[d] * scale;
                            dvj[d] += p * doi[d];
                        }
                    }
            }

    if (rope) {
        oracle_rope(dq, B, Hq, T, D, rope_base, rope_pairing, 1);
        oracle_rope(dk, B, Hkv, T, D, rope_base, rope_pairing, 1);
    }
    free(qr);
    free(kr);
    free(lse);
    free(delta);
    return failed ? -2 : 0;
}

/*
 * Decode step against a key/value cache.  The pages say the attention supports a KV cache for
 * autoregressive generation ("NanoEuler" article on ainews.cool, section "technical deep
 * dive", attention item) and list GPU generation among the program's modes (Japanese README
 * translation, command list).  Reading: one new query per (batch, query head); it sees the
 * cached keys 0 .. lens[b] - 1 of its key/value head, which already include its own position,
 * so no further mask applies.  It is the last row of causal attention over a sequence of
 * length lens[b] whose final query is q (the test-suite checks exactly that).  Any RoPE has
 * been applied to q and to the cached keys by the caller.
 *
 * q, o: [B][Hq][D]; k, v: [B][Hkv][Tc][D] (the cache, Tc >= every lens[b]); lse: [B][Hq];
 * lens: [B].  lens[b] = 0 gives o = 0 and lse = -inf.
 */
int oracle_attn_decode(const double *q, const double *k, const double *v, const int *lens,
                       double *o, double *lse, int B, int Hq, int Hkv, int Tc, int D)
{
    if (check_args(B, Hq, Hkv, Tc, D, 0, 0)) return -1;
    if (!q || !k || !v || !lens || !o) return -1;
    for (int b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > Tc) return -1;
    int G = Hq / Hkv;
    double scale = 1.0 / sqrt((double)D);
    int failed = 0;

    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Tc * sizeof(double));
        if (!s) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for collapse(2) schedule(dynamic, 4)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < Hq; ++h) {
                if (!s) continue;
                int g = h / G, n = lens[b];
                const double *qh = q + ((size_t)b * Hq + h) * D;
                double *oh = o + ((size_t)b * Hq + h) * D;
                for (int d = 0; d < D; ++d) oh[d] = 0.0;
                double m = -INFINITY;
                for (int j = 0; j < n; ++j) {
                    s[j] = dot(qh, k + IDX4(b, g, j, 0, Hkv, Tc, D), D) * scale;
                    if (s[j] > m) m = s[j];
                }
                double l = 0.0;
                for (int j = 0; j < n; ++j) l += exp(s[j] - m);
                for (int j = 0; j < n; ++j) {
                    double p = exp(s[j] - m) / l;
                    const double *vj = v + IDX4(b, g, j, 0, Hkv, Tc, D);
                    for (int d = 0; d < D; ++d) oh[d] += p * vj[d];
                }
                if (lse) lse[(size_t)b * Hq + h] = n > 0 ? m + log(l) : -INFINITY;
            }
        free(s);
    }
    return failed ? -2 : 0;
}

/*
 * Prefill of a chunk of Tq new queries against a cache that already holds Tk - Tq earlier
 * positions plus the chunk's own (Tk keys in all): query i of the chunk is at position
 * i + Tk - Tq and, causally, sees keys 0 .. i + Tk - Tq.  Reading: the generation mode the pages
 * mention (KV cache for autoregressive generation: "NanoEuler" article on ainews.cool, section
 * "technical deep dive") processes a prompt, or a continuation, in chunks; with Tq = Tk this is
 * the causal forward, with Tq = 1 a decode step.  The test-suite pins both.  Any RoPE has been
 * applied by the caller.
 *
 * q, o: [B][Hq][Tq][D]; k, v: [B][Hkv][Tk][D]; lse: [B][Hq][Tq].  1 <= Tq <= Tk.
 */
int oracle_attn_prefill(const double *q, const double *k, const double *v, double *o,
                        double *lse, int B, int Hq, int Hkv, int Tq, int Tk, int D)
{
    if (check_args(B, Hq, Hkv, Tk, D, 0, 0) || Tq < 1 || Tq > Tk) return -1;
    if (!q || !k || !v || !o) return -1;
    int G = Hq / Hkv, off = Tk - Tq;
    double scale = 1.0 / sqrt((double)D);
    int failed = 0;

    #pragma omp parallel
    {
        double *s = (double *)malloc((size_t)Tk * sizeof(double));
        if (!s) {
            #pragma omp atomic write
            failed = 1;
        }
        #pragma omp for collapse(3) schedule(dynamic, 16)
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < Hq; ++h)
                for (int i = 0; i < Tq; ++i) {
                    if (!s) continue;
                    int g = h / G, n = i + off + 1;
                    const double *qi = q + IDX4(b, h, i, 0, Hq, Tq, D);
                    double m = -INFINITY;
                    for (int j = 0; j < n; ++j) {
                        s[j] = dot(qi, k + IDX4(b, g, j, 0, Hkv, Tk, D), D) * scale;
                        if (s[j] > m) m = s[j];
                    }
                    double l = 0.0;
                    for (int j = 0; j < n; ++j) l += exp(s[j] - m);
                    double *oi = o + IDX4(b, h, i, 0, Hq, Tq, D);
                    for (int d = 0; d < D; ++d) oi[d] = 0.0;
                    for (int j = 0; j < n; ++j) {
                        double p = exp(s[j] - m) / l;
                        const double *vj = v + IDX4(b, g, j, 0, Hkv, Tk, D);
                        for (int d = 0; d < D; ++d) oi[d] += p * vj[d];
                    }
                    if (lse) lse[((size_t)b * Hq + h) * Tq + i] = m + log(l);
                }
        free(s);
    }
    return failed ? -2 : 0;
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    int n = 1;
    #pragma omp parallel
    {
        #pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}
