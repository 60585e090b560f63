/*
 * lit_oracle.c -- plain fp64 CPU oracle for the sparse-attention step
 * (lightning indexer -> per-query top-k -> attention over window + selected rows).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * helper with the HIP library: it decodes the byte formats itself, loops over
 * the definitions in the order the pages state them, and accumulates in double.
 * It is deliberately slow and unblocked so that every line can be checked
 * against the pages by eye.
 *
 * Sources (cited by page title and symbol):
 *   [V4.1] DeepSeek-V4.1-Flash-NVFP4, inference/model.py
 *          module globals (fp8 block size, ue8m0 scale format), get_window_topk_idxs,
 *          Indexer.forward, Attention._window_kv, Attention.forward.
 *   [V3.2] DeepSeek-V3.2-Exp, inference/model.py
 *          Indexer.forward (fp8_index over e4m3 keys with block scales),
 *          MLA.forward (dense scores + index mask + softmax: the brute-force form).
 *
 * Every function returns 0 on success and a negative code for an argument it
 * refuses (documented per function); nothing here aborts.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void);

#define ORC_E_ARG (-1)   /* a size or pointer argument is invalid  */
#define ORC_E_CODE (-2)  /* a NaN-coded fp8 / e8m0 byte was met     */
#define ORC_E_INDEX (-3) /* an index list entry is out of range     */

/* ------------------------------------------------------------------------ */
/* Byte formats.  [V4.1] module globals: the activation format is e4m3 with  */
/* one power-of-two (ue8m0) scale per 32 elements; the indexer's fp4 format  */
/* is e2m1 with the same scales.                                             */
/* ------------------------------------------------------------------------ */

/* OCP e4m3fn: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities; exponent 15 with mantissa 7 is NaN; exponent 0 is subnormal. */
double orc_e4m3(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* OCP e2m1 (MXFP4 element), one 4-bit code: 1 sign bit, 2 exponent bits (bias
 * 1), 1 mantissa bit, no infinities or NaN; exponent 0 is subnormal (0 or 0.5).
 * [V4.1] quantises the index queries and keys to this format with one ue8m0
 * scale per 32 elements (fp4 block size 32, Indexer.forward). */
double orc_e2m1(uint8_t code) {
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v;
    if (e == 0)
        v = (double)m / 2.0;
    else
        v = ldexp(1.0 + (double)m / 2.0, e - 1);
    return s ? -v : v;
}

/* ue8m0: an unsigned biased exponent, value 2^(c-127); 255 is NaN. */
double orc_e8m0(uint8_t code) {
    if (code == 255) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double orc_bf16(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------ */
/* Visibility.  [V4.1] Indexer.forward: compressed row j covers tokens        */
/* j*r .. j*r+r-1 and becomes visible once the query has passed its last      */
/* token, so a query at absolute position P sees rows j < (P+1)//r.  The     */
/* prefill form there (arange(1, S+1)//r) and the decode form (end_pos//r)   */
/* are the cases start_pos == 0 and S == 1 of this rule.                     */
/* ------------------------------------------------------------------------ */
int orc_n_visible(int start_pos, int i, int ratio) {
    if (ratio <= 0) return 0;
    return (start_pos + i + 1) / ratio;
}

/* ------------------------------------------------------------------------ */
/* Indexer score.  [V4.1] Indexer.forward: index_score[b,s,t] =              */
/*   sum_h  w[b,s,h] * relu( q[b,s,h,:] . k[b,t,:] ),                        */
/* with q and k the dequantised values ([V3.2] fp8_index takes the e4m3      */
/* codes and their block scales; [V4.1] quantises both to fp4 with the same  */
/* 32-element ue8m0 blocks).  Each operand is dequantised per block of 32    */
/* along the head dimension: x = code * 2^(scale-127).                       */
/*                                                                           */
/* fmt selects the element codes: ORC_FMT_E4M3, one byte per element, or    */
/* ORC_FMT_E2M1, two elements per byte with element 2j in the low nibble of  */
/* byte j (the order is a reading: the pages store two fp4 values per byte   */
/* without saying which comes first; a score does not depend on it as long   */
/* as q and k share it, since both nibbles of a byte lie in one scale block).*/
/*                                                                           */
/* Layouts (row-major), E = Di for e4m3 and Di/2 for e2m1: q8 [B,S,Hi,E],    */
/* q_sc [B,S,Hi,Di/32], w [B,S,Hi] f32, k8 [B,T_cap,E], k_sc [B,T_cap,Di/32].*/
/* Output scores [B,S,T] doubles with T = (start_pos+S)//ratio; entries of   */
/* rows a query cannot see are -inf.  Returns ORC_E_ARG for bad sizes or an  */
/* unknown fmt, ORC_E_CODE for a NaN code.                                   */
/* ------------------------------------------------------------------------ */
#define ORC_FMT_E4M3 0
#define ORC_FMT_E2M1 1

/* Value of element d of a code row in format fmt (scale not applied). */
static double orc_code_at(const uint8_t *row, int fmt, int d) {
    if (fmt == ORC_FMT_E2M1) {
        uint8_t byte = row[d / 2];
        uint8_t nib = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
        return orc_e2m1(nib);
    }
    return orc_e4m3(row[d]);
}

int orc_index_scores(int fmt, const uint8_t *q8, const uint8_t *q_sc, const float *w,
                     const uint8_t *k8, const uint8_t *k_sc, int B, int S,
                     int Hi, int Di, int T_cap, int start_pos, int ratio,
                     double *scores) {
    if (B < 0 || S < 0 || Hi <= 0 || Di <= 0 || Di % 32 != 0 || ratio <= 0 ||
        start_pos < 0 || (fmt != ORC_FMT_E4M3 && fmt != ORC_FMT_E2M1))
        return ORC_E_ARG;
    const int T = (start_pos + S) / ratio;
    if (T > T_cap) return ORC_E_ARG;
    const int nb = Di / 32;
    const size_t E = fmt == ORC_FMT_E2M1 ? (size_t)Di / 2 : (size_t)Di; /* bytes per row */
    int bad = 0;
    const size_t nq = (size_t)B * S;
    /* every query's heads, dequantised */
    double *qall = (double *)malloc(sizeof(double) * (nq > 0 ? nq : 1) * (size_t)Hi * Di);
    if (!qall) return ORC_E_ARG;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (size_t qi = 0; qi < nq; ++qi) {
        double *qh = qall + qi * (size_t)Hi * Di;
        for (int h = 0; h < Hi; ++h)
            for (int d = 0; d < Di; ++d) {
                const uint8_t *qrow = q8 + (qi * Hi + h) * E;
                size_t si = (qi * Hi + h) * nb + d / 32;
                double v = orc_code_at(qrow, fmt, d) * orc_e8m0(q_sc[si]);
                if (isnan(v)) bad = 1;
                qh[(size_t)h * Di + d] = v;
            }
    }
    /* one score per (query, row); the loops over (b, i, t) are independent */
#pragma omp parallel for collapse(3) schedule(static) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < S; ++i) {
            for (int t = 0; t < T; ++t) {
                const int nvis = orc_n_visible(start_pos, i, ratio);
                const double *qh = qall + ((size_t)b * S + i) * (size_t)Hi * Di;
                double *srow = scores + ((size_t)b * S + i) * T;
                if (t >= nvis) {
                    srow[t] = -INFINITY;
                    continue;
                }
                double s = 0.0;
                for (int h = 0; h < Hi; ++h) {
                    double dot = 0.0;
                    for (int d = 0; d < Di; ++d) {
                        const uint8_t *krow = k8 + ((size_t)b * T_cap + t) * E;
                        size_t ks = ((size_t)b * T_cap + t) * nb + d / 32;
                        double kv = orc_code_at(krow, fmt, d) * orc_e8m0(k_sc[ks]);
                        if (isnan(kv)) bad = 1;
                        dot += qh[(size_t)h * Di + d] * kv;
                    }
                    double wh = (double)w[((size_t)b * S + i) * Hi + h];
                    s += wh * (dot > 0.0 ? dot : 0.0);
                }
                srow[t] = s;
            }
        }
    }
    free(qall);
    return bad ? ORC_E_CODE : 0;
}

/* ------------------------------------------------------------------------ */
/* Top-k.  [V4.1] Indexer.forward: k_eff = min(index_topk, end_pos//r); the  */
/* k_eff best scores are taken, their row numbers listed in ascending order, */
/* and a pick the query cannot see becomes -1 (which, being a larger row     */
/* number than every visible one, sorts to the end).                         */
/*                                                                           */
/* Here the picks are made among the visible rows only, ordered by score     */
/* descending and, for equal scores, by row ascending (the pages leave ties  */
/* open; this is the reading taken).  The first min(k_eff, n_visible) rows   */
/* are emitted in ascending row order and the rest of the k_eff slots are    */
/* -1.  scores: [B,S,ld] doubles.  idx: [B,S,k_eff] int32.                   */
/* ------------------------------------------------------------------------ */
typedef struct {
    double s;
    int t;
} orc_pick;

static int orc_pick_cmp(const void *a, const void *b) {
    const orc_pick *x = (const orc_pick *)a, *y = (const orc_pick *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int orc_int_cmp(const void *a, const void *b) {
    int x = *(const int *)a, y = *(const int *)b;
    return (x > y) - (x < y);
}

int orc_topk_width(int S, int start_pos, int ratio, int index_topk) {
    if (ratio <= 0 || index_topk < 0) return 0;
    int T = (start_pos + S) / ratio;
    return index_topk < T ? index_topk : T;
}

int orc_topk(const double *scores, int ld, int B, int S, int start_pos,
             int ratio, int index_topk, int32_t *idx) {
    if (B < 0 || S < 0 || ratio <= 0 || index_topk < 0 || start_pos < 0)
        return ORC_E_ARG;
    const int T = (start_pos + S) / ratio;
    if (ld < T) return ORC_E_ARG;
    const int keff = orc_topk_width(S, start_pos, ratio, index_topk);
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < S; ++i) {
            const double *srow = scores + ((size_t)b * S + i) * ld;
            int32_t *orow = idx + ((size_t)b * S + i) * keff;
            int nvis = orc_n_visible(start_pos, i, ratio);
            if (nvis > T) nvis = T;
            orc_pick *p = (orc_pick *)malloc(sizeof(orc_pick) * (size_t)(nvis > 0 ? nvis : 1));
            int *sel = (int *)malloc(sizeof(int) * (size_t)(keff > 0 ? keff : 1));
            for (int t = 0; t < nvis; ++t) {
                p[t].s = srow[t];
                p[t].t = t;
                if (isnan(srow[t])) bad = 1;
            }
            qsort(p, (size_t)nvis, sizeof(orc_pick), orc_pick_cmp);
            int take = keff < nvis ? keff : nvis;
            for (int j = 0; j < take; ++j) sel[j] = p[j].t;
            qsort(sel, (size_t)take, sizeof(int), orc_int_cmp);
            for (int j = 0; j < keff; ++j) orow[j] = j < take ? sel[j] : -1;
            free(p);
            free(sel);
        }
    }
    return bad ? ORC_E_ARG : 0;
}

/* ------------------------------------------------------------------------ */
/* Candidate blocks: level one of the two-level top-k.  [V4.1]               */
/* select_candidate_blocks, with Indexer.forward's compress_lens:            */
/*   1. the score row (width T, -inf where the query cannot see) is padded   */
/*      with -inf to a multiple of block_size;                               */
/*   2. each block scores the max of its positions;                          */
/*   3. the block holding the query's newest visible row, (n_vis-1) //       */
/*      block_size, is set to +inf (none when n_vis == 0: Python's floor     */
/*      division gives block -1);                                            */
/*   4. the min(topk_blocks, n_blocks) best blocks are taken -- ties by the  */
/*      lower block, a reading: the pages' topk leaves ties open -- and any  */
/*      taken block whose score is -inf is dropped.                          */
/* The pages return this as a mask over positions; here it is the list of    */
/* kept block numbers in ascending order, -1 padded to                       */
/* kb = min(topk_blocks, n_blocks) per query, n_blocks = ceil(T/block_size). */
/* Level two ([V4.1] Indexer.forward, uses_candidates) sets every score      */
/* outside the kept blocks to -inf and runs the ordinary top-k.              */
/* scores: [B,S,ld] doubles; blocks: [B,S,kb] int32.                         */
/* ------------------------------------------------------------------------ */
int orc_candidate_blocks_width(int S, int start_pos, int ratio, int topk_blocks,
                               int block_size) {
    if (ratio <= 0 || block_size <= 0 || topk_blocks < 0) return 0;
    const int T = (start_pos + S) / ratio;
    const int nblocks = (T + block_size - 1) / block_size;
    return topk_blocks < nblocks ? topk_blocks : nblocks;
}

int orc_candidate_blocks(const double *scores, int ld, int B, int S, int start_pos,
                         int ratio, int topk_blocks, int block_size, int32_t *blocks) {
    if (B < 0 || S < 0 || ratio <= 0 || topk_blocks < 0 || block_size <= 0 ||
        start_pos < 0)
        return ORC_E_ARG;
    const int T = (start_pos + S) / ratio;
    if (ld < T) return ORC_E_ARG;
    const int nblocks = (T + block_size - 1) / block_size;
    const int kb = orc_candidate_blocks_width(S, start_pos, ratio, topk_blocks, block_size);
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < S; ++i) {
            const double *srow = scores + ((size_t)b * S + i) * ld;
            int32_t *orow = blocks + ((size_t)b * S + i) * kb;
            const int nvis = orc_n_visible(start_pos, i, ratio);
            orc_pick *p = (orc_pick *)malloc(sizeof(orc_pick) * (size_t)(nblocks > 0 ? nblocks : 1));
            int *sel = (int *)malloc(sizeof(int) * (size_t)(kb > 0 ? kb : 1));
            for (int j = 0; j < nblocks; ++j) {
                double m = -INFINITY; /* the -inf padding of the last block */
                for (int t = j * block_size; t < (j + 1) * block_size && t < T; ++t) {
                    if (isnan(srow[t])) bad = 1;
                    if (srow[t] > m) m = srow[t];
                }
                p[j].s = m;
                p[j].t = j;
            }
            if (nvis >= 1 && (nvis - 1) / block_size < nblocks)
                p[(nvis - 1) / block_size].s = INFINITY;
            qsort(p, (size_t)nblocks, sizeof(orc_pick), orc_pick_cmp);
            int take = 0;
            for (int j = 0; j < kb; ++j)
                if (p[j].s > -INFINITY) sel[take++] = p[j].t;
            qsort(sel, (size_t)take, sizeof sel[0], orc_int_cmp); /* ascending blocks */
            for (int j = 0; j < kb; ++j) orow[j] = j < take ? sel[j] : -1;
            free(p);
            free(sel);
        }
    }
    return bad ? ORC_E_ARG : 0;
}

/* ------------------------------------------------------------------------ */
/* Window rows.  [V4.1] get_window_topk_idxs and Attention._window_kv: a     */
/* query at absolute position P attends to the window positions              */
/* max(0, P-W+1) .. P.  The window source is a ring of R slots holding       */
/* position p in slot p mod R.                                               */
/*   * start_pos == 0 (prefill of the chunk itself): each row has             */
/*     min(S, W) entries, positions max(0, i-W+1) + j, and an entry past the */
/*     query (p > i) is -1.                                                  */
/*   * start_pos > 0: each row has W entries, positions P-W+1+j oldest       */
/*     first, and a position before the sequence start is -1.  With S == 1  */
/*     and R == W this is the decode ring of the pages; with S > 1 it is the */
/*     chunked-prefill generalisation (requires R >= W + S - 1 so that no    */
/*     two needed positions share a slot).                                   */
/* win_idx: [B,S,width] int32, the same for every b.                         */
/* ------------------------------------------------------------------------ */
int orc_window_width(int S, int start_pos, int W) {
    if (W <= 0) return 0;
    if (start_pos == 0) return S < W ? S : W;
    return W;
}

int orc_window_indices(int B, int S, int start_pos, int W, int R,
                       int32_t *win_idx) {
    if (B < 0 || S < 0 || W < 0 || start_pos < 0 || R <= 0) return ORC_E_ARG;
    const int width = orc_window_width(S, start_pos, W);
    const long need = start_pos == 0 ? (long)S : (long)W + S - 1;
    if (width > 0 && R < (need < (long)start_pos + S ? need : (long)start_pos + S))
        return ORC_E_ARG;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < S; ++i) {
            int32_t *row = win_idx + ((size_t)b * S + i) * width;
            const long P = (long)start_pos + i;
            for (int j = 0; j < width; ++j) {
                long p;
                int valid;
                if (start_pos == 0) {
                    long base = P - W + 1 > 0 ? P - W + 1 : 0;
                    p = base + j;
                    valid = p <= P;
                } else {
                    p = P - W + 1 + j;
                    valid = p >= 0;
                }
                row[j] = valid ? (int32_t)(p % R) : -1;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Attention.  [V4.1] Attention.forward hands sparse_attn the concatenation  */
/* of the window KV and the compressed KV plus the concatenated index lists; */
/* one KV row serves as both key and value (a single shared latent head).    */
/* [V3.2] MLA.forward gives the dense form: scores over positions, -inf      */
/* outside the index set, softmax, weighted sum of values.                   */
/*                                                                           */
/* For each (b, i, h): J = the window rows listed in win_idx (slots of       */
/* win_kv) followed by the compressed rows listed in comp_idx (rows of       */
/* comp_kv); -1 entries are skipped, repeats are kept.  l_j = scale * q.kv_j  */
/* over all D dims; with an optional per-head sink logit s_h:                 */
/*   m = max(l_j, s_h),  Z = sum_j e^(l_j-m) + e^(s_h-m),                     */
/*   o[d] = sum_j e^(l_j-m) kv_j[d] / Z   for d < dv.                        */
/* The sink enters the normaliser only (the pages pass attn_sink without     */
/* stating its role; this is the reading taken).  Empty J gives o = 0.       */
/* Two passes over J (max, then sums): the plain definition, not the online  */
/* recurrence a kernel would use.                                            */
/*                                                                           */
/* KV rows come in one of three forms, each source with its own:             */
/*   ORC_KV_BF16: bf16 bits, rows of D;                                      */
/*   ORC_KV_E4M3: e4m3 codes, rows of D bytes, with one ue8m0 scale per 32   */
/*     ([V4.1] Attention._window_kv quantises the window KV with act_quant,  */
/*     fp8 block size 32, ue8m0 scales, over the whole post-RoPE row);       */
/*   ORC_KV_E2M1: fp4 codes, rows of D/2 bytes (element 2j in the low        */
/*     nibble of byte j), with one e4m3 scale per 16 ([V4.1]                 */
/*     Attention._compress_kv quantises the compressed KV with fp4_act_quant */
/*     in groups of 16 with e4m3 scales).                                    */
/* A row's values are code * scale, decoded exactly in double.               */
/*                                                                           */
/* Layouts: q [B,S,H,D] bf16 bits; win_kv [B,R,*] with win_sc [B,R,*];       */
/* win_idx [B,S,W]; comp_kv [B,T_cap,*] with comp_sc [B,T_cap,*];            */
/* comp_idx [B,S,K]; sink [H] float or NULL; out [B,S,H,dv] doubles.         */
/* Returns ORC_E_INDEX for an entry out of range, ORC_E_ARG for bad sizes.   */
/* ------------------------------------------------------------------------ */
#define ORC_KV_BF16 0
#define ORC_KV_E4M3 1
#define ORC_KV_E2M1 2

/* Row `row` of a KV source, decoded into v[0..D). */
static void orc_kv_row(int fmt, const void *data, const uint8_t *sc, size_t row, int D,
                       double *v) {
    if (fmt == ORC_KV_E4M3) {
        const uint8_t *c = (const uint8_t *)data + row * (size_t)D;
        const uint8_t *s = sc + row * (size_t)(D / 32);
        for (int d = 0; d < D; ++d) v[d] = orc_e4m3(c[d]) * orc_e8m0(s[d / 32]);
    } else if (fmt == ORC_KV_E2M1) {
        const uint8_t *c = (const uint8_t *)data + row * (size_t)(D / 2);
        const uint8_t *s = sc + row * (size_t)(D / 16);
        for (int d = 0; d < D; ++d) {
            uint8_t nib = (d % 2 == 0) ? (c[d / 2] & 15) : (c[d / 2] >> 4);
            v[d] = orc_e2m1(nib) * orc_e4m3(s[d / 16]);
        }
    } else {
        const uint16_t *r = (const uint16_t *)data + row * (size_t)D;
        for (int d = 0; d < D; ++d) v[d] = orc_bf16(r[d]);
    }
}

int orc_sparse_attn_fmt(const uint16_t *q, int B, int S, int H, int D, int dv,
                        int win_fmt, const void *win_kv, const uint8_t *win_sc, int R,
                        const int32_t *win_idx, int W, int comp_fmt, const void *comp_kv,
                        const uint8_t *comp_sc, int T_cap, const int32_t *comp_idx, int K,
                        const float *sink, double scale, double *out) {
    if (B < 0 || S < 0 || H <= 0 || D <= 0 || dv <= 0 || dv > D || W < 0 ||
        K < 0)
        return ORC_E_ARG;
    if ((W > 0 && (win_kv == NULL || win_idx == NULL || R <= 0)) ||
        (K > 0 && (comp_kv == NULL || comp_idx == NULL || T_cap <= 0)))
        return ORC_E_ARG;
    if (win_fmt < ORC_KV_BF16 || win_fmt > ORC_KV_E2M1 || comp_fmt < ORC_KV_BF16 ||
        comp_fmt > ORC_KV_E2M1)
        return ORC_E_ARG;
    if ((W > 0 && win_fmt != ORC_KV_BF16 && (win_sc == NULL || D % 32 != 0)) ||
        (K > 0 && comp_fmt != ORC_KV_BF16 && (comp_sc == NULL || D % 32 != 0)))
        return ORC_E_ARG;
    int bad = 0;
    /* queries in parallel when there are enough of them, else the heads of each query */
    const int par_q = (long)B * S >= orc_num_threads();
#pragma omp parallel for collapse(2) schedule(dynamic) reduction(| : bad) if (par_q)
    for (int b = 0; b < B; ++b) {
        for (int i = 0; i < S; ++i) {
            const int n = W + K;
            double *kv = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)D);
            int nj = 0;
            for (int j = 0; j < W; ++j) {
                int32_t s = win_idx[((size_t)b * S + i) * W + j];
                if (s < 0) continue;
                if (s >= R) { bad = 1; continue; }
                orc_kv_row(win_fmt, win_kv, win_sc, (size_t)b * R + s, D, kv + (size_t)nj++ * D);
            }
            for (int j = 0; j < K; ++j) {
                int32_t t = comp_idx[((size_t)b * S + i) * K + j];
                if (t < 0) continue;
                if (t >= T_cap) { bad = 1; continue; }
                orc_kv_row(comp_fmt, comp_kv, comp_sc, (size_t)b * T_cap + t, D, kv + (size_t)nj++ * D);
            }
#pragma omp parallel for schedule(static) if (!par_q)
            for (int h = 0; h < H; ++h) {
                const uint16_t *qh = q + (((size_t)b * S + i) * H + h) * D;
                double *oh = out + (((size_t)b * S + i) * H + h) * dv;
                for (int d = 0; d < dv; ++d) oh[d] = 0.0;
                if (nj == 0) continue;
                double *l = (double *)malloc(sizeof(double) * (size_t)nj);
                double m = -INFINITY;
                for (int j = 0; j < nj; ++j) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d) dot += orc_bf16(qh[d]) * kv[(size_t)j * D + d];
                    l[j] = scale * dot;
                    if (l[j] > m) m = l[j];
                }
                double sk = sink ? (double)sink[h] : -INFINITY;
                if (sk > m) m = sk;
                double Z = sink ? exp(sk - m) : 0.0;
                for (int j = 0; j < nj; ++j) Z += exp(l[j] - m);
                for (int j = 0; j < nj; ++j) {
                    double p = exp(l[j] - m) / Z;
                    for (int d = 0; d < dv; ++d) oh[d] += p * kv[(size_t)j * D + d];
                }
                free(l);
            }
            free(kv);
        }
    }
    return bad ? ORC_E_INDEX : 0;
}

/* The bf16 form of both sources. */
int orc_sparse_attn(const uint16_t *q, int B, int S, int H, int D, int dv,
                    const uint16_t *win_kv, int R, const int32_t *win_idx,
                    int W, const uint16_t *comp_kv, int T_cap,
                    const int32_t *comp_idx, int K, const float *sink,
                    double scale, double *out) {
    return orc_sparse_attn_fmt(q, B, S, H, D, dv, ORC_KV_BF16, win_kv, NULL, R, win_idx, W,
                               ORC_KV_BF16, comp_kv, NULL, T_cap, comp_idx, K, sink, scale, out);
}

/* ------------------------------------------------------------------------ */
/* Producer side: the cache writes of one decode step.                       */
/*                                                                           */
/* [V4.1] Compressor.forward (decode): the new token's kv and gate score     */
/* (fp32, after the wkv / wgate projections, which are outside the path)     */
/* fill slot start_pos % ratio of the sequence's kv_state / score_state; when */
/* the group completes ((start_pos + 1) % ratio == 0) the latent is           */
/* sum over slots of kv_state * softmax(score_state over the slots), per     */
/* feature, cast to bf16 and RMS-normalised (RMSNorm.forward: x / sqrt(mean  */
/* x^2 + eps) times the weight, computed in float, result in bf16).  Ratio 1 */
/* has no state: the latent is the norm of the token's kv (cast to bf16).    */
/* [V4.1] Attention._compress_kv then rotates the latent's last rd dims at   */
/* position start_pos + 1 - ratio (apply_rotary_emb: adjacent pairs as       */
/* complex numbers times freqs_cis, result back in bf16), quantises it with  */
/* fp4_act_quant in groups of 16 with e4m3 scales and writes cache row       */
/* start_pos / ratio.  [V4.1] Attention._window_kv: the token's window KV    */
/* (after kv_norm) is rotated at start_pos, quantised with act_quant (e4m3,  */
/* ue8m0 scale per 32) and written to ring slot start_pos % R.               */
/*                                                                           */
/* The quantisers' rounding is not on the pages (their kernels are absent);  */
/* the readings taken, with every decision made exactly:                     */
/*   e4m3 / ue8m0: scale 2^e with e the smallest integer such that           */
/*     amax <= 448 * 2^e (amax 0: e = -127); code = x / 2^e rounded to the   */
/*     nearest e4m3 value, ties to the even code;                            */
/*   e2m1 / e4m3: scale s the smallest e4m3 value with 6 s >= amax (amax 0:  */
/*     the smallest positive e4m3, code 1; amax > 6 * 448: 448); code = the  */
/*     e2m1 value nearest to x / s, ties to the even code, sign of x kept.   */
/* Intermediate values are exact (double) and rounded to bf16 where the      */
/* pages store bf16: after the cast of the pooled kv, after the norm, after  */
/* the rotation -- except the rotation itself, which the pages compute in    */
/* fp32 (apply_rotary_emb: x.float() viewed as complex64 times freqs_cis):   */
/* there each product and the sum or difference is rounded to fp32 in turn,  */
/* no fused multiply-add (the plainest fp32 reading), then to bf16.  The     */
/* pooling and the norm are fp32 on the pages too, but their last bits       */
/* depend on the exp / rsqrt implementation and the summation order, which   */
/* the pages do not fix; the exact values are kept here (and returned        */
/* unrounded, so that a test can see how close to a bf16 rounding midpoint a  */
/* value lies).  freqs: [positions, rd/2, 2] floats (cos, sin), as           */
/* precompute_freqs_cis tabulates them.                                      */
/* ------------------------------------------------------------------------ */

/* Round to the nearest bfloat16 value (8 significant bits), ties to even. */
double orc_round_bf16(double x) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    double a = fabs(x);
    double r;
    if (a < ldexp(1.0, -126)) { /* subnormal spacing 2^-133 */
        r = ldexp(nearbyint(ldexp(a, 133)), -133);
    } else {
        int e;
        double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
        r = ldexp(nearbyint(ldexp(m, 8)), e - 8);
    }
    return x < 0 ? -r : r;
}

/* e4m3 code of y, |y| <= 448, to nearest (ties to the even code). */
uint8_t orc_e4m3_encode(double y) {
    int neg = y < 0 || (y == 0 && signbit(y));
    double a = fabs(y);
    int code;
    if (a > 448.0) a = 448.0;
    if (a < ldexp(1.0, -6)) {
        code = (int)nearbyint(ldexp(a, 9)); /* subnormal steps of 2^-9 (8 = 2^-6) */
    } else {
        int e = ilogb(a);
        int q = (int)nearbyint((ldexp(a, -e) - 1.0) * 8.0);
        if (q == 8) { ++e; q = 0; }
        code = ((e + 7) << 3) | q;
    }
    return (uint8_t)(code | (neg ? 0x80 : 0));
}

/* e2m1 code (4 bits) of x / s, to nearest (ties to the even code). */
static uint8_t orc_e2m1_encode_scaled(double x, double s) {
    double a = fabs(x);
    int c = (a > 0.25 * s) + (a >= 0.75 * s) + (a > 1.25 * s) + (a >= 1.75 * s) +
            (a > 2.5 * s) + (a >= 3.5 * s) + (a > 5.0 * s);
    return (uint8_t)(c | (x < 0 ? 8 : 0));
}

/* Quantise D values (D % 32 == 0) into e4m3 codes with ue8m0 scales per 32. */
void orc_quant_e4m3(const double *x, int D, uint8_t *codes, uint8_t *scales) {
    for (int b0 = 0; b0 < D; b0 += 32) {
        double amax = 0.0;
        for (int d = b0; d < b0 + 32; ++d) if (fabs(x[d]) > amax) amax = fabs(x[d]);
        int e = -127;
        if (amax > 0.0) {
            e = ilogb(amax) - 9;
            while (amax > 448.0 * ldexp(1.0, e)) ++e;
            while (e > -127 && amax <= 448.0 * ldexp(1.0, e - 1)) --e;
        }
        if (e > 127) e = 127;
        scales[b0 / 32] = (uint8_t)(e + 127);
        for (int d = b0; d < b0 + 32; ++d) codes[d] = orc_e4m3_encode(ldexp(x[d], -e));
    }
}

/* Quantise D values (D % 16 == 0) into packed e2m1 codes with e4m3 scales per 16. */
void orc_quant_e2m1(const double *x, int D, uint8_t *codes, uint8_t *scales) {
    for (int b0 = 0; b0 < D; b0 += 16) {
        double amax = 0.0;
        for (int d = b0; d < b0 + 16; ++d) if (fabs(x[d]) > amax) amax = fabs(x[d]);
        int sc = 1; /* positive e4m3 values rise with the code */
        while (sc < 0x7E && 6.0 * orc_e4m3((uint8_t)sc) < amax) ++sc;
        scales[b0 / 16] = (uint8_t)sc;
        double s = orc_e4m3((uint8_t)sc);
        for (int d = b0; d < b0 + 16; d += 2) {
            uint8_t lo = orc_e2m1_encode_scaled(x[d], s), hi = orc_e2m1_encode_scaled(x[d + 1], s);
            codes[d / 2] = (uint8_t)(lo | (hi << 4));
        }
    }
}

/* RMSNorm of D values (each already a bf16 value), result rounded to bf16;  */
/* raw (may be NULL) receives the values before that rounding.               */
static void orc_rmsnorm_bf16(const double *x, const float *w, int D, double eps, double *y, double *raw) {
    double ss = 0.0;
    for (int d = 0; d < D; ++d) ss += x[d] * x[d];
    double r = 1.0 / sqrt(ss / D + eps);
    for (int d = 0; d < D; ++d) {
        const double v = (double)w[d] * (x[d] * r);
        if (raw) raw[d] = v;
        y[d] = orc_round_bf16(v);
    }
}

/* Rotate the last rd of D bf16 values at table row `pos`: the complex product */
/* in fp32 (products, then their difference / sum, each rounded to fp32),     */
/* then rounded to bf16.                                                      */
static void orc_rope_bf16(double *x, int D, int rd, const float *freqs, int pos) {
    const float *f = freqs + (size_t)pos * rd; /* rd/2 (cos, sin) pairs */
    for (int j = 0; j < rd / 2; ++j) {
        const float a = (float)x[D - rd + 2 * j], b = (float)x[D - rd + 2 * j + 1];
        const float c = f[2 * j], sn = f[2 * j + 1];
        const float ac = a * c, bs = b * sn, as = a * sn, bc = b * c;
        const float re = ac - bs, im = as + bc;
        x[D - rd + 2 * j] = orc_round_bf16((double)re);
        x[D - rd + 2 * j + 1] = orc_round_bf16((double)im);
    }
}

/* The compressed-cache write of one latent (D bf16 values, pre-rotation): rotated at */
/* position pos, quantised to e2m1 / e4m3-16 into one row (codes D/2, scales D/16).   */
int orc_compress_write(int D, const double *latent, const float *freqs, int rd, int pos,
                       uint8_t *codes, uint8_t *scales) {
    if (D <= 0 || D % 32 != 0 || pos < 0 || rd < 0 || rd > D || rd % 2 != 0) return ORC_E_ARG;
    double *y = (double *)malloc(sizeof(double) * (size_t)D);
    for (int d = 0; d < D; ++d) y[d] = latent[d];
    orc_rope_bf16(y, D, rd, freqs, pos);
    orc_quant_e2m1(y, D, codes, scales);
    free(y);
    return 0;
}

/* One decode step of the compressor and the compressed-cache write.  kv, score:
 * [B, D] floats; kv_state, score_state: [B, ratio, D] floats (ratio > 1; updated);
 * codes [B, T_cap, D/2], scales [B, T_cap, D/16] (row start_pos/ratio written when
 * the group completes); latent [B, D] doubles (pre-rotation bf16 values, may be
 * NULL); pooled_raw and norm_raw [B, D] doubles (may be NULL): the pooled kv before
 * its bf16 cast and the norm's result before its bf16 rounding.  Returns 1 when a
 * row was written, 0 when the group is still filling. */
int orc_compress_append(int B, int D, int ratio, int start_pos, const float *kv,
                        const float *score, float *kv_state, float *score_state,
                        const float *norm_w, double eps, const float *freqs, int rd,
                        uint8_t *codes, uint8_t *scales, int T_cap, double *latent,
                        double *pooled_raw, double *norm_raw) {
    if (B < 0 || D <= 0 || D % 32 != 0 || ratio < 1 || start_pos < 0 || rd < 0 ||
        rd > D || rd % 2 != 0)
        return ORC_E_ARG;
    const int done = (start_pos + 1) % ratio == 0;
    const int row = start_pos / ratio;
    if (done && row >= T_cap) return ORC_E_ARG;
    const int pos = start_pos + 1 - ratio; /* the group's first token */
    for (int b = 0; b < B; ++b) {
        const float *k = kv + (size_t)b * D, *g = score + (size_t)b * D;
        double *x = (double *)malloc(sizeof(double) * (size_t)D * 2);
        double *y = x + D;
        if (ratio == 1) {
            for (int d = 0; d < D; ++d) {
                if (pooled_raw) pooled_raw[(size_t)b * D + d] = k[d];
                x[d] = orc_round_bf16(k[d]);
            }
        } else {
            float *ks = kv_state + (size_t)b * ratio * D, *gs = score_state + (size_t)b * ratio * D;
            const int slot = start_pos % ratio;
            for (int d = 0; d < D; ++d) {
                ks[(size_t)slot * D + d] = k[d];
                gs[(size_t)slot * D + d] = g[d];
            }
            if (!done) { free(x); continue; }
            for (int d = 0; d < D; ++d) {
                double m = -INFINITY;
                for (int r = 0; r < ratio; ++r) if (gs[(size_t)r * D + d] > m) m = gs[(size_t)r * D + d];
                double z = 0.0, acc = 0.0;
                for (int r = 0; r < ratio; ++r) {
                    double e = exp((double)gs[(size_t)r * D + d] - m);
                    z += e;
                    acc += e * (double)ks[(size_t)r * D + d];
                }
                if (pooled_raw) pooled_raw[(size_t)b * D + d] = acc / z;
                x[d] = orc_round_bf16(acc / z); /* kv.to(dtype) */
            }
        }
        orc_rmsnorm_bf16(x, norm_w, D, eps, y, norm_raw ? norm_raw + (size_t)b * D : NULL);
        if (latent) for (int d = 0; d < D; ++d) latent[(size_t)b * D + d] = y[d];
        orc_rope_bf16(y, D, rd, freqs, pos);
        orc_quant_e2m1(y, D, codes + ((size_t)b * T_cap + row) * (D / 2),
                       scales + ((size_t)b * T_cap + row) * (D / 16));
        free(x);
    }
    return done;
}

/* One decode step's window-cache write: kv [B, D] bf16 bits (after kv_norm) rotated
 * at start_pos, quantised to e4m3 / ue8m0-32, written to slot start_pos % R of
 * codes [B, R, D] and scales [B, R, D/32]. */
int orc_window_append(int B, int D, int start_pos, const uint16_t *kv, const float *freqs,
                      int rd, int R, uint8_t *codes, uint8_t *scales) {
    if (B < 0 || D <= 0 || D % 32 != 0 || start_pos < 0 || R <= 0 || rd < 0 || rd > D ||
        rd % 2 != 0)
        return ORC_E_ARG;
    const int slot = start_pos % R;
    double *x = (double *)malloc(sizeof(double) * (size_t)D);
    for (int b = 0; b < B; ++b) {
        for (int d = 0; d < D; ++d) x[d] = orc_bf16(kv[(size_t)b * D + d]);
        orc_rope_bf16(x, D, rd, freqs, start_pos);
        orc_quant_e4m3(x, D, codes + ((size_t)b * R + slot) * D, scales + ((size_t)b * R + slot) * (D / 32));
    }
    free(x);
    return 0;
}

/* Threads the OpenMP loops above will use (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
