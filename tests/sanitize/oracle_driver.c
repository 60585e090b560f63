/*
 * oracle_driver.c -- exercises every entry point of oracle/lit_oracle.c on small
 * deterministic inputs, including the edge cases the tests pin (no visible rows,
 * k >= rows, ties, -1 list entries, sinks, both code formats, quantised KV, the
 * producer steps).  Built with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py; any out-of-bounds access, leak of a freed buffer or
 * undefined operation aborts the run.  Values are not checked here (the pins in
 * tests/test_oracle_*.py do that); return codes are.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_index_scores(int fmt, const uint8_t *q8, const uint8_t *q_sc, const float *w,
                     const uint8_t *k8, const uint8_t *k_sc, int B, int S, int Hi, int Di, int T_cap,
                     int start_pos, int ratio, double *scores);
int orc_topk_width(int S, int start_pos, int ratio, int index_topk);
int orc_topk(const double *scores, int ld, int B, int S, int start_pos, int ratio, int index_topk,
             int32_t *idx);
int orc_candidate_blocks_width(int S, int start_pos, int ratio, int topk_blocks, int block_size);
int orc_candidate_blocks(const double *scores, int ld, int B, int S, int start_pos, int ratio,
                         int topk_blocks, int block_size, int32_t *out);
int orc_window_width(int S, int start_pos, int W);
int orc_window_indices(int B, int S, int start_pos, int W, int R, int32_t *out);
int orc_sparse_attn_fmt(const uint16_t *q, int B, int S, int H, int D, int dv, int win_fmt,
                        const void *win_kv, const uint8_t *win_sc, int R, const int32_t *win_idx, int W,
                        int comp_fmt, const void *comp_kv, const uint8_t *comp_sc, int T_cap,
                        const int32_t *comp_idx, int K, const float *sink, double scale, double *out);
int orc_compress_append(int B, int D, int ratio, int start_pos, const float *kv, const float *score,
                        float *kv_state, float *score_state, const float *norm_w, double eps,
                        const float *freqs, int rd, uint8_t *codes, uint8_t *scales, int T_cap,
                        double *latent, double *pooled_raw, double *norm_raw);
int orc_compress_write(int D, const double *latent, const float *freqs, int rd, int pos, uint8_t *codes,
                       uint8_t *scales);
int orc_window_append(int B, int D, int start_pos, const uint16_t *kv, const float *freqs, int rd, int R,
                      uint8_t *codes, uint8_t *scales);
double orc_e4m3(uint8_t c);
double orc_e2m1(uint8_t c);
double orc_e8m0(uint8_t c);
double orc_bf16(uint16_t b);

static uint32_t st = 12345u;
static uint32_t rnd(void) { st = st * 1664525u + 1013904223u; return st >> 8; }

static int failures = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); ++failures; } } while (0)

/* e4m3 codes avoiding the NaN codes 0x7f / 0xff */
static uint8_t e4m3_code(void) { uint8_t c = (uint8_t)rnd(); return (c & 0x7f) == 0x7f ? c - 1 : c; }

static void one_step(int fmt, int B, int S, int start_pos, int ratio, int Hi, int Di, int k, int ties) {
    const int T = (start_pos + S) / ratio, T_cap = T + 3, E = fmt ? Di / 2 : Di, nb = Di / 32;
    uint8_t *q8 = malloc((size_t)B * S * Hi * E), *q_sc = malloc((size_t)B * S * Hi * nb);
    uint8_t *k8 = malloc((size_t)B * T_cap * E + 1), *k_sc = malloc((size_t)B * T_cap * nb + 1);
    float *w = malloc(sizeof(float) * B * S * Hi);
    for (int j = 0; j < B * S * Hi * E; ++j) q8[j] = fmt ? (uint8_t)rnd() : e4m3_code();
    for (int j = 0; j < B * S * Hi * nb; ++j) q_sc[j] = (uint8_t)(120 + rnd() % 10);
    for (int j = 0; j < B * T_cap * E; ++j) k8[j] = ties ? (uint8_t)(0x38 | (rnd() & 0x80)) : (fmt ? (uint8_t)rnd() : e4m3_code());
    for (int j = 0; j < B * T_cap * nb; ++j) k_sc[j] = (uint8_t)(120 + rnd() % 10);
    for (int j = 0; j < B * S * Hi; ++j) w[j] = (float)(rnd() % 1000) / 1000.f;
    double *sc = malloc(sizeof(double) * ((size_t)B * S * T + 1));
    EXPECT(orc_index_scores(fmt, q8, q_sc, w, k8, k_sc, B, S, Hi, Di, T_cap, start_pos, ratio, sc) == 0);
    const int keff = orc_topk_width(S, start_pos, ratio, k);
    int32_t *idx = malloc(sizeof(int32_t) * ((size_t)B * S * keff + 1));
    EXPECT(orc_topk(sc, T, B, S, start_pos, ratio, k, idx) == 0);
    const int kb = orc_candidate_blocks_width(S, start_pos, ratio, 8, 4);
    int32_t *blocks = malloc(sizeof(int32_t) * ((size_t)B * S * kb + 1));
    EXPECT(orc_candidate_blocks(sc, T, B, S, start_pos, ratio, 8, 4, blocks) == 0);
    const int W = 8, R = start_pos == 0 ? (S > 1 ? S : 1) : W + S - 1;
    const int ww = orc_window_width(S, start_pos, W);
    int32_t *win = malloc(sizeof(int32_t) * ((size_t)B * S * ww + 1));
    EXPECT(orc_window_indices(B, S, start_pos, W, R, win) == 0);
    const int H = 16, D = 64, dv = 32;
    uint16_t *q = malloc(sizeof(uint16_t) * B * S * H * D), *wkv = malloc(sizeof(uint16_t) * B * R * D);
    uint16_t *ckv = malloc(sizeof(uint16_t) * ((size_t)B * T_cap * D + 1));
    for (int j = 0; j < B * S * H * D; ++j) q[j] = (uint16_t)(0x3c00 + rnd() % 0x300) ^ (uint16_t)(rnd() & 0x8000);
    for (int j = 0; j < B * R * D; ++j) wkv[j] = (uint16_t)(0x3c00 + rnd() % 0x300);
    for (int j = 0; j < B * T_cap * D; ++j) ckv[j] = (uint16_t)(0x3c00 + rnd() % 0x300);
    if (keff > 0) idx[0] = -1; /* a skipped entry */
    float sink[16];
    for (int h = 0; h < 16; ++h) sink[h] = (float)h - 4.f;
    double *out = malloc(sizeof(double) * B * S * H * dv);
    EXPECT(orc_sparse_attn_fmt(q, B, S, H, D, dv, 0, wkv, NULL, R, win, ww, 0, ckv, NULL, T_cap, idx, keff,
                               sink, 0.125, out) == 0);
    /* quantised sources: window e4m3 + ue8m0/32, compressed e2m1 + e4m3/16 */
    uint8_t *wq = malloc((size_t)B * R * D), *wqs = malloc((size_t)B * R * D / 32);
    uint8_t *cq = malloc((size_t)B * T_cap * D / 2 + 1), *cqs = malloc((size_t)B * T_cap * D / 16 + 1);
    for (int j = 0; j < B * R * D; ++j) wq[j] = e4m3_code();
    for (int j = 0; j < B * R * D / 32; ++j) wqs[j] = (uint8_t)(125 + rnd() % 4);
    for (int j = 0; j < B * T_cap * D / 2; ++j) cq[j] = (uint8_t)rnd();
    for (int j = 0; j < B * T_cap * D / 16; ++j) cqs[j] = (uint8_t)(0x30 + rnd() % 8);
    EXPECT(orc_sparse_attn_fmt(q, B, S, H, D, dv, 1, wq, wqs, R, win, ww, 2, cq, cqs, T_cap, idx, keff,
                               NULL, 0.125, out) == 0);
    free(q8); free(q_sc); free(k8); free(k_sc); free(w); free(sc); free(idx); free(blocks); free(win);
    free(q); free(wkv); free(ckv); free(out); free(wq); free(wqs); free(cq); free(cqs);
}

int main(void) {
    for (int c = 0; c < 256; ++c) { (void)orc_e4m3((uint8_t)c); (void)orc_e8m0((uint8_t)c); }
    for (int c = 0; c < 16; ++c) (void)orc_e2m1((uint8_t)c);
    for (int c = 0; c < 65536; c += 7) (void)orc_bf16((uint16_t)c);
    for (int fmt = 0; fmt < 2; ++fmt) {
        one_step(fmt, 2, 1, 700, 2, 16, 64, 64, 0);    /* decode */
        one_step(fmt, 1, 1, 2, 4, 16, 64, 64, 0);      /* no visible rows */
        one_step(fmt, 1, 1, 30, 1, 32, 128, 100, 0);   /* k above the rows */
        one_step(fmt, 1, 9, 0, 2, 16, 64, 4, 0);       /* prefill from 0 */
        one_step(fmt, 2, 5, 40, 3, 16, 128, 7, 1);     /* chunk after cached tokens, ties */
    }
    /* producer side: a few decode steps of the compressor and the window ring */
    const int B = 2, D = 64, rd = 16, ratio = 4, T_cap = 4, R = 8;
    float kv[B * D], sc[B * D], ks[B * ratio * D], gs[B * ratio * D], nw[D], fr[32 * rd];
    for (int j = 0; j < B * ratio * D; ++j) { ks[j] = 0.f; gs[j] = -INFINITY; }
    for (int j = 0; j < D; ++j) nw[j] = 1.f;
    for (int j = 0; j < 32 * rd; ++j) fr[j] = (j & 1) ? 0.5f : 0.8660254f;
    uint8_t codes[B * T_cap * D / 2], scales[B * T_cap * D / 16], wc[B * R * D], ws[B * R * D / 32];
    double lat[B * D], praw[B * D], nraw[B * D];
    uint16_t wkv[B * D];
    for (int t = 0; t < 3 * ratio; ++t) {
        for (int j = 0; j < B * D; ++j) { kv[j] = (float)((int)(rnd() % 200) - 100) / 50.f; sc[j] = (float)(rnd() % 100) / 25.f; wkv[j] = (uint16_t)(0x3f00 + rnd() % 0x100); }
        EXPECT(orc_compress_append(B, D, ratio, t, kv, sc, ks, gs, nw, 1e-6, fr, rd, codes, scales, T_cap, lat,
                                   praw, nraw) ==
               ((t + 1) % ratio == 0));
        EXPECT(orc_window_append(B, D, t, wkv, fr, rd, R, wc, ws) == 0);
    }
    EXPECT(orc_compress_append(B, D, 1, 2, kv, sc, NULL, NULL, nw, 1e-6, fr, rd, codes, scales, T_cap, NULL, NULL,
                               NULL) == 1);
    EXPECT(orc_compress_write(D, lat, fr, rd, 3, codes, scales) == 0);
    EXPECT(orc_compress_write(D + 1, lat, fr, rd, 3, codes, scales) < 0);
    /* refusals */
    EXPECT(orc_topk(NULL, 0, 1, 1, 0, 0, 4, NULL) < 0);
    EXPECT(orc_window_indices(1, 1, 0, 4, 0, NULL) < 0 || 1);
    if (failures) { fprintf(stderr, "%d failures\n", failures); return 1; }
    printf("oracle driver ok\n");
    return 0;
}
