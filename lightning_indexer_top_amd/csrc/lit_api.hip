// lit_api.hip -- the C ABI declared in include/lit.h: host-side argument checks,
// workspace sizing, and the stream-ordered launches of the kernels in indexer.hip,
// topk.hip, attention.hip and the fused decode kernel.  Nothing here allocates, frees
// or synchronises.
#include "../../include/lit.h"

#include <limits.h>

#include <atomic>
#include <mutex>

#include "lit_internal.h"

using namespace lit;

namespace {

// Queries (b, i) index the second grid dimension of the indexer and attention launches.
constexpr long kMaxQueries = 65535;
// Bytes of one sequence's bf16 KV source (R or T_cap rows of D): rows are addressed by
// 32-bit offsets, with the top bit marking a missing row.
constexpr long kMaxSourceBytes = 0x7fffffffL;

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

lit_status hip_status(hipError_t e) {
    if (e == hipSuccess) return LIT_OK;
    (void)hipGetLastError();
    return LIT_E_HIP;
}

int topk_width(int S, int start_pos, int ratio, int index_topk) {
    if (ratio <= 0 || index_topk <= 0) return 0;
    const long T = ((long)start_pos + S) / ratio;
    return (int)(index_topk < T ? index_topk : T);
}

lit_status check_indexer(int fmt, const uint8_t *q8, const uint8_t *q_sc, const float *w,
                         const uint8_t *k8, const uint8_t *k_sc, int B, int S, int Hi, int Di, int T_cap,
                         int start_pos, int ratio, const float *scores, int ld_scores) {
    if (fmt != LIT_INDEX_E4M3 && fmt != LIT_INDEX_E2M1) return LIT_E_UNSUPPORTED;
    if (B < 0 || S < 0 || start_pos < 0 || ratio < 1 || T_cap < 0) return LIT_E_SHAPE;
    if ((long)start_pos + S > INT_MAX) return LIT_E_SHAPE;
    const long T = ((long)start_pos + S) / ratio;
    if (T > T_cap) return LIT_E_SHAPE;
    if (Hi <= 0 || Hi % 16 != 0) return Hi <= 0 ? LIT_E_SHAPE : LIT_E_UNSUPPORTED;
    if (Hi > 64) return LIT_E_UNSUPPORTED;
    if ((long)B * S > kMaxQueries) return LIT_E_UNSUPPORTED;
    if (Di != 64 && Di != 128) return Di <= 0 || Di % 32 ? LIT_E_SHAPE : LIT_E_UNSUPPORTED;
    if (ld_scores < T) return LIT_E_SHAPE;
    if (ld_scores % 4 != 0) return LIT_E_ALIGN;
    if (B == 0 || S == 0 || T == 0) return LIT_OK;
    if (!q8 || !q_sc || !w || !k8 || !k_sc || !scores) return LIT_E_NULL;
    if (!aligned16(q8) || !aligned16(k8) || !aligned16(scores)) return LIT_E_ALIGN;
    return LIT_OK;
}

lit_status check_topk(const float *scores, int ld_scores, int B, int S, int start_pos, int ratio,
                      int index_topk, const int32_t *idx) {
    if (B < 0 || S < 0 || start_pos < 0 || ratio < 1 || index_topk < 0) return LIT_E_SHAPE;
    if ((long)start_pos + S > INT_MAX) return LIT_E_SHAPE;
    const long T = ((long)start_pos + S) / ratio;
    if (ld_scores < T) return LIT_E_SHAPE;
    if (ld_scores % 4 != 0) return LIT_E_ALIGN;
    const int keff = topk_width(S, start_pos, ratio, index_topk);
    if (B == 0 || S == 0 || keff == 0) return LIT_OK;
    if (!scores || !idx) return LIT_E_NULL;
    if (!aligned16(scores)) return LIT_E_ALIGN;
    return LIT_OK;
}

long window_need(int S, int start_pos, int W) {
    if (W <= 0 || S <= 0) return 0;
    const long span = start_pos == 0 ? (long)S : (long)W + S - 1;
    const long seen = (long)start_pos + S;
    return span < seen ? span : seen;
}

lit_status check_attn(const uint16_t *q, int B, int S, int H, int D, int dv, const uint16_t *win_kv,
                      int R, const int32_t *win_idx, int W, const uint16_t *comp_kv, int T_cap,
                      const int32_t *comp_idx, int K, const uint16_t *out) {
    if (B < 0 || S < 0 || W < 0 || K < 0 || R < 0 || T_cap < 0) return LIT_E_SHAPE;
    if ((long)B * S > kMaxQueries) return LIT_E_UNSUPPORTED;
    if (H <= 0 || D <= 0 || dv <= 0 || dv > D) return LIT_E_SHAPE;
    if (H != 16) return LIT_E_UNSUPPORTED;
    if (D != 64 && D != 128 && D != 192 && D != 256) return LIT_E_UNSUPPORTED;
    if (dv % 16 != 0) return LIT_E_UNSUPPORTED;
    if (W > 0 && R <= 0) return LIT_E_SHAPE;
    if (K > 0 && T_cap <= 0) return LIT_E_SHAPE;
    if ((long)R * D * 2 > kMaxSourceBytes || (long)T_cap * D * 2 > kMaxSourceBytes) return LIT_E_UNSUPPORTED;
    if (B == 0 || S == 0) return LIT_OK;
    if (!q || !out) return LIT_E_NULL;
    if (W > 0 && (!win_kv || !win_idx)) return LIT_E_NULL;
    if (K > 0 && (!comp_kv || !comp_idx)) return LIT_E_NULL;
    if (!aligned16(q) || (W > 0 && !aligned16(win_kv)) || (K > 0 && !aligned16(comp_kv)))
        return LIT_E_ALIGN;
    return LIT_OK;
}

}  // namespace

extern "C" {

const char *lit_status_str(int status) {
    switch (status) {
        case LIT_OK: return "LIT_OK";
        case LIT_E_NULL: return "LIT_E_NULL: a required pointer is NULL";
        case LIT_E_SHAPE: return "LIT_E_SHAPE: sizes are invalid or inconsistent";
        case LIT_E_ALIGN: return "LIT_E_ALIGN: a pointer or leading dimension is misaligned";
        case LIT_E_UNSUPPORTED: return "LIT_E_UNSUPPORTED: shape outside the implemented kernels";
        case LIT_E_WORKSPACE: return "LIT_E_WORKSPACE: workspace missing or too small";
        case LIT_E_HIP: return "LIT_E_HIP: a HIP launch failed";
        default: return "unknown lit_status";
    }
}

int lit_abi_version(void) { return LIT_ABI_VERSION; }

int lit_topk_width(int S, int start_pos, int ratio, int index_topk) {
    if (S < 0 || start_pos < 0) return 0;
    return topk_width(S, start_pos, ratio, index_topk);
}

int lit_compress_writes_row(int start_pos, int ratio) {
    if (ratio < 1 || start_pos < 0) return 0;
    return (start_pos + 1) % ratio == 0 ? 1 : 0;
}

lit_status lit_indexer_scores_fmt(int index_format, const uint8_t *q8, const uint8_t *q_sc,
                                  const float *w, const uint8_t *k8, const uint8_t *k_sc, int B,
                                  int S, int Hi, int Di, int T_cap, int start_pos, int ratio,
                                  float *scores, int ld_scores, void *stream) {
    lit_status st = check_indexer(index_format, q8, q_sc, w, k8, k_sc, B, S, Hi, Di, T_cap,
                                  start_pos, ratio, scores, ld_scores);
    if (st != LIT_OK) return st;
    IndexerArgs a{q8, q_sc, w, k8, k_sc, index_format, B, S, Hi, Di, T_cap, start_pos, ratio,
                  (start_pos + S) / ratio, scores, (long)ld_scores};
    return hip_status(launch_indexer_scores(a, (hipStream_t)stream));
}

lit_status lit_indexer_scores(const uint8_t *q8, const uint8_t *q_sc, const float *w,
                              const uint8_t *k8, const uint8_t *k_sc, int B, int S, int Hi, int Di,
                              int T_cap, int start_pos, int ratio, float *scores, int ld_scores,
                              void *stream) {
    return lit_indexer_scores_fmt(LIT_INDEX_E4M3, q8, q_sc, w, k8, k_sc, B, S, Hi, Di, T_cap,
                                  start_pos, ratio, scores, ld_scores, stream);
}

size_t lit_topk_workspace_bytes(int B, int S, int start_pos, int ratio, int index_topk) {
    (void)B; (void)S; (void)start_pos; (void)ratio; (void)index_topk;
    return 0;
}

lit_status lit_topk(const float *scores, int ld_scores, int B, int S, int start_pos, int ratio,
                    int index_topk, int32_t *idx, void *ws, size_t ws_bytes, void *stream) {
    (void)ws; (void)ws_bytes;
    lit_status st = check_topk(scores, ld_scores, B, S, start_pos, ratio, index_topk, idx);
    if (st != LIT_OK) return st;
    TopkArgs a{scores, (long)ld_scores, B, S, start_pos, ratio, (start_pos + S) / ratio,
               topk_width(S, start_pos, ratio, index_topk), idx};
    return hip_status(launch_topk(a, (hipStream_t)stream));
}

int lit_candidate_blocks_width(int S, int start_pos, int ratio, int topk_blocks, int block_size) {
    if (S < 0 || start_pos < 0 || ratio < 1 || topk_blocks < 0 || block_size < 1) return 0;
    if ((long)start_pos + S > INT_MAX) return 0;
    const long T = ((long)start_pos + S) / ratio;
    const long nb = (T + block_size - 1) / block_size;
    return (int)(topk_blocks < nb ? topk_blocks : nb);
}

static long block_ld(int S, int start_pos, int ratio, int block_size) {
    const long T = ((long)start_pos + S) / ratio;
    return (long)round_up((size_t)((T + block_size - 1) / block_size), 4);
}

size_t lit_candidate_blocks_workspace_bytes(int B, int S, int start_pos, int ratio, int block_size) {
    if (B <= 0 || S <= 0 || start_pos < 0 || ratio < 1 || block_size < 1) return 0;
    if ((long)start_pos + S > INT_MAX) return 0;
    return round_up((size_t)B * S * block_ld(S, start_pos, ratio, block_size) * sizeof(float), 256);
}

lit_status lit_candidate_blocks(const float *scores, int ld_scores, int B, int S, int start_pos, int ratio,
                                int topk_blocks, int block_size, int32_t *blocks, void *ws, size_t ws_bytes,
                                void *stream) {
    if (block_size < 1 || topk_blocks < 0) return LIT_E_SHAPE;
    lit_status st = check_topk(scores, ld_scores, B, S, start_pos, ratio, 1, blocks);
    if (st != LIT_OK) return st;
    const int kb = lit_candidate_blocks_width(S, start_pos, ratio, topk_blocks, block_size);
    if (B == 0 || S == 0 || kb == 0) return LIT_OK;
    const size_t need = lit_candidate_blocks_workspace_bytes(B, S, start_pos, ratio, block_size);
    if (!ws || ws_bytes < need) return LIT_E_WORKSPACE;
    if (!aligned16(ws)) return LIT_E_ALIGN;
    hipStream_t hs = (hipStream_t)stream;
    const int T = (start_pos + S) / ratio;
    const long ldb = block_ld(S, start_pos, ratio, block_size);
    float *bs = (float *)ws;
    hipError_t e = launch_block_max(scores, ld_scores, B, S, start_pos, ratio, T, block_size, bs, ldb, hs);
    if (e != hipSuccess) return hip_status(e);
    TopkArgs a{bs, ldb, B, S, start_pos, ratio, T, kb, blocks};
    a.vis_block = block_size;
    return hip_status(launch_topk(a, hs));
}

lit_status lit_topk_candidates(const float *scores, int ld_scores, int B, int S, int start_pos, int ratio,
                               int index_topk, const int32_t *blocks, int kb, int block_size, int32_t *idx,
                               void *ws, size_t ws_bytes, void *stream) {
    (void)ws; (void)ws_bytes;
    if (block_size < 1 || kb < 0) return LIT_E_SHAPE;
    lit_status st = check_topk(scores, ld_scores, B, S, start_pos, ratio, index_topk, idx);
    if (st != LIT_OK) return st;
    const int keff = topk_width(S, start_pos, ratio, index_topk);
    if (B == 0 || S == 0 || keff == 0) return LIT_OK;
    const long T = ((long)start_pos + S) / ratio;
    if ((T + block_size - 1) / block_size > kCandMaxBlocks) return LIT_E_UNSUPPORTED;
    if (kb > 0 && !blocks) return LIT_E_NULL;
    TopkArgs a{scores, (long)ld_scores, B, S, start_pos, ratio, (int)T, keff, idx};
    a.masked = true;  // kb == 0: every row is outside the (empty) candidate set
    a.cand = kb > 0 ? blocks : nullptr;
    a.cand_k = kb;
    a.cand_bs = block_size;
    return hip_status(launch_topk(a, (hipStream_t)stream));
}

int lit_window_width(int S, int start_pos, int W) {
    if (S < 0 || start_pos < 0) return 0;
    return window_width(S, start_pos, W);
}

lit_status lit_window_indices(int B, int S, int start_pos, int W, int R, int32_t *win_idx,
                              void *stream) {
    if (B < 0 || S < 0 || start_pos < 0 || W < 0 || R < 0) return LIT_E_SHAPE;
    const long width = window_width(S, start_pos, W);
    if ((long)B * S * width == 0) return LIT_OK;
    if (R < window_need(S, start_pos, W)) return LIT_E_SHAPE;
    if (!win_idx) return LIT_E_NULL;
    return hip_status(launch_window_indices(B, S, start_pos, W, R, win_idx, (hipStream_t)stream));
}

// Partial-state bytes of the attention's split plan.
static size_t attn_ws_bytes(int B, int S, int H, int dv, int W, int K) {
    return attention_partial_bytes(B, S, H, dv, plan_attention(B, S, attn_list_len(W, K)));
}

size_t lit_sparse_attn_workspace_bytes(int B, int S, int H, int dv, int W, int K) {
    if (B <= 0 || S <= 0 || H <= 0 || dv <= 0 || W < 0 || K < 0) return 0;
    return attn_ws_bytes(B, S, H, dv, W, K);
}

// Checks of the KV formats and scale pointers; sets the quantised sources of `a`.
static lit_status set_kv_formats(AttnArgs &a, int win_format, const void *win_kv, const uint8_t *win_scales,
                                 int comp_format, const void *comp_kv, const uint8_t *comp_scales) {
    if (win_format != LIT_KV_BF16 && win_format != LIT_KV_E4M3) return LIT_E_UNSUPPORTED;
    if (comp_format != LIT_KV_BF16 && comp_format != LIT_KV_E2M1) return LIT_E_UNSUPPORTED;
    if (win_format != LIT_KV_BF16 && a.W > 0) {
        if (!win_scales) return LIT_E_NULL;
        a.win_fmt = kKvE4M3;
        a.win_codes = (const uint8_t *)win_kv;
        a.win_scales = win_scales;
        a.win_kv = nullptr;
    }
    if (comp_format != LIT_KV_BF16 && a.K > 0) {
        if (!comp_scales) return LIT_E_NULL;
        a.comp_fmt = kKvE2M1;
        a.comp_codes = (const uint8_t *)comp_kv;
        a.comp_scales = comp_scales;
        a.comp_kv = nullptr;
    }
    return LIT_OK;
}

lit_status lit_sparse_attn_fmt(const uint16_t *q, int B, int S, int H, int D, int dv, int win_format,
                               const void *win_kv, const uint8_t *win_scales, int R, const int32_t *win_idx, int W,
                               int comp_format, const void *comp_kv, const uint8_t *comp_scales, int T_cap,
                               const int32_t *comp_idx, int K, const float *sink, float scale, uint16_t *out,
                               void *ws, size_t ws_bytes, void *stream) {
    lit_status st = check_attn(q, B, S, H, D, dv, (const uint16_t *)win_kv, R, win_idx, W,
                               (const uint16_t *)comp_kv, T_cap, comp_idx, K, out);
    if (st != LIT_OK) return st;
    // An explicit window list of width W (W == 0: no window rows).  The kernel derives
    // the window itself only when win_idx is NULL with W > 0, which only the steps and
    // the layered call ask for.
    AttnArgs a{q, B, S, H, D, dv, W > 0 ? (const uint16_t *)win_kv : nullptr, R, W > 0 ? win_idx : nullptr, W, 0,
               K > 0 ? (const uint16_t *)comp_kv : nullptr, T_cap, K > 0 ? comp_idx : nullptr, K, sink, scale, out,
               (float *)ws};
    if ((st = set_kv_formats(a, win_format, win_kv, win_scales, comp_format, comp_kv, comp_scales)) != LIT_OK)
        return st;
    if (B == 0 || S == 0) return LIT_OK;
    const AttnPlan p = plan_attention(B, S, attn_list_len(W, K));
    const size_t need = attention_partial_bytes(B, S, H, dv, p);
    if (need > 0 && (!ws || ws_bytes < need)) return LIT_E_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return LIT_E_ALIGN;
    return hip_status(launch_sparse_attn(a, p, (hipStream_t)stream));
}

lit_status lit_sparse_attn(const uint16_t *q, int B, int S, int H, int D, int dv,
                           const uint16_t *win_kv, int R, const int32_t *win_idx, int W,
                           const uint16_t *comp_kv, int T_cap, const int32_t *comp_idx, int K,
                           const float *sink, float scale, uint16_t *out, void *ws, size_t ws_bytes,
                           void *stream) {
    return lit_sparse_attn_fmt(q, B, S, H, D, dv, LIT_KV_BF16, win_kv, nullptr, R, win_idx, W, LIT_KV_BF16,
                               comp_kv, nullptr, T_cap, comp_idx, K, sink, scale, out, ws, ws_bytes, stream);
}

static bool step_uses_candidates(const lit_step_args *s) { return s->cand_in || s->cand_out; }
static bool step_quant_kv(const lit_step_args *s) { return s->win_kv_format != 0 || s->comp_kv_format != 0; }
static int step_layers(const lit_step_args *s) { return s->layers > 1 ? s->layers : 1; }

// Layer strides of the per-layer arrays of a step (elements of q / out, codes or bf16
// elements of the window source).
static void set_layers(AttnArgs &a, const lit_step_args *s) {
    a.L = step_layers(s);
    a.q_ls = (long)s->B * s->S * s->H * s->D;
    a.win_ls = (long)s->B * s->R * s->D;
    a.out_ls = (long)s->B * s->S * s->H * s->dv;
}

size_t lit_sparse_attn_layers_workspace_bytes(int L, int B, int S, int H, int dv, int W, int K) {
    if (L <= 0 || B <= 0 || S <= 0 || H <= 0 || dv <= 0 || W < 0 || K < 0) return 0;
    if ((long)L * B * S > kMaxQueries) return 0;
    return attn_ws_bytes(L * B, S, H, dv, W, K);
}

lit_status lit_sparse_attn_layers(int L, const uint16_t *q, int B, int S, int H, int D, int dv,
                                  const uint16_t *win_kv, int R, const int32_t *win_idx, int W, int start_pos,
                                  const uint16_t *comp_kv, int T_cap, const int32_t *comp_idx, int K,
                                  const float *sink, float scale, uint16_t *out, void *ws, size_t ws_bytes,
                                  void *stream) {
    if (L < 1 || start_pos < 0) return LIT_E_SHAPE;
    // a derived window (win_idx NULL) lists window_width(S, start_pos, W) slots
    const bool derived = W > 0 && !win_idx;
    const int nwin = derived ? window_width(S, start_pos, W) : W;
    lit_status st = check_attn(q, B, S, H, D, dv, win_kv, R, derived ? (const int32_t *)16 : win_idx, nwin,
                               comp_kv, T_cap, comp_idx, K, out);
    if (st != LIT_OK) return st;
    if (derived && R < window_need(S, start_pos, W)) return LIT_E_SHAPE;
    if ((long)L * B * S > kMaxQueries) return LIT_E_UNSUPPORTED;
    if (B == 0 || S == 0) return LIT_OK;
    const AttnPlan p = plan_attention(L * B, S, attn_list_len(nwin, K));
    const size_t need = attention_partial_bytes(L * B, S, H, dv, p);
    if (need > 0 && (!ws || ws_bytes < need)) return LIT_E_WORKSPACE;
    if (need > 0 && !aligned16(ws)) return LIT_E_ALIGN;
    AttnArgs a{q, B, S, H, D, dv, W > 0 ? win_kv : nullptr, R, W > 0 ? win_idx : nullptr, W, start_pos,
               K > 0 ? comp_kv : nullptr, T_cap, K > 0 ? comp_idx : nullptr, K, sink, scale, out,
               (float *)ws};
    a.L = L;
    a.q_ls = (long)B * S * H * D;
    a.win_ls = (long)B * R * D;
    a.out_ls = (long)B * S * H * dv;
    return hip_status(launch_sparse_attn(a, p, (hipStream_t)stream));
}

static lit_status check_produce(int B, int D, int rd, int pos, int n_pos, const void *freqs) {
    if (B < 0 || D <= 0 || rd < 0 || n_pos < 0) return LIT_E_SHAPE;
    if (D % 32 != 0 || rd % 2 != 0 || rd > D) return LIT_E_SHAPE;
    if (D > 256) return LIT_E_UNSUPPORTED;
    if (B > 0 && (pos < 0 || pos >= n_pos)) return LIT_E_SHAPE;
    if (B > 0 && rd > 0 && !freqs) return LIT_E_NULL;
    return LIT_OK;
}

lit_status lit_compress_append(int B, int D, int ratio, int start_pos, const float *kv, const float *score,
                               float *kv_state, float *score_state, const float *norm_w, float eps,
                               const float *freqs, int n_pos, int rd, uint8_t *codes, uint8_t *scales, int T_cap,
                               uint16_t *latent, void *stream) {
    if (ratio < 1 || start_pos < 0 || T_cap < 0) return LIT_E_SHAPE;
    const bool done = lit_compress_writes_row(start_pos, ratio) != 0;
    lit_status st = check_produce(B, D, rd, done ? start_pos + 1 - ratio : 0, done ? n_pos : 1, freqs);
    if (st != LIT_OK) return st;
    if (B == 0) return LIT_OK;
    if (done && start_pos / ratio >= T_cap) return LIT_E_SHAPE;
    if (!kv || !norm_w || (ratio > 1 && (!score || !kv_state || !score_state))) return LIT_E_NULL;
    if (done && (!codes || !scales)) return LIT_E_NULL;
    ProduceArgs p{};
    p.B = B; p.D = D; p.ratio = ratio; p.start_pos = start_pos; p.rd = rd;
    p.kv = kv; p.score = score; p.kv_state = kv_state; p.score_state = score_state;
    p.norm_w = norm_w; p.eps = eps; p.freqs = freqs; p.codes = codes; p.scales = scales;
    p.T_cap = T_cap; p.latent = latent;
    return hip_status(launch_compress_append(p, (hipStream_t)stream));
}

lit_status lit_window_append(int B, int D, int start_pos, const uint16_t *kv, const float *freqs, int n_pos,
                             int rd, uint8_t *codes, uint8_t *scales, int R, void *stream) {
    if (start_pos < 0 || R < 0) return LIT_E_SHAPE;
    lit_status st = check_produce(B, D, rd, start_pos, n_pos, freqs);
    if (st != LIT_OK) return st;
    if (B == 0) return LIT_OK;
    if (R < 1) return LIT_E_SHAPE;
    if (!kv || !codes || !scales) return LIT_E_NULL;
    ProduceArgs p{};
    p.B = B; p.D = D; p.start_pos = start_pos; p.rd = rd; p.freqs = freqs;
    p.win_in = kv; p.codes = codes; p.scales = scales; p.R = R;
    return hip_status(launch_window_append(p, (hipStream_t)stream));
}

int lit_compress_chunk_rows(int start_pos, int S, int ratio) { return compress_chunk_rows(start_pos, S, ratio); }

lit_status lit_compress_chunk(int B, int S, int D, int ratio, int start_pos, const float *kv, const float *score,
                              float *kv_state, float *score_state, const float *norm_w, float eps,
                              const float *freqs, int n_pos, int rd, uint8_t *codes, uint8_t *scales, int T_cap,
                              uint16_t *latent, void *stream) {
    if (ratio < 1 || start_pos < 0 || S < 0 || T_cap < 0) return LIT_E_SHAPE;
    if ((long)start_pos + S > INT_MAX) return LIT_E_SHAPE;
    const int n = compress_chunk_rows(start_pos, S, ratio);
    // the last written row's rotation position is the largest one
    const int last_pos = n > 0 ? (start_pos / ratio + n - 1) * ratio : 0;
    lit_status st = check_produce(B, D, rd, last_pos, n > 0 ? n_pos : 1, freqs);
    if (st != LIT_OK) return st;
    if (B == 0 || S == 0) return LIT_OK;
    if (n > 0 && start_pos / ratio + n - 1 >= T_cap) return LIT_E_SHAPE;
    if (!kv || !norm_w || (ratio > 1 && (!score || !kv_state || !score_state))) return LIT_E_NULL;
    if (n > 0 && (!codes || !scales)) return LIT_E_NULL;
    ProduceArgs p{};
    p.B = B; p.D = D; p.ratio = ratio; p.start_pos = start_pos; p.rd = rd; p.S = S;
    p.kv = kv; p.score = score; p.kv_state = kv_state; p.score_state = score_state;
    p.norm_w = norm_w; p.eps = eps; p.freqs = freqs; p.codes = codes; p.scales = scales;
    p.T_cap = T_cap; p.latent = latent;
    return hip_status(launch_compress_chunk(p, (hipStream_t)stream));
}

lit_status lit_window_chunk(int B, int S, int D, int start_pos, const uint16_t *kv, const float *freqs, int n_pos,
                            int rd, uint8_t *codes, uint8_t *scales, int R, void *stream) {
    if (start_pos < 0 || S < 0 || R < 0) return LIT_E_SHAPE;
    if ((long)start_pos + S > INT_MAX) return LIT_E_SHAPE;
    lit_status st = check_produce(B, D, rd, S > 0 ? start_pos + S - 1 : 0, S > 0 ? n_pos : 1, freqs);
    if (st != LIT_OK) return st;
    if (B == 0 || S == 0) return LIT_OK;
    if (R < 1) return LIT_E_SHAPE;
    if (!kv || !codes || !scales) return LIT_E_NULL;
    ProduceArgs p{};
    p.B = B; p.D = D; p.start_pos = start_pos; p.rd = rd; p.freqs = freqs; p.S = S;
    p.win_in = kv; p.codes = codes; p.scales = scales; p.R = R;
    return hip_status(launch_window_chunk(p, (hipStream_t)stream));
}

// Workspace of the multi-kernel step: scores [B*S, ld] fp32, then the attention partials
// (level one's block scores share the partials' space: they are used up before).
static size_t step_layout(const lit_step_args *s, size_t *scores_bytes, long *ld, AttnPlan *plan) {
    const long T = ((long)s->start_pos + s->S) / s->ratio;
    *ld = (long)round_up((size_t)(T > 0 ? T : 1), 4);
    *scores_bytes = round_up((size_t)s->B * s->S * (*ld) * sizeof(float), 256);
    const int nwin = window_width(s->S, s->start_pos, s->W);
    const int keff = topk_width(s->S, s->start_pos, s->ratio, s->index_topk);
    *plan = plan_attention(step_layers(s) * s->B, s->S, attn_list_len(nwin, keff));
    size_t rest = round_up(attention_partial_bytes(step_layers(s) * s->B, s->S, s->H, s->dv, *plan), 256);
    if (s->cand_out) {
        const size_t bb = lit_candidate_blocks_workspace_bytes(s->B, s->S, s->start_pos, s->ratio,
                                                               s->cand_block_size);
        if (bb > rest) rest = bb;
    }
    return *scores_bytes + rest;
}

// The fused kernel takes a level-two layer with 1..2048 candidate blocks per query; a
// candidate source (cand_out) runs fused when its blocks divide the members' chunks (the
// kernel writes the block maxima, level one's top-k follows as one kernel).
constexpr int kFusedCandMaxApi = 2048;

static FusedPlan step_fused_plan(const lit_step_args *s) {
    FusedPlan p{};
    p.ok = false;
    if (s->flags & LIT_STEP_UNFUSED) return p;
    const bool masked = s->cand_in != nullptr;
    if (masked && (s->cand_k < 1 || s->cand_k > kFusedCandMaxApi)) return p;
    // quantised KV runs fused when both sources are quantised (e4m3 window, e2m1 compressed)
    const bool qkv = step_quant_kv(s);
    if (qkv && (s->win_kv_format != LIT_KV_E4M3 || s->comp_kv_format != LIT_KV_E2M1)) return p;
    const bool layers = step_layers(s) > 1;
    const int keff = topk_width(s->S, s->start_pos, s->ratio, s->index_topk);
    p = plan_fused(s->index_format, masked, qkv, layers, s->B, s->S, s->start_pos, s->ratio, s->Hi, s->Di, s->D,
                   s->dv, s->W, keff);
    // partial states are addressed with 32-bit offsets within a query's slots
    if (p.ok && fused_part_bytes_per_query(p, s->dv, step_layers(s)) >= ((size_t)1 << 31)) p.ok = false;
    if (p.ok && s->cand_out && (s->cand_block_size < 1 || p.chunk % s->cand_block_size != 0)) p.ok = false;
    return p;
}

// Workspace of the fused step: the kernel's, then a candidate source's block maxima.
static size_t step_fused_ws_bytes(const lit_step_args *s, const FusedPlan &fp) {
    size_t need = round_up(fused_ws_bytes(fp, s->dv, step_layers(s)), 256);
    if (s->cand_out)
        need += lit_candidate_blocks_workspace_bytes(s->B, s->S, s->start_pos, s->ratio, s->cand_block_size);
    return need;
}

static lit_status check_step(const lit_step_args *s) {
    if (!s) return LIT_E_NULL;
    if (s->ratio < 1 || s->B < 0 || s->S < 0 || s->start_pos < 0) return LIT_E_SHAPE;
    if ((long)s->start_pos + s->S > INT_MAX) return LIT_E_SHAPE;
    const long T = ((long)s->start_pos + s->S) / s->ratio;
    if (T > INT_MAX / 4) return LIT_E_SHAPE;
    const int ld = (int)round_up((size_t)(T > 0 ? T : 1), 4);
    lit_status st = check_indexer(s->index_format, s->q8, s->q_sc, s->w, s->k8, s->k_sc, s->B, s->S,
                                  s->Hi, s->Di, s->T_cap, s->start_pos, s->ratio, (const float *)16, ld);
    if (st != LIT_OK) return st;
    const int keff = topk_width(s->S, s->start_pos, s->ratio, s->index_topk);
    if (s->index_topk < 0) return LIT_E_SHAPE;
    if (s->W > 0 && s->R < window_need(s->S, s->start_pos, s->W)) return LIT_E_SHAPE;
    st = check_attn(s->q, s->B, s->S, s->H, s->D, s->dv, s->win_kv, s->R, (const int32_t *)16,
                    window_width(s->S, s->start_pos, s->W), s->comp_kv, s->T_cap,
                    (const int32_t *)16, keff, s->out);
    if (st != LIT_OK) return st;
    if (s->B > 0 && s->S > 0 && keff > 0 && !s->topk_idx) return LIT_E_NULL;
    if (s->layers < 0) return LIT_E_SHAPE;
    if ((long)step_layers(s) * s->B * s->S > kMaxQueries) return LIT_E_UNSUPPORTED;
    if (step_quant_kv(s)) {
        if ((s->win_kv_format != LIT_KV_BF16 && s->win_kv_format != LIT_KV_E4M3) ||
            (s->comp_kv_format != LIT_KV_BF16 && s->comp_kv_format != LIT_KV_E2M1))
            return LIT_E_UNSUPPORTED;
        if (s->B > 0 && s->S > 0 && ((s->win_kv_format && s->W > 0 && !s->win_kv_scales) ||
                                     (s->comp_kv_format && keff > 0 && !s->comp_kv_scales)))
            return LIT_E_NULL;
    }
    if (step_uses_candidates(s)) {
        if (s->cand_block_size < 1 || s->cand_k < 0 || s->cand_topk_blocks < 0) return LIT_E_SHAPE;
        if (s->cand_in && (T + s->cand_block_size - 1) / s->cand_block_size > kCandMaxBlocks)
            return LIT_E_UNSUPPORTED;
    }
    return LIT_OK;
}

size_t lit_sparse_step_workspace_bytes(const lit_step_args *s) {
    if (check_step(s) != LIT_OK) return 0;
    size_t sb;
    long ld;
    AttnPlan p;
    size_t need = step_layout(s, &sb, &ld, &p);
    const FusedPlan fp = step_fused_plan(s);
    if (fp.ok) {
        const size_t fused = step_fused_ws_bytes(s, fp);
        if (fused > need) need = fused;
    }
    return need;
}

size_t lit_sparse_step_state_bytes(const lit_step_args *s) {
    if (check_step(s) != LIT_OK) return 0;
    const FusedPlan fp = step_fused_plan(s);
    return fp.ok ? fused_state_bytes(fp) : 0;
}

}  // extern "C"

// The step on a caller's (or the library's) workspace and state; err_word, when set,
// receives a fused team timeout instead of the state's first word.
static lit_status step_run(const lit_step_args *s, void *ws, size_t ws_bytes, uint32_t *err_word, void *stream) {
    lit_status st = check_step(s);
    if (st != LIT_OK) return st;
    if (s->B == 0 || s->S == 0) return LIT_OK;
    size_t scores_bytes;
    long ld;
    AttnPlan plan;
    const size_t need = step_layout(s, &scores_bytes, &ld, &plan);
    if (!ws || ws_bytes < need) return LIT_E_WORKSPACE;
    if (((uintptr_t)ws & 255u) != 0) return LIT_E_ALIGN;
    hipStream_t hs = (hipStream_t)stream;
    const int T = (s->start_pos + s->S) / s->ratio;
    const int keff = topk_width(s->S, s->start_pos, s->ratio, s->index_topk);
    float *scores = (float *)ws;
    hipError_t e = hipSuccess;
    auto mark = [&](int k) -> hipError_t {
        return s->stage_events[k] ? hipEventRecord((hipEvent_t)s->stage_events[k], hs) : hipSuccess;
    };
    if ((e = mark(0)) != hipSuccess) return hip_status(e);
    const FusedPlan fp = step_fused_plan(s);
    if (fp.ok && s->state && s->state_bytes >= fused_state_bytes(fp)) {
        if (((uintptr_t)s->state & 255u) != 0) return LIT_E_ALIGN;
        if (ws_bytes < step_fused_ws_bytes(s, fp)) return LIT_E_WORKSPACE;
        FusedArgs f{};
        f.ia = IndexerArgs{s->q8, s->q_sc, s->w, s->k8, s->k_sc, s->index_format, s->B, s->S, s->Hi,
                           s->Di, s->T_cap, s->start_pos, s->ratio, T, nullptr, 0};
        f.aa = AttnArgs{s->q, s->B, s->S, s->H, s->D, s->dv, s->W > 0 ? s->win_kv : nullptr, s->R,
                        nullptr, s->W, s->start_pos, s->comp_kv, s->T_cap, nullptr, keff, s->sink,
                        s->scale, s->out, nullptr};
        f.topk_out = s->topk_idx;
        f.keff = keff;
        set_layers(f.aa, s);
        if (s->cand_in) {
            f.cand = s->cand_in;
            f.cand_k = s->cand_k;
            f.cand_bs = s->cand_block_size;
        }
        if (step_quant_kv(s) && set_kv_formats(f.aa, s->win_kv_format, s->win_kv, s->win_kv_scales,
                                               s->comp_kv_format, s->comp_kv, s->comp_kv_scales) != LIT_OK)
            return LIT_E_UNSUPPORTED;
        const int kb = s->cand_out ? lit_candidate_blocks_width(s->S, s->start_pos, s->ratio, s->cand_topk_blocks,
                                                                s->cand_block_size)
                                   : 0;
        if (kb > 0 && T > 0) {  // candidate source: the kernel writes level one's block maxima
            f.bmax = (float *)((char *)ws + round_up(fused_ws_bytes(fp, s->dv, step_layers(s)), 256));
            f.ldb = block_ld(s->S, s->start_pos, s->ratio, s->cand_block_size);
            f.bmax_bs = s->cand_block_size;
        }
        f.spin_limit = 1u << 22;
        if ((e = launch_fused(f, fp, ws, s->state, hs, err_word)) != hipSuccess) return hip_status(e);
        if (f.bmax) {
            TopkArgs la{f.bmax, f.ldb, s->B, s->S, s->start_pos, s->ratio, T, kb, s->cand_out};
            la.vis_block = s->cand_block_size;
            if ((e = launch_topk(la, hs)) != hipSuccess) return hip_status(e);
        }
        for (int k = 1; k < 4; ++k)
            if ((e = mark(k)) != hipSuccess) return hip_status(e);
        return LIT_OK;
    }
    if (keff > 0) {
        IndexerArgs ia{s->q8, s->q_sc, s->w, s->k8, s->k_sc, s->index_format, s->B, s->S, s->Hi,
                       s->Di, s->T_cap, s->start_pos, s->ratio, T, scores, ld};
        ia.visible_only = true;  // the top-k reads no column past a query's visible rows
        if ((e = launch_indexer_scores(ia, hs)) != hipSuccess) return hip_status(e);
    }
    if ((e = mark(1)) != hipSuccess) return hip_status(e);
    char *rest = (char *)ws + scores_bytes;
    if (s->cand_out) {  // candidate source: level one over this layer's scores
        const int kb = lit_candidate_blocks_width(s->S, s->start_pos, s->ratio, s->cand_topk_blocks,
                                                  s->cand_block_size);
        if (kb > 0 && T > 0) {
            const long ldb = block_ld(s->S, s->start_pos, s->ratio, s->cand_block_size);
            if ((e = launch_block_max(scores, ld, s->B, s->S, s->start_pos, s->ratio, T, s->cand_block_size,
                                      (float *)rest, ldb, hs)) != hipSuccess)
                return hip_status(e);
            TopkArgs la{(const float *)rest, ldb, s->B, s->S, s->start_pos, s->ratio, T, kb, s->cand_out};
            la.vis_block = s->cand_block_size;
            if ((e = launch_topk(la, hs)) != hipSuccess) return hip_status(e);
        }
    }
    if (keff > 0) {
        TopkArgs ta{scores, ld, s->B, s->S, s->start_pos, s->ratio, T, keff, s->topk_idx};
        if (s->cand_in) {  // level two
            ta.masked = true;
            ta.cand = s->cand_k > 0 ? s->cand_in : nullptr;
            ta.cand_k = s->cand_k;
            ta.cand_bs = s->cand_block_size;
        }
        if ((e = launch_topk(ta, hs)) != hipSuccess) return hip_status(e);
    }
    if ((e = mark(2)) != hipSuccess) return hip_status(e);
    AttnArgs aa{s->q, s->B, s->S, s->H, s->D, s->dv, s->W > 0 ? s->win_kv : nullptr, s->R,
                nullptr, s->W, s->start_pos, keff > 0 ? s->comp_kv : nullptr, s->T_cap,
                keff > 0 ? s->topk_idx : nullptr, keff, s->sink, s->scale, s->out,
                (float *)rest};
    set_layers(aa, s);
    if (step_quant_kv(s)) {
        // the derived window keeps W as its size; the checks ran in check_step
        aa.K = keff;
        if (set_kv_formats(aa, s->win_kv_format, s->win_kv, s->win_kv_scales, s->comp_kv_format, s->comp_kv,
                           s->comp_kv_scales) != LIT_OK)
            return LIT_E_UNSUPPORTED;
    }
    if ((e = launch_sparse_attn(aa, plan, hs)) != hipSuccess) return hip_status(e);
    return hip_status(mark(3));
}

// ---------------------------------------------------------------------------
// The no-allocation form: workspace and fused-form state in the library's own scratch.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = (size_t)16 << 20;      // per device
constexpr size_t kScratchStateBytes = (size_t)1 << 20;  // the fused form's state, first
// Device memory of lit_sparse_step_noalloc: its workspace and its fused-form state.  Every
// GPU the library runs on holds its own copy until the process ends (zero at load, which
// is the state's required initial value).  In host code this name is not a device address:
// only the address hipGetSymbolAddress gives for the current device is ever passed on.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's copy of `scratch`, looked up once per device.
lit_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return LIT_E_HIP;
    }
    void *p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
                (void)hipGetLastError();
                return LIT_E_HIP;
            }
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return LIT_OK;
}
}  // namespace

extern "C" {

lit_status lit_sparse_step(const lit_step_args *s, void *ws, size_t ws_bytes, void *stream) {
    return step_run(s, ws, ws_bytes, nullptr, stream);
}

lit_status lit_sparse_step_noalloc(const lit_step_args *s, uint32_t *err_word, void *stream) {
    lit_status st = check_step(s);
    if (st != LIT_OK) return st;
    if (s->B == 0 || s->S == 0) return LIT_OK;
    lit_step_args a = *s;
    a.state = nullptr;
    a.state_bytes = 0;
    // the fused form when its state fits the reserved first MiB (else the kernels)
    const size_t sb = (s->flags & LIT_STEP_UNFUSED) ? 0 : lit_sparse_step_state_bytes(&a);
    const bool fused = sb > 0 && sb <= kScratchStateBytes;
    if (!fused) a.flags |= LIT_STEP_UNFUSED;
    const size_t need = lit_sparse_step_workspace_bytes(&a);
    if (need > kScratchBytes - kScratchStateBytes) return LIT_E_WORKSPACE;
    void *p = nullptr;
    if ((st = scratch_address(&p)) != LIT_OK) return st;
    if (fused) {
        a.state = p;
        a.state_bytes = kScratchStateBytes;
    }
    return step_run(&a, (char *)p + kScratchStateBytes, kScratchBytes - kScratchStateBytes, err_word, stream);
}

}  // extern "C"
