// lit_internal.h -- device-side types, helpers and the launchers each kernel file
// exports to the C-ABI layer (lit_api.hip).  gfx950 (CDNA4) only: 64-lane waves,
// MFMA matrix cores, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lit {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Indexer scores (indexer.hip)
// ---------------------------------------------------------------------------
// Code formats of the index queries and keys (both use one ue8m0 scale per 32
// elements): one e4m3 byte per element, or two e2m1 (fp4) codes per byte with
// element 2j in the low nibble of byte j.
constexpr int kFmtE4M3 = 0;
constexpr int kFmtE2M1 = 1;
__host__ __device__ constexpr int idx_row_bytes(int Di, int fmt) { return fmt == kFmtE2M1 ? Di / 2 : Di; }

struct IndexerArgs {
    const uint8_t *q8;    // [B,S,Hi,E] codes, E = idx_row_bytes(Di, fmt)
    const uint8_t *q_sc;  // [B,S,Hi,Di/32]
    const float *w;       // [B,S,Hi]
    const uint8_t *k8;    // [B,T_cap,E]
    const uint8_t *k_sc;  // [B,T_cap,Di/32]
    int fmt;              // kFmtE4M3 or kFmtE2M1
    int B, S, Hi, Di, T_cap, start_pos, ratio;
    int T;                // (start_pos + S) / ratio, columns written per row
    float *scores;        // [B,S,ld]
    long ld;
    // only the visible columns are written (the step's own scores, which nothing reads past a
    // query's visible rows); otherwise the invisible columns below T get -inf
    bool visible_only = false;
};
hipError_t launch_indexer_scores(const IndexerArgs &a, hipStream_t stream);

// ---------------------------------------------------------------------------
// Top-k selection (topk.hip)
// ---------------------------------------------------------------------------
struct TopkArgs {
    const float *scores;  // [B,S,ld]
    long ld;
    int B, S, start_pos, ratio;
    int T;                // columns that exist per row
    int keff;             // entries written per row
    int32_t *idx;         // [B,S,keff]
    // Two-level top-k.  vis_block > 1: the columns are blocks of vis_block rows, and a
    // query sees ceil(visible rows / vis_block) of them (level one).  masked: a column
    // outside the blocks listed for its query (cand [B,S,cand_k], blocks of cand_bs
    // rows, -1 = none; cand may be NULL when cand_k == 0) counts as -inf (level two).
    int vis_block = 1;
    bool masked = false;
    const int32_t *cand = nullptr;
    int cand_k = 0, cand_bs = 1;
};
hipError_t launch_topk(const TopkArgs &a, hipStream_t stream);
// Level one's block scores: bscores[row, j] = max of the visible scores of block j (rows
// j*bs .. j*bs+bs-1), +inf for the block holding the query's newest visible row.
hipError_t launch_block_max(const float *scores, long ld, int B, int S, int start_pos, int ratio, int T, int bs,
                            float *bscores, long ldb, hipStream_t stream);
// Most blocks level two can hold as a bitmap in LDS.
constexpr int kCandMaxBlocks = 65536;

// ---------------------------------------------------------------------------
// Sparse attention (attention.hip) and window lists
// ---------------------------------------------------------------------------
// KV row formats of the attention sources (dequantised on gather, tile_ops.h).
constexpr int kKvBf16 = 0;
constexpr int kKvE4M3 = 1;  // e4m3 codes, ue8m0 scale per 32
constexpr int kKvE2M1 = 2;  // e2m1 codes (two a byte), e4m3 scale per 16
struct AttnArgs {
    const uint16_t *q;        // [B,S,H,D] bf16
    int B, S, H, D, dv;
    const uint16_t *win_kv;   // [B,R,D]
    int R;
    const int32_t *win_idx;   // [B,S,W] explicit list, or NULL: derive from start_pos
    int W;                    // list width (explicit) or window size (derived)
    int start_pos;            // used when win_idx == NULL
    const uint16_t *comp_kv;  // [B,T_cap,D]
    int T_cap;
    const int32_t *comp_idx;  // [B,S,K]
    int K;
    const float *sink;        // [H] or NULL
    float scale;
    uint16_t *out;            // [B,S,H,dv] bf16
    float *part;              // split partials (workspace), may be NULL when 1 split
    // Several layers over one row list (cross-layer reuse): layer l reads q, win_kv and
    // sink at l times their layer strides and writes out (and its partials) likewise;
    // the lists and comp_kv are shared.
    int L = 1;
    long q_ls = 0, win_ls = 0, out_ls = 0;
    // Quantised sources (kKvE4M3 window, kKvE2M1 compressed; tile_ops.h): codes and scale
    // bytes replace win_kv / comp_kv.  The window entries then fill whole 32-row tiles
    // (the list is padded to a tile boundary) so no tile mixes the two formats.
    int win_fmt = 0, comp_fmt = 0;
    const uint8_t *win_codes = nullptr, *win_scales = nullptr;
    const uint8_t *comp_codes = nullptr, *comp_scales = nullptr;
};
// Entries of the list the attention kernel walks: window entries, padded to whole 32-row
// tiles so that no tile mixes the two sources, then the compressed entries.
__host__ __device__ inline int attn_list_len(int nwin, int K) { return (nwin + 31) / 32 * 32 + K; }
// Split plan: how many workgroups share one query's row list.
struct AttnPlan {
    int list_len;        // window width + K
    int tiles_per_wave;  // 32-row tiles each wave handles
    int n_splits;        // workgroups per query
    bool per_wave;       // one wave per query instead (many queries: chunked prefill)
};
// Query rows (times layers) from which every query gets a wave of its own.
constexpr int kWaveFormQueries = 2048;
AttnPlan plan_attention(int B, int S, int list_len);  // B*S: query rows (times layers)
size_t attention_partial_bytes(int B, int S, int H, int dv, const AttnPlan &p);
hipError_t launch_sparse_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t stream);

// Entries per window list: min(S, W) for a chunk starting at position 0, else W.
__host__ __device__ inline int window_width(int S, int start_pos, int W) {
    if (W <= 0) return 0;
    if (start_pos == 0) return S < W ? S : W;
    return W;
}
hipError_t launch_window_indices(int B, int S, int start_pos, int W, int R, int32_t *win_idx,
                                 hipStream_t stream);

// The window rule shared by the list builder and the attention kernel: entry j of
// query i's window list, as a ring slot, or -1.
__host__ __device__ inline int window_slot(int S, int start_pos, int W, int R, int i, int j) {
    long p;
    bool valid;
    if (start_pos == 0) {
        long base = i - W + 1 > 0 ? i - W + 1 : 0;
        p = base + j;
        valid = p <= i;
    } else {
        p = (long)start_pos + i - W + 1 + j;
        valid = p >= 0;
    }
    return valid ? (int)(p % R) : -1;
}

// The same rule with the division done once per query: entry j of query i's list is
// position p0 + j at ring slot (s0 + j) mod R.  Positions stay below 2^31 (start_pos + S
// is checked to fit an int), so 32-bit arithmetic is exact.
struct WindowBase {
    int p0;  // position of entry 0 (negative before the sequence's start)
    int s0;  // its slot, p0 mod R in [0, R)
};
__host__ __device__ inline WindowBase window_base(int start_pos, int W, int R, int i) {
    WindowBase w;
    w.p0 = start_pos == 0 ? (i - W + 1 > 0 ? i - W + 1 : 0) : start_pos + i - W + 1;
    const int m = w.p0 % R;
    w.s0 = m < 0 ? m + R : m;
    return w;
}
__host__ __device__ inline int window_slot_at(const WindowBase &w, int start_pos, int R, int i, int j) {
    const int p = w.p0 + j;
    const bool valid = start_pos == 0 ? p <= i : p >= 0;
    int s = w.s0 + j;
    if (s >= R) s -= R;
    if (s >= R) s %= R;  // a ring shorter than the window (early in a sequence)
    return valid ? s : -1;
}


// ---------------------------------------------------------------------------
// Producer side: the cache writes of one decode step (produce.hip)
// ---------------------------------------------------------------------------
struct ProduceArgs {
    int B, D, ratio, start_pos, rd;
    const float *kv, *score;        // [B,S,D] compressor inputs (fp32; S = 1: a decode step)
    float *kv_state, *score_state;  // [B,ratio,D] (ratio > 1)
    const float *norm_w;            // [D]
    float eps;
    const float *freqs;             // [positions, rd/2, 2] (cos, sin)
    const uint16_t *win_in;         // [B,S,D] bf16 window KV rows (window append / chunk)
    uint8_t *codes, *scales;        // cache codes / scale bytes
    int T_cap, R;
    uint16_t *latent;               // [B,rows,D] bf16 pre-rotation latents, or NULL
    int S = 1;                      // tokens per sequence (a chunk)
};
hipError_t launch_compress_append(const ProduceArgs &p, hipStream_t stream);
hipError_t launch_window_append(const ProduceArgs &p, hipStream_t stream);
// Chunks: S tokens per sequence, the S decode steps' writes in one launch each.
int compress_chunk_rows(int start_pos, int S, int ratio);  // compressed rows a chunk writes
hipError_t launch_compress_chunk(const ProduceArgs &p, hipStream_t stream);
hipError_t launch_window_chunk(const ProduceArgs &p, hipStream_t stream);

// ---------------------------------------------------------------------------
// Fused decode step (fused_decode.hip)
// ---------------------------------------------------------------------------
// Division by a divisor known at launch: for 0 <= n < 2^31, n / d = (n * m) >> s with
// l = ceil(log2 d), s = 31 + l and m = ceil(2^s / d) < 2^32 (the multiplier of Granlund
// and Montgomery's division by invariant integers, for 31-bit dividends).  A multiply and
// a shift instead of a division sequence on the kernel's dependent paths.
struct FastDiv {
    uint32_t m = 1u << 31;
    int s = 31;  // (the divisor 1)
};
inline FastDiv fast_div(uint32_t d) {
    FastDiv f;
    int l = 0;
    while ((1ull << l) < d) ++l;
    f.s = 31 + l;
    f.m = (uint32_t)(((1ull << f.s) + d - 1) / d);
    return f;
}
__host__ __device__ inline int fdiv(int n, FastDiv f) { return (int)(((uint64_t)(uint32_t)n * f.m) >> f.s); }

struct FusedArgs {
    IndexerArgs ia;       // scores / ld unused
    AttnArgs aa;          // win_idx unused (window derived), comp_idx unused, part unused
    int32_t *topk_out;    // [B,S,keff] output
    int keff;
    int team_size, chunk, win_tiles, n_slots;
    int vbins;            // value bins of the selection (256, 1024 or 4096; fewer for short rows)
    long ld;              // team score array stride
    uint32_t spin_limit;
    uint32_t *err;                // sticky error word (state)
    char *qstate;                 // per query: launch count and barrier flag slots (state)
    float *scores;                // per team: scores of the visible rows
    float *part;                  // per member: partial attention state
    int slot_floats;              // floats per member state
    int merge_per;                // (layer, head, dim quad) outputs each member merges
    // divisors of the kernel's index arithmetic: team size, queries per sequence, compress
    // ratio, window ring rows, dim quads dv / 4, head-dim quads 16 * dv / 4, candidate
    // block size
    FastDiv div_team, div_S, div_ratio, div_R, div_qdv, div_hq, div_cbs;
    bool cache_lds;               // the team's scores are kept in LDS during selection
    bool lds_bins;                // otherwise: their 16-bit value bins are kept in LDS
    int bins_words;               // 32-bit words those bins take (candidate positions follow)
    // level two of the two-level top-k: candidate blocks [B*S, cand_k] of cand_bs rows
    // (masked kernels only; 1 <= cand_k <= 2048)
    const int32_t *cand = nullptr;
    int cand_k = 0, cand_bs = 1;
    // level one of a candidate source: per query, the maxima of blocks of bmax_bs rows of
    // the unmasked scores (the newest visible block +inf), [B*S, ldb]; NULL: none.  The
    // chunk is a multiple of bmax_bs, so each block lies in one member's chunk.
    float *bmax = nullptr;
    long ldb = 0;
    int bmax_bs = 1;
};
struct FusedPlan {
    bool ok;
    int n_teams, team_size, chunk, win_tiles, n_slots, grid, vbins;
    bool cache_lds, lds_bins;
    long ld;
    size_t dyn_bytes;
};
FusedPlan plan_fused(int fmt, bool masked, bool qkv, bool layers, int B, int S, int start_pos, int ratio, int Hi,
                     int Di, int D, int dv, int W, int keff);
size_t fused_state_bytes(const FusedPlan &p);  // zero-filled before first use
size_t fused_ws_bytes(const FusedPlan &p, int dv, int layers);
// Bytes of one query's partial states (every member and layer): the kernel addresses
// them with 32-bit offsets, so a plan is usable only while this stays below 2^31.
size_t fused_part_bytes_per_query(const FusedPlan &p, int dv, int layers);
// err_word: where a team timeout is reported (NULL: the state's first word).
hipError_t launch_fused(FusedArgs f, const FusedPlan &p, void *ws, void *state, hipStream_t stream,
                        uint32_t *err_word = nullptr);
// The fused kernel's forms: index-code format x level-two masking x quantised attention
// KV x several layers over one top-k.  fused_forms.hip is compiled once per entry, with
// the entry's fields as macros, and defines that form's launcher and occupancy query.
//   X(name, index format, masking, quantised KV, layers)
// masking: rows outside the query's candidate blocks score -inf (FusedArgs::cand);
// quantised KV: the attention sources are codes (AttnArgs win_codes / comp_codes);
// layers: AttnArgs::L layers attend over the step's top-k.
#define LIT_FUSED_FORMS(X)                                  \
    X(e4m3, kFmtE4M3, false, false, false)                  \
    X(e2m1, kFmtE2M1, false, false, false)                  \
    X(e4m3_cand, kFmtE4M3, true, false, false)              \
    X(e2m1_cand, kFmtE2M1, true, false, false)              \
    X(e4m3_qkv, kFmtE4M3, false, true, false)               \
    X(e2m1_qkv, kFmtE2M1, false, true, false)               \
    X(e4m3_layers, kFmtE4M3, false, false, true)            \
    X(e2m1_layers, kFmtE2M1, false, false, true)            \
    X(e4m3_qkv_cand, kFmtE4M3, true, true, false)           \
    X(e2m1_qkv_cand, kFmtE2M1, true, true, false)           \
    X(e4m3_qkv_layers, kFmtE4M3, false, true, true)         \
    X(e2m1_qkv_layers, kFmtE2M1, false, true, true)         \
    X(e4m3_cand_layers, kFmtE4M3, true, false, true)        \
    X(e2m1_cand_layers, kFmtE2M1, true, false, true)        \
    X(e4m3_qkv_cand_layers, kFmtE4M3, true, true, true)     \
    X(e2m1_qkv_cand_layers, kFmtE2M1, true, true, true)
// Per form: launch, and co-resident workgroups per CU for a shape (0 when not instantiated).
#define LIT_FUSED_DECLARE(name, fmt, mask, qkv, layers)                                                   \
    hipError_t launch_fused_##name(const FusedArgs &f, int grid, size_t dyn_bytes, hipStream_t stream); \
    int fused_per_cu_##name(int D, int DI, int HT, size_t dyn_bytes, bool cached);
LIT_FUSED_FORMS(LIT_FUSED_DECLARE)
#undef LIT_FUSED_DECLARE

}  // namespace lit
