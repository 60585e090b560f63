// attention.hip -- sparse gather-attention over the sliding window and the selected
// compressed rows, plus the window row lists.
//
// What is computed (DeepSeek-V4.1-Flash-NVFP4 inference/model.py, Attention.forward
// and its sparse_attn call; DeepSeek-V3.2-Exp inference/model.py, MLA.forward gives
// the dense equivalent): for every query (b, i) and head h, over the row set J = the
// listed window slots followed by the listed compressed rows (-1 skipped),
//   l_j = scale * q[h] . row_j,   o[h] = sum_j e^(l_j) row_j[:dv] / (sum_j e^(l_j) + e^(sink_h)).
// One bf16 row is both key and value (a single shared latent head).
//
// Mapping onto the chip.  A wave takes 32 listed rows at a time.  Each lane (g, c)
// gathers 16-byte pieces of row c (and row 16+c) straight from HBM: these are the
// A operands of V_MFMA_F32_16X16X32_BF16 for S^T = rows x Q^T (32 head dims per
// instruction; Q^T stays in VGPRs), so lane (g, h) ends up holding the 8 logits of
// head h for rows 4g..4g+3 and 16+4g..16+4g+3.  The online softmax for head h is
// therefore per lane (plus two cross-lane max/sum steps), and the 8 probabilities,
// rounded to bf16, are already the B operand of O^T = V^T x P^T.  V^T needs the same
// rows column-wise, so the gathered rows are also written once to LDS and read back
// transposed (8 row entries of one column per lane).  O^T accumulates in fp32 VGPRs,
// lane (g, h) owning dims 4g..4g+3 of every 16-dim tile for head h.
//
// A query's list is cut into splits (workgroups of 4 waves); the 4 waves of a split
// merge through LDS, and a second kernel merges splits (log-sum-exp), adds the sink
// and writes bf16.  With a single split the first kernel writes bf16 itself.
//
// Several layers can share one call (DeepSeek-V4.1-Flash-NVFP4 inference/model.py:
// layers between index sources reuse the source's top-k list and the shared compressed
// KV, each with its own queries, window KV and sink): the grid then holds every layer's
// workgroups, those of one query side by side.
#include "tile_ops.h"

namespace lit {

namespace {

constexpr int kWaves = 4;
constexpr int kHeads = 16;

// Row of list entry p as an index into its source ([B*R] window slots or [B*T_cap]
// compressed rows), or -1; `win` tells which source (padded list: window entries occupy
// [0, wpad), wpad a multiple of 32).
__device__ inline long list_row_index(const AttnArgs &a, int b, int i, int nwin, int wpad, const WindowBase &wb,
                                      int p, bool &win) {
    const size_t bs = (size_t)b * a.S + i;
    win = p < wpad;
    if (win) {
        if (p >= nwin) return -1;
        const int slot = a.win_idx ? a.win_idx[bs * a.W + p] : window_slot_at(wb, a.start_pos, a.R, i, p);
        if (slot < 0 || slot >= a.R) return -1;
        return (long)b * a.R + slot;
    }
    const int t = a.comp_idx[bs * a.K + (p - wpad)];
    if (t < 0 || t >= a.T_cap) return -1;
    return (long)b * a.T_cap + t;
}

// One tile of rows from a quantised list (window tiles and compressed tiles are
// separate, so the format is uniform over the wave).
template <int D, int WF, int CF>
__device__ inline void quant_tile_load(AttnRows<D> &rows, const AttnArgs &a, int b, int i, int nwin, int wpad,
                                       const WindowBase &wb, int p0, int p1, int end, int g) {
    bool w0, w1;
    const long r0 = p0 < end ? list_row_index(a, b, i, nwin, wpad, wb, p0, w0) : -1;
    const long r1 = p1 < end ? list_row_index(a, b, i, nwin, wpad, wb, p1, w1) : -1;
    if (p0 - (p0 & 31) < wpad) {  // a window tile
        if constexpr (WF == kKvBf16)
            attn_tile_load<D>(rows, r0 >= 0 ? a.win_kv + (size_t)r0 * D : nullptr,
                              r1 >= 0 ? a.win_kv + (size_t)r1 * D : nullptr, g);
        else
            kv_tile_load<D, WF>(rows, a.win_codes, a.win_scales, r0, r1, g);
    } else {
        if constexpr (CF == kKvBf16)
            attn_tile_load<D>(rows, r0 >= 0 ? a.comp_kv + (size_t)r0 * D : nullptr,
                              r1 >= 0 ? a.comp_kv + (size_t)r1 * D : nullptr, g);
        else
            kv_tile_load<D, CF>(rows, a.comp_codes, a.comp_scales, r0, r1, g);
    }
}

// Layer l's view of the arguments (its q, window source, sink and output).
__device__ inline AttnArgs layer_args(const AttnArgs &a0, int l) {
    AttnArgs a = a0;
    a.q += (size_t)l * a.q_ls;
    if (a.win_kv) a.win_kv += (size_t)l * a.win_ls;
    if (a.win_codes) {  // quantised window: codes and scales per layer
        a.win_codes += (size_t)l * a.win_ls;
        a.win_scales += (size_t)l * a.win_ls / (a.win_fmt == kKvE4M3 ? 32 : 16);
    }
    if (a.sink) a.sink += (size_t)l * kHeads;
    a.out += (size_t)l * a.out_ls;
    return a;
}

template <int D, int WF, int CF>
__global__ __launch_bounds__(kWaves * 64) void sparse_attn_kernel(AttnArgs a0, AttnPlan pl) {
    constexpr bool QUANT = WF != kKvBf16 || CF != kKvBf16;
    constexpr int LD = D + 4;       // LDS row stride in bf16 (8 bytes of padding)
    __shared__ __attribute__((aligned(16))) uint16_t lds[kWaves * 32 * LD];
    __shared__ float wm[kWaves][kHeads], wl[kWaves][kHeads];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: tile bases are scalars
    const int g = lane >> 4;
    const int c = lane & 15;
    // the layers of one query are neighbours in the grid, so they run together and the
    // shared rows one of them gathers are cache hits for the others
    const int layer = blockIdx.y % a0.L;
    const int bs = blockIdx.y / a0.L;
    const AttnArgs a = layer_args(a0, layer);
    const int b = bs / a.S;
    const int i = bs % a.S;
    const int split = blockIdx.x;
    const int nwin = a.win_idx ? a.W : (a.W > 0 ? window_width(a.S, a.start_pos, a.W) : 0);
    const WindowBase wb = window_base(a.start_pos, a.W, a.R > 0 ? a.R : 1, i);
    const int list_len = attn_list_len(nwin, a.K);
    const int wpad = list_len - a.K;  // window entries, padded to whole tiles
    const int ndt = a.dv / 16;
    const float sl2 = a.scale * kLog2e;

    bf16x8 qb[D / 32];
    load_q_operands<D>(qb, a.q, (size_t)bs, g, c);
    AttnState<D> st;
    attn_init<D>(st);

    uint16_t *tile = lds + wave * 32 * LD;
    const int split_begin = split * kWaves * pl.tiles_per_wave * 32;
    const int split_end = min(list_len, split_begin + kWaves * pl.tiles_per_wave * 32);

    const int first = split_begin + wave * pl.tiles_per_wave * 32;
    if constexpr (QUANT) {
        for (int it = 0; it < pl.tiles_per_wave; ++it) {
            const int base = first + it * 32;
            if (base >= split_end) break;
            AttnRows<D> rows;
            quant_tile_load<D, WF, CF>(rows, a, b, i, nwin, wpad, wb, base + c, base + 16 + c, split_end, g);
            attn_tile_compute<D>(st, qb, rows, tile, ndt, sl2, g, c);
        }
    } else {
        // bf16 sources by buffer loads: a tile is all window or all compressed entries
        // (the window part of the list is padded to whole tiles), so its source is
        // uniform; a lane without a row reads zeros from past the source's end.  The
        // list entries of the next tile are requested before the current tile's rows
        // are used, so their round trip overlaps the current tile's.
        const uint16_t *wsrc = a.win_kv ? a.win_kv + (size_t)b * a.R * D : nullptr;
        const uint16_t *csrc = a.comp_kv ? a.comp_kv + (size_t)b * a.T_cap * D : nullptr;
        const rsrc_t win_r = make_rsrc(wsrc, wsrc ? (uint32_t)a.R * D * 2u : 0u);
        const rsrc_t comp_r = make_rsrc(csrc, csrc ? (uint32_t)a.T_cap * D * 2u : 0u);
        const rsrc_t widx_r = make_rsrc(a.win_idx ? a.win_idx + (size_t)bs * a.W : nullptr,
                                        a.win_idx ? (uint32_t)a.W * 4u : 0u);
        const rsrc_t cidx_r = make_rsrc(a.comp_idx ? a.comp_idx + (size_t)bs * a.K : nullptr,
                                        a.comp_idx ? (uint32_t)a.K * 4u : 0u);
        const bool derived = a.win_idx == nullptr;
        const int wave_end = min(split_end, first + pl.tiles_per_wave * 32);  // this wave's entries
        // entries of the tile at `base` for this lane's rows base+c and base+16+c: a
        // loaded entry (window slot or compressed row), a derived window slot, and
        // whether the list position is inside the split and the window / list
        int ld0, ld1, sl0 = -1, sl1 = -1;
        bool ok0, ok1;
        auto fetch = [&](int base) {
            const bool win = base < wpad;
            const int p0 = base + c, p1 = base + 16 + c;
            const rsrc_t ir = win ? widx_r : cidx_r;
            const int o = win ? 0 : wpad;
            ld0 = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (int)(4u * (uint32_t)(p0 - o)), 0, 0);
            ld1 = (int)__builtin_amdgcn_raw_buffer_load_b32(ir, (int)(4u * (uint32_t)(p1 - o)), 0, 0);
            if (win && derived) {
                sl0 = window_slot_at(wb, a.start_pos, a.R, i, p0);
                sl1 = window_slot_at(wb, a.start_pos, a.R, i, p1);
            }
            ok0 = p0 < wave_end && (!win || p0 < nwin);
            ok1 = p1 < wave_end && (!win || p1 < nwin);
        };
        fetch(first);
        for (int it = 0; it < pl.tiles_per_wave; ++it) {
            const int base = first + it * 32;
            if (base >= wave_end) break;
            const bool win = base < wpad;
            const int e0 = win && derived ? sl0 : ld0, e1 = win && derived ? sl1 : ld1;
            const uint32_t lim = win ? (uint32_t)a.R : (uint32_t)a.T_cap;
            const uint32_t off0 = ok0 && (uint32_t)e0 < lim ? (uint32_t)e0 * (2u * D) : kOffNone;
            const uint32_t off1 = ok1 && (uint32_t)e1 < lim ? (uint32_t)e1 * (2u * D) : kOffNone;
            AttnRows<D> rows;
            attn_tile_load_buf<D>(rows, win ? win_r : comp_r, off0, off1, g);
            fetch(base + 32);  // past the wave's entries: every entry comes back not ok
            attn_tile_compute<D>(st, qb, rows, tile, ndt, sl2, g, c);
        }
    }
    __syncthreads();  // every wave is done with its LDS rows
    // Reuse the row buffer for the 4 waves' states.
    float *ow = reinterpret_cast<float *>(lds);
    attn_wave_publish<D>(st, ow, &wm[0][0], &wl[0][0], wave, a.dv, g, c);
    __syncthreads();

    const bool direct = pl.n_splits == 1;
    for (int e = threadIdx.x; e < kHeads * a.dv; e += kWaves * 64) {
        const int h = e / a.dv;
        const int d = e - h * a.dv;
        float O, M, L;
        attn_combine(ow, &wm[0][0], &wl[0][0], kWaves, h, d, a.dv, O, M, L);
        if (direct) {
            a.out[((size_t)bs * kHeads + h) * a.dv + d] = attn_finish(O, M, L, a.sink, h);
        } else {
            float *dst = a.part + ((((size_t)layer * a.B * a.S + bs) * pl.n_splits + split) * kHeads + h) * (a.dv + 2);
            dst[d] = O;
            if (d == 0) {
                dst[a.dv] = M;
                dst[a.dv + 1] = L;
            }
        }
    }
}

// Many queries (chunked prefill): one wave per (layer, query) walks the query's whole
// list, so no state is merged across waves or workgroups.  bf16 rows are gathered
// coalesced into the wave's LDS tile (tile_ops.h, RowPieces): a tile's rows are requested
// a tile ahead and its list entries two tiles ahead, so the gather overlaps a whole tile
// of compute.  The four waves of a workgroup share nothing but the launch (a wave past
// the last query returns at once; no workgroup barrier follows).
constexpr int kWaveRG = 4;  // V^T tiles read per group (fewer live registers)
template <int D, int WF, int CF>
__global__ __launch_bounds__(kWaves * 64) void sparse_attn_wave_kernel(AttnArgs a0, int n_queries) {
    constexpr bool QUANT = WF != kKvBf16 || CF != kKvBf16;
    constexpr int LDR = QUANT ? D + 4 : D + 8;  // LDS row stride (16-byte aligned rows for the staged form)
    __shared__ __attribute__((aligned(16))) uint16_t lds[kWaves * 32 * LDR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4;
    const int c = lane & 15;
    const int qq = blockIdx.x * kWaves + wave;
    if (qq >= n_queries) return;
    const int layer = qq % a0.L;  // the layers of one query are neighbours
    const int bs = qq / a0.L;
    const AttnArgs a = layer_args(a0, layer);
    const int b = bs / a.S;
    const int i = bs % a.S;
    const int nwin = a.win_idx ? a.W : (a.W > 0 ? window_width(a.S, a.start_pos, a.W) : 0);
    const WindowBase wb = window_base(a.start_pos, a.W, a.R > 0 ? a.R : 1, i);
    const int list_len = attn_list_len(nwin, a.K);
    const int wpad = list_len - a.K;
    const int ndt = a.dv / 16;
    const float sl2 = a.scale * kLog2e;

    bf16x8 qb[D / 32];
    load_q_operands<D>(qb, a.q, (size_t)bs, g, c);
    AttnState<D> st;
    attn_init<D>(st);
    uint16_t *tile = lds + wave * 32 * LDR;

    if constexpr (QUANT) {
        AttnRows<D> rows;
        quant_tile_load<D, WF, CF>(rows, a, b, i, nwin, wpad, wb, c, 16 + c, list_len, g);
        for (int base = 0; base < list_len; base += 32) {
            const AttnLogits lg = attn_tile_logits<D>(qb, rows, tile, g, c);
            const int nb = base + 32;
            if (nb < list_len)
                quant_tile_load<D, WF, CF>(rows, a, b, i, nwin, wpad, wb, nb + c, nb + 16 + c, list_len, g);
            attn_tile_update<D, kWaveRG, LDR>(st, lg, tile, ndt, sl2, g, c);
        }
    } else {
        const uint16_t *wsrc = a.win_kv ? a.win_kv + (size_t)b * a.R * D : nullptr;
        const uint16_t *csrc = a.comp_kv ? a.comp_kv + (size_t)b * a.T_cap * D : nullptr;
        const rsrc_t win_r = make_rsrc(wsrc, wsrc ? (uint32_t)a.R * D * 2u : 0u);
        const rsrc_t comp_r = make_rsrc(csrc, csrc ? (uint32_t)a.T_cap * D * 2u : 0u);
        const rsrc_t widx_r = make_rsrc(a.win_idx ? a.win_idx + (size_t)bs * a.W : nullptr,
                                        a.win_idx ? (uint32_t)a.W * 4u : 0u);
        const rsrc_t cidx_r = make_rsrc(a.comp_idx ? a.comp_idx + (size_t)bs * a.K : nullptr,
                                        a.comp_idx ? (uint32_t)a.K * 4u : 0u);
        const bool derived = a.win_idx == nullptr;
        const int r = lane & 31;  // the tile row whose entry this lane holds
        // the list entry of row r of the tile at `base` (past a list its buffer reads 0)
        auto request = [&](int base) {
            const bool win = base < wpad;
            return (int)__builtin_amdgcn_raw_buffer_load_b32(win ? widx_r : cidx_r,
                                                             (int)(4u * (uint32_t)(base + r - (win ? 0 : wpad))), 0, 0);
        };
        // its byte offset in the tile's source, kOffNone when the row is not listed
        auto offset_of = [&](int base, int e) {
            const bool win = base < wpad;
            const int p = base + r;
            const int ent = win && derived ? window_slot_at(wb, a.start_pos, a.R, i, p) : e;
            const bool ok = p < list_len && (!win || p < nwin);
            const uint32_t lim = win ? (uint32_t)a.R : (uint32_t)a.T_cap;
            return ok && (uint32_t)ent < lim ? (uint32_t)ent * (2u * D) : kOffNone;
        };
        auto src_of = [&](int base) { return base < wpad ? win_r : comp_r; };
        RowPieces<D> rp;
        int ent = request(0);
        row_pieces_load<D>(rp, src_of(0), offset_of(0, ent), lane);
        ent = request(32);
        row_pieces_stage<D, LDR>(rp, tile, lane);
        uint64_t valid = rp.valid;
        row_pieces_load<D>(rp, src_of(32), offset_of(32, ent), lane);
        ent = request(64);
        wave_lds_sync();
        for (int base = 0; base < list_len; base += 32) {
            const AttnLogits lg = attn_tile_logits_lds<D, LDR>(qb, valid, tile, g, c);
            attn_tile_update<D, kWaveRG, LDR>(st, lg, tile, ndt, sl2, g, c);  // ends with the reads done
            // the next tile's rows (requested a tile ago) into LDS; the one after is requested
            row_pieces_stage<D, LDR>(rp, tile, lane);
            valid = rp.valid;
            row_pieces_load<D>(rp, src_of(base + 64), offset_of(base + 64, ent), lane);
            ent = request(base + 96);
            wave_lds_sync();
        }
    }

    // lane (g, h) holds dims 16dt+4g..16dt+4g+3 of head h: normalise and store 4 bf16
    attn_wave_total<D>(st);
    uint16_t *orow = a.out + ((size_t)bs * kHeads + c) * a.dv + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        if (dt < ndt) *reinterpret_cast<u32x2 *>(orow + 16 * dt) = attn_finish4(st.o[dt], st.m, st.l, a.sink, c);
}

// Split merge: one wave per (query, head).  Lane s holds split s's max and
// normaliser (several splits per lane when there are more than 64); the wave reduces
// them, leaves each split's weight e^(m_s - M) / L in LDS, and then every lane sums
// its output dims over the splits with independent loads.
constexpr int kMaxSplits = 1024;

__global__ __launch_bounds__(64) void attn_merge_kernel(AttnArgs a0, AttnPlan pl) {
    __shared__ float wgt[kMaxSplits];
    const int layer = blockIdx.x % a0.L;
    const int bs = blockIdx.x / a0.L;
    const AttnArgs a = layer_args(a0, layer);
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int ns = pl.n_splits;
    const size_t stride = (size_t)kHeads * (a.dv + 2);
    const float *src = a.part + (((size_t)layer * a.B * a.S + bs) * ns * kHeads + h) * (a.dv + 2);
    const float s2 = a.sink ? a.sink[h] * kLog2e : -INFINITY;
    float M = s2;
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, src[s * stride + a.dv]);
    M = wave_max_f(M);
    float L = 0.f;
    for (int s = lane; s < ns; s += 64) {
        const float ms = src[s * stride + a.dv];
        const float f = (ms == -INFINITY || M == -INFINITY) ? 0.f : exp2f(ms - M);
        wgt[s] = f;
        L += f * src[s * stride + a.dv + 1];
    }
    L = wave_sum_f(L);
    if (a.sink && M != -INFINITY) L += exp2f(s2 - M);
    const float inv = L > 0.f ? 1.f / L : 0.f;
    __syncthreads();
    for (int d = lane; d < a.dv; d += 64) {
        float O = 0.f;
        int s = 0;
        for (; s + 8 <= ns; s += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = src[(s + u) * stride + d];
#pragma unroll
            for (int u = 0; u < 8; ++u) O += wgt[s + u] * v[u];
        }
        for (; s < ns; ++s) O += wgt[s] * src[s * stride + d];
        a.out[((size_t)bs * kHeads + h) * a.dv + d] = __builtin_bit_cast(uint16_t, (__bf16)(O * inv));
    }
}

__global__ void window_indices_kernel(int B, int S, int start_pos, int W, int R, int width,
                                      int32_t *win_idx) {
    const long n = (long)B * S * width;
    for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
        const int j = (int)(e % width);
        const int i = (int)((e / width) % S);
        win_idx[e] = window_slot(S, start_pos, W, R, i, j);
    }
}

template <int D, int WF, int CF>
hipError_t launch_d(const AttnArgs &a, const AttnPlan &p, hipStream_t stream) {
    if (p.per_wave) {
        const int nq = a.B * a.S * a.L;
        hipLaunchKernelGGL((sparse_attn_wave_kernel<D, WF, CF>), dim3((nq + kWaves - 1) / kWaves),
                           dim3(kWaves * 64), 0, stream, a, nq);
        return hipGetLastError();
    }
    dim3 grid(p.n_splits, a.B * a.S * a.L);
    hipLaunchKernelGGL((sparse_attn_kernel<D, WF, CF>), grid, dim3(kWaves * 64), 0, stream, a, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_splits == 1) return e;
    hipLaunchKernelGGL(attn_merge_kernel, dim3(a.B * a.S * a.L, kHeads), dim3(64), 0, stream, a, p);
    return hipGetLastError();
}

}  // namespace

AttnPlan plan_attention(int B, int S, int list_len) {
    AttnPlan p;
    p.list_len = list_len;
    const int tiles = (list_len + 31) / 32;
    const int queries = B * S > 0 ? B * S : 1;  // an empty batch sizes like one query
    // Enough queries to give every SIMD several waves: one wave per query (no merges).
    p.per_wave = queries >= kWaveFormQueries;
    if (p.per_wave) {
        p.n_splits = 1;
        p.tiles_per_wave = tiles;
        return p;
    }
    // Aim for at least ~512 workgroups, but never fewer than one tile per wave.
    int splits = (512 + queries - 1) / queries;
    const int max_splits = (tiles + kWaves - 1) / kWaves;
    if (splits > max_splits) splits = max_splits;
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits < 1) splits = 1;
    p.tiles_per_wave = (tiles + kWaves * splits - 1) / (kWaves * splits);
    if (p.tiles_per_wave < 1) p.tiles_per_wave = 1;
    p.n_splits = (tiles + kWaves * p.tiles_per_wave - 1) / (kWaves * p.tiles_per_wave);
    if (p.n_splits < 1) p.n_splits = 1;
    return p;
}

size_t attention_partial_bytes(int B, int S, int H, int dv, const AttnPlan &p) {
    if (p.per_wave || p.n_splits <= 1) return 0;
    return (size_t)B * S * p.n_splits * H * (dv + 2) * sizeof(float);
}

template <int WF, int CF>
hipError_t launch_fmt(const AttnArgs &a, const AttnPlan &p, hipStream_t stream) {
    switch (a.D) {
        case 64: return launch_d<64, WF, CF>(a, p, stream);
        case 128: return launch_d<128, WF, CF>(a, p, stream);
        case 192: return launch_d<192, WF, CF>(a, p, stream);
        case 256: return launch_d<256, WF, CF>(a, p, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_sparse_attn(const AttnArgs &a, const AttnPlan &p, hipStream_t stream) {
    if (a.B <= 0 || a.S <= 0) return hipSuccess;
    const bool qw = a.win_fmt == kKvE4M3, qc = a.comp_fmt == kKvE2M1;
    if ((a.win_fmt != kKvBf16 && !qw) || (a.comp_fmt != kKvBf16 && !qc)) return hipErrorInvalidValue;
    if (qw && qc) return launch_fmt<kKvE4M3, kKvE2M1>(a, p, stream);
    if (qw) return launch_fmt<kKvE4M3, kKvBf16>(a, p, stream);
    if (qc) return launch_fmt<kKvBf16, kKvE2M1>(a, p, stream);
    return launch_fmt<kKvBf16, kKvBf16>(a, p, stream);
}

hipError_t launch_window_indices(int B, int S, int start_pos, int W, int R, int32_t *win_idx,
                                 hipStream_t stream) {
    const int width = window_width(S, start_pos, W);
    const long n = (long)B * S * width;
    if (n <= 0) return hipSuccess;
    const int threads = 256;
    long blocks = (n + threads - 1) / threads;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(window_indices_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, B, S,
                       start_pos, W, R, width, win_idx);
    return hipGetLastError();
}

}  // namespace lit
