// fused_kernel.h -- the whole sparse-attention step for decode-sized batches in one
// launch: indexer scores -> exact top-k -> gather attention -> merge.  Included by one
// source file per index-code format and variant (fused_e4m3.hip, fused_e2m1.hip, their
// _cand forms for level-two layers of the two-level top-k, _qkv forms for quantised
// attention KV and _layers forms for several layers over one top-k), each of which
// instantiates its kernels; fused_decode.hip plans and dispatches.
//
// What is computed is exactly what indexer.hip, topk.hip and attention.hip compute
// (DeepSeek-V4.1-Flash-NVFP4 inference/model.py, Indexer.forward and
// Attention.forward; the window rows of get_window_topk_idxs), but in one kernel:
// at decode every kernel boundary of a dependent chain costs several microseconds on
// MI355X, which is more than the streaming time of a whole 16K-context step.
//
// Organisation.  Every query (b, i) gets a team of `team_size` workgroups; the grid is
// sized so that every workgroup is resident at once (at most the co-resident capacity
// of the device), and the teams are laid out XCD-major so that a team shares one XCD
// where the sizes allow.  Member m of a team owns key chunk [m*chunk, (m+1)*chunk) of
// its query's visible rows and keeps that chunk's scores in LDS.
//   A. Every member scores its chunk (MX-scaled fp8 or fp4 MFMA, as in indexer.hip; in the
//      MASK form rows outside the query's candidate blocks then score -inf).  When the
//      query sees more rows than it keeps, it publishes the chunk's scores to the team
//      buffer and its chunk's max / min score keys in its barrier-A flag.
//   -- team barrier A (skipped when every visible row is kept) --
//   S. Every member loads all of the team's scores and finds, on its own, the exact k-th
//      (key, position) with the value-bin selection of select_ops.h: a 4096-bin histogram
//      between the team's min and max, the bin where the count from the top reaches k,
//      then the few scores of that bin ranked exactly (narrowed first when there are
//      many; radix levels when they overflow LDS).  Every member reaches the same cut
//      from the same data.  Once the cut's bin is known, each wave requests its first
//      tile of candidate rows, so the row gather overlaps the rest of the selection.
//   D. Every member attends over its share of the window rows and over its chunk's picks
//      (candidates that miss the cut are masked), counts its picks from the tiles'
//      masks, and publishes its partial state -- for each layer that shares the top-k,
//      one after the other, in the LAYERS form.
//   -- team barrier C (the flag carries the member's pick count) --
//   M. Members merge the team's partial states (log-sum-exp) for a slice of the
//      (layer, head, dim) outputs, add the sink, and write bf16.  Meanwhile the wave without
//      merge work writes the member's picks to the top-k list (ascending), at the offset
//      the pick counts of the members before it give (when every wave merges, each wave
//      writes a quarter of the chunk's picks after its merge share).
//
// Cross-workgroup data moves through agent-scope relaxed atomic loads and stores and
// coherent (sc1) 16-byte buffer loads and stores.  The barriers are flag arrays, not
// counters: a member waits for its own stores to complete (vmcnt) and then writes a
// 16-byte flag tagged with the query index and the query's launch count, kept in the
// state buffer; waiters poll one flag per lane.  No two workgroups update one address
// and no agent-scope fence is used (on this device such a fence writes back or
// invalidates a whole XCD's L2).
//
// Every wait is a bounded spin: if a team does not assemble in time (workgroups not
// co-resident, e.g. another kernel holding CUs), the waiter sets the sticky error word
// and goes on, so the kernel always finishes; results are then undefined and the
// error word reports it.
#pragma once

#include <type_traits>

#include "select_ops.h"

namespace lit {

namespace {

constexpr int kThreads = kSelThreads;
constexpr int kHeads = 16;
constexpr int kCacheQ = 8;      // team score quads per thread kept in registers (and LDS)
constexpr int kBatch = 16;      // team score quads per thread loaded per round (uncached form)
constexpr int kChunkMax = 8192;     // largest member chunk the plan takes
constexpr int kFusedCandMax = 2048; // candidate blocks per query the fused level two takes

// Per-query region of the state buffer, at a fixed stride whatever the team size: the
// query's launch counter, then one 16-byte flag slot per member for each of the two
// team barriers (A: scores published, C: partial state published).
constexpr int kTeamMax = kThreads;
constexpr size_t kQCtrl = 256;
constexpr size_t kQState = kQCtrl + 2 * (size_t)kTeamMax * 16;

__device__ inline uint32_t ld_agent(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st_agent(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline float ldf_agent(const float *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void stf_agent(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread's earlier global stores and atomics have completed (gfx9 counts stores
// in vmcnt).  A compiler barrier on both sides keeps memory operations from moving
// across it.
__device__ inline void stores_done() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt(7), lgkmcnt(15)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

struct FusedLds : SelLds {
    float fred[kThreads / 64];
    int wcnt[kThreads / 64];      // per-wave counts (attention list; then the top-k list ranges)
    uint32_t mm[kThreads / 64][2];
    uint32_t cnt[kTeamMax];       // the team's pick counts (from barrier C)
    uint32_t wpick[kThreads / 64];  // this member's picks counted by each wave
};

// Lane exchange within a row of 16 lanes by DPP (no LDS round trip).
template <int CTRL>
__device__ inline float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ inline uint64_t pack2(float a, float b) {
    return (uint64_t)__float_as_uint(a) | ((uint64_t)__float_as_uint(b) << 32);
}
__device__ inline float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ inline float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }
__device__ inline uint64_t ld64_agent(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void st64_agent(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int kSc1 = 16;  // buffer cache policy: coherent at agent scope (sc1)
__device__ inline u32x4 ld128_agent(rsrc_t r, uint32_t byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kSc1);
}
__device__ inline void st128_agent(rsrc_t r, uint32_t byte_off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)byte_off, 0, kSc1);
}

// Team barrier by flags.  A member publishes its slot {x, y, q, epoch} once every one of
// its earlier stores has completed; a waiter polls slot j on lane j until the slot carries
// this launch's tag.  The tag holds the query index as well as the query's launch count,
// so a slot left by an earlier launch (of any shape) never matches.  Waits are bounded:
// past `limit` polls the sticky error word is set and the wait gives up.
__device__ inline void team_flag(const rsrc_t &slots, int m, uint32_t x, uint32_t y, uint32_t q, uint32_t ep) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) st128_agent(slots, (uint32_t)m * 16u, u32x4{x, y, q, ep});
}

__device__ inline u32x4 team_poll(const rsrc_t &slots, int team, uint32_t q, uint32_t ep, uint32_t limit,
                                  uint32_t *err, uint32_t *x_out = nullptr) {
    u32x4 v = {0u, 0u, 0u, 0u};
    const int j = threadIdx.x;
    if (j < team) {
        uint32_t n = 0;
        for (;;) {
            v = ld128_agent(slots, (uint32_t)j * 16u);
            if (v[2] == q && v[3] == ep) break;
            if (++n > limit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        if (x_out) x_out[j] = v[0];
    }
    __syncthreads();
    return v;
}
// Workgroup max / min / sum (every thread gets the result).
__device__ inline float wg_max(float v, float *red) {
    v = wave_max_f(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}
__device__ inline float wg_min(float v, float *red) {
    v = wave_min_f(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fminf(r, red[w]);
    __syncthreads();
    return r;
}
__device__ inline uint32_t wg_sum(uint32_t v, uint32_t *red) {
    v = wave_sum_u32(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r += red[w];
    __syncthreads();
    return r;
}

// CACHED: the team's scores fit the per-thread register cache (and LDS).  The two forms
// are separate kernels so that the re-reading form's loads never share a code path with
// the cached form (a load pending on one path of a branch makes the compiler wait for
// every load in flight where the paths join, which would stall the early row gather).
// MASK: a level-two layer of the two-level top-k (DeepSeek-V4.1-Flash-NVFP4 model.py,
// Indexer.forward with candidates): rows outside the query's candidate blocks score
// -inf before the selection.
// QKV: the attention KV sources are quantised (window e4m3 / ue8m0-32, compressed
// e2m1 / e4m3-16); rows are loaded as codes and dequantised when their tile is computed.
// LAYERS: several layers share the step's top-k (AttnArgs::L of them attend); without it
// the layer count is the constant 1.
template <int D, int DI, int FMT, int HT, bool CACHED, bool MASK, bool QKV, bool LAYERS>
__global__ __launch_bounds__(kThreads) void fused_decode_kernel(FusedArgs f) {
    using WinRows = std::conditional_t<QKV, KvRows<D, kKvE4M3>, AttnRows<D>>;
    using PickRows = std::conditional_t<QKV, KvRows<D, kKvE2M1>, AttnRows<D>>;
    constexpr int LD = D + 4;
    __shared__ FusedLds sm;
    __shared__ __attribute__((aligned(16))) uint16_t attn_lds[4 * 32 * LD];  // rows / candidates / merge
    __shared__ float wm[4 * kHeads], wl[4 * kHeads];
    __shared__ float hf[4 * kHeads], hl[kHeads], hm[kHeads];  // per-head merge factors
    extern __shared__ __attribute__((aligned(16))) float dyn[];  // chunk scores, picks (ints), team scores
    __shared__ uint32_t ckeep[MASK ? kChunkMax / 32 + 2 : 1];  // kept candidate blocks of this chunk

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;

    // team / member of this workgroup (XCD-major order when the grid allows it)
    const int G = gridDim.x;
    const int lin = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    // (the divisions by launch constants are multiplies by their FastDiv multipliers: they
    // stand before the first key loads)
    const int q = fdiv(lin, f.div_team);
    const int m = lin - q * f.team_size;
    const IndexerArgs &ia = f.ia;
    const AttnArgs &aa = f.aa;
    const int b = fdiv(q, f.div_S);
    const int i = q - b * ia.S;
    const int nvis = min(ia.T, fdiv(ia.start_pos + i + 1, f.div_ratio));
    const bool select = nvis > f.keff;  // otherwise every visible row is picked
    const int c0 = m * f.chunk;
    const int c1 = min(c0 + f.chunk, nvis);
    const int n = max(0, c1 - c0);
    char *qstate = f.qstate + (size_t)q * kQState;
    uint32_t *epoch = reinterpret_cast<uint32_t *>(qstate);
    const uint32_t ep = ld_agent(epoch) + 1u;  // this launch's tag
    const rsrc_t slot_a = make_rsrc(qstate + kQCtrl, kTeamMax * 16u);
    const rsrc_t slot_c = make_rsrc(qstate + kQCtrl + kTeamMax * 16, kTeamMax * 16u);
    float *ts = f.scores + (size_t)q * f.ld;  // the team's scores
    const rsrc_t ts_r = make_rsrc(ts, (uint32_t)f.ld * 4u);
    float *sc = dyn;
    int *picks = reinterpret_cast<int *>(dyn + f.chunk);
    float *tsl = dyn + 2 * f.chunk;  // the team's scores in position order (cached form)


    // level two: the query's candidate blocks are requested now and turned into a bitmap
    // of the blocks that meet this member's chunk after scoring
    int cblk[MASK ? kFusedCandMax / kThreads : 1];
    const int blk0 = MASK ? fdiv(c0, f.div_cbs) : 0;
    const int nbk = MASK && n > 0 ? fdiv(c1 - 1, f.div_cbs) - blk0 + 1 : 0;
    if constexpr (MASK) {
        const int32_t *cl = f.cand + (size_t)q * f.cand_k;
#pragma unroll
        for (int r = 0; r < kFusedCandMax / kThreads; ++r) cblk[r] = cl[min(tid + kThreads * r, f.cand_k - 1)];
        for (int j = tid; j < (nbk + 31) / 32; j += kThreads) ckeep[j] = 0u;
    }

    // ------------------------------------------------------------------ phase A
    {
        IdxQuery<DI, FMT, HT> qr;
        load_idx_query<DI, FMT, HT>(qr, ia, (size_t)q, true, g, c);
        for (int base = c0 + wave * 64; base < c1; base += 4 * 64) {
            IdxKeys kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kb[u] = load_idx_keys<DI, FMT>(ia, (size_t)b * ia.T_cap + min(base + 16 * u + c, nvis - 1), g);
            const float s = idx_score4<DI, FMT, HT>(qr, kb, g);
            const int t = base + 16 * g + c;
            if (t < c1) sc[t - c0] = s;
        }
    }
    __syncthreads();
    if (f.bmax) {  // level one of a candidate source: this chunk's block maxima
        const int bs = f.bmax_bs;
        const int jb0 = c0 / bs, jpin = (nvis - 1) / bs;
        float *bq = f.bmax + (size_t)q * f.ldb;
        for (int j = tid; j * bs < n; j += kThreads) {
            float mx = -INFINITY;
            for (int t = j * bs; t < min(j * bs + bs, n); ++t) mx = fmaxf(mx, sc[t]);
            bq[jb0 + j] = jb0 + j == jpin ? INFINITY : mx;
        }
    }
    if constexpr (MASK) {
        if (select) {  // (every visible row is picked otherwise, masked or not)
#pragma unroll
            for (int r = 0; r < kFusedCandMax / kThreads; ++r) {
                const int blk = cblk[r] - blk0;
                if (tid + kThreads * r < f.cand_k && cblk[r] >= 0 && blk >= 0 && blk < nbk)
                    atomicOr(&ckeep[blk >> 5], 1u << (blk & 31));
            }
            __syncthreads();
            for (int t = tid; t < n; t += kThreads) {
                const int blk = fdiv(c0 + t, f.div_cbs) - blk0;
                if (!((ckeep[blk >> 5] >> (blk & 31)) & 1u)) sc[t] = -INFINITY;
            }
            __syncthreads();
        }
    }
    if (select) {
        // publish this chunk's scores (16-byte coherent stores; chunks start at multiples of 256)
        uint32_t kmax = 0u, kminc = 0u;  // team max key, and max of complemented keys (= min)
        for (int j = tid; 4 * j < n; j += kThreads) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = 4 * j + e < n ? sc[4 * j + e] : sc[4 * j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t k = order_key(v[e]);
                kmax = max(kmax, k);
                // masked rows (-inf) stay out of the value range; they share its lowest bin
                if (!MASK || v[e] != -INFINITY) kminc = max(kminc, ~k);
            }
            st128_agent(ts_r, (uint32_t)(c0 + 4 * j) * 4u,
                        u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                              __float_as_uint(v[3])});
        }
        kmax = wave_max_u32(kmax);
        kminc = wave_max_u32(kminc);
        if (lane == 0) {
            sm.mm[wave][0] = kmax;
            sm.mm[wave][1] = kminc;
        }
        __syncthreads();
        uint32_t a = 0u, cmin = 0u;
        for (int w = 0; w < kThreads / 64; ++w) {
            a = max(a, sm.mm[w][0]);
            cmin = max(cmin, sm.mm[w][1]);
        }
        team_flag(slot_a, m, a, cmin, (uint32_t)q, ep);  // barrier A: scores published
    }

    // attention operands that do not depend on the selection, requested once the chunk's
    // scores are published (before, their round trip would delay scoring and the flag,
    // which waits for every load in flight)
    bf16x8 qb[D / 32];
    load_q_operands<D>(qb, aa.q, (size_t)q, g, c);

    // window rows of this member, prefetched by waves 3, 2, ... (tile w -> wave 3 - w)
    const int nwin = window_width(ia.S, ia.start_pos, aa.W);
    const int my_win = m < f.win_tiles ? fdiv(f.win_tiles - 1 - m, f.div_team) + 1 : 0;
    const int win_w = 3 - wave;  // this wave's prefetched window tile, if < my_win
    // rows of a window tile; a lane off the list reads the query's own slot instead (always
    // attended), so that the loads need no branch
    const int Rr = max(aa.R, 1);
    const int own_slot = ia.start_pos + i - fdiv(ia.start_pos + i, f.div_R) * Rr;
    WindowBase wbase;  // window_base(), its ring division by the multiplier
    wbase.p0 = ia.start_pos == 0 ? max(i - aa.W + 1, 0) : ia.start_pos + i - aa.W + 1;
    wbase.s0 = wbase.p0 >= 0 ? wbase.p0 - fdiv(wbase.p0, f.div_R) * Rr : window_base(ia.start_pos, aa.W, Rr, i).s0;
    // (layer l's window source: the layers sharing this top-k each have their own)
    auto win_tile_load = [&](WinRows &rows, int j, int l) {
        const int p0 = 32 * j + c, p1 = 32 * j + 16 + c;
        const int s0 = p0 < nwin ? window_slot_at(wbase, ia.start_pos, aa.R, i, p0) : -1;
        const int s1 = p1 < nwin ? window_slot_at(wbase, ia.start_pos, aa.R, i, p1) : -1;
        const size_t r0 = (size_t)b * aa.R + (s0 >= 0 ? s0 : own_slot);
        const size_t r1 = (size_t)b * aa.R + (s1 >= 0 ? s1 : own_slot);
        if constexpr (QKV)
            kv_rows_load<D, kKvE4M3>(rows, aa.win_codes + (size_t)l * aa.win_ls,
                                     aa.win_scales + (size_t)l * aa.win_ls / 32, r0, s0 >= 0, r1, s1 >= 0, g);
        else
            attn_tile_load_rows<D>(rows, aa.win_kv + (size_t)l * aa.win_ls + r0 * D, s0 >= 0,
                                   aa.win_kv + (size_t)l * aa.win_ls + r1 * D, s1 >= 0, g);
    };
    WinRows wrows;
    if (win_w < my_win) win_tile_load(wrows, m + win_w * f.team_size, 0);

    // Attention list: positions of this chunk's rows to attend.  With a cut it holds the
    // chunk's scores in bins >= the cut's bin (sure picks and candidates, ascending); the
    // candidates that miss the cut are masked when their tile is computed.
    int *al = picks;
    int na = 0;
    // rows of listed tile tt; a lane past the list reads the first listed row instead
    auto pick_tile_load = [&](PickRows &rows, int tt) {
        const int p0 = 32 * tt + c, p1 = p0 + 16;
        const size_t rb = (size_t)b * aa.T_cap;
        const size_t r0 = rb + al[p0 < na ? p0 : 0], r1 = rb + al[p1 < na ? p1 : 0];
        if constexpr (QKV)
            kv_rows_load<D, kKvE2M1>(rows, aa.comp_codes, aa.comp_scales, r0, p0 < na, r1, p1 < na, g);
        else
            attn_tile_load_rows<D>(rows, aa.comp_kv + r0 * D, p0 < na, aa.comp_kv + r1 * D, p1 < na, g);
    };
    PickRows pre;  // this wave's first tile of listed rows, requested during selection
    bool have_pre = false;

    // ------------------------------------------------------------- phase S
    uint32_t kstar = 0u;  // a pick is key > kstar, or key == kstar with position <= pstar
    int pstar = 0x7fffffff;
    if (select) {
        // barrier A; the members' slots also carry their chunks' max / min keys
        const u32x4 sa = team_poll(slot_a, f.team_size, (uint32_t)q, ep, f.spin_limit, f.err);
        const int nquad = (nvis + 3) / 4;
        // cached form: thread t keeps the score quads t + kThreads*r (positions 4(t + kThreads*r) + e)
        constexpr bool cached = CACHED;  // the plan guarantees nquad <= kCacheQ * kThreads
        const bool full = 4 * (tid + kThreads * (kCacheQ - 1)) + 4 <= nvis;  // all 32 visible
        u32x4 vals[kCacheQ];
        if (cached) {
#pragma unroll
            for (int r = 0; r < kCacheQ; ++r) {
                const int qi = tid + kThreads * r;
                vals[r] = qi < nquad ? ld128_agent(ts_r, (uint32_t)qi * 16u) : u32x4{0u, 0u, 0u, 0u};
            }
        }
        // every visible (position, score) of the team, read from the team buffer
        // (rounds of kBatch quads per thread, all requested before any is used; a quad past
        // the team buffer reads as zeros)
        auto each = [&](auto &&fn) {
            for (int q0 = 0; q0 < nquad; q0 += kBatch * kThreads) {
                u32x4 v[kBatch];
#pragma unroll
                for (int r = 0; r < kBatch; ++r) v[r] = ld128_agent(ts_r, (uint32_t)(q0 + tid + kThreads * r) * 16u);
#pragma unroll
                for (int r = 0; r < kBatch; ++r) {
                    const int qi = q0 + tid + kThreads * r;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * qi + e < nvis) fn(4 * qi + e, __uint_as_float(v[r][e]));
                }
                // the loads are consumed under lane conditions: wait for them here, so that no
                // load of this loop is still counted as in flight where the paths join
                __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
            }
        };
        // team max / min from the members' slots
        {
            uint32_t a = tid < f.team_size ? sa[0] : 0u, cmin = tid < f.team_size ? sa[1] : 0u;
            a = wave_max_u32(a);
            cmin = wave_max_u32(cmin);
            if (lane == 0) {
                sm.mm[wave][0] = a;
                sm.mm[wave][1] = cmin;
            }
        }
        // value bins between the team's min and max: fewer for short rows (f.vbins: 256, 1024
        // or 4096), so clearing and searching them costs less
        const int nbv = f.vbins;
        for (int j = tid; j < nbv / 4 + 1; j += kThreads)  // + the spill bin
            reinterpret_cast<u32x4 *>(sm.hist)[j] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        uint32_t kmax = 0u, kminc = 0u;
        for (int w = 0; w < kThreads / 64; ++w) {
            kmax = max(kmax, sm.mm[w][0]);
            kminc = max(kminc, sm.mm[w][1]);
        }
        const float mx = key_float(kmax);
        const float mn = key_float(~kminc);
        const float scale = mx > mn ? (float)nbv / (mx - mn) : 0.f;
        const float bias = -mn * scale;
        // pass 1: value bins (kept, 16 bits each) and histogram; cached positions past the
        // visible rows take the spill bin nbv.  Masked rows (-inf, level two) fall in bin
        // 0; they are counted per thread and added once per wave, since thousands of LDS
        // atomics on one counter would serialise.
        uint32_t bins[kCacheQ * 2];
        uint32_t ninf = 0;
        auto hist_add = [&](uint32_t bin, float x) {
            if (MASK && x == -INFINITY)
                ++ninf;
            else
                atomicAdd(&sm.hist[bin], 1u);
        };
        if (cached) {
            if (full) {
#pragma unroll
                for (int r = 0; r < kCacheQ; ++r) {
                    *reinterpret_cast<u32x4 *>(tsl + 4 * (tid + kThreads * r)) = vals[r];
                    uint32_t bb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bb[e] = (uint32_t)value_bin_n(__uint_as_float(vals[r][e]), scale, bias, nbv);
                        hist_add(bb[e], __uint_as_float(vals[r][e]));
                    }
                    bins[2 * r] = bb[0] | (bb[1] << 16);
                    bins[2 * r + 1] = bb[2] | (bb[3] << 16);
                }
            } else {
                const uint32_t spill2 = (uint32_t)nbv * 0x10001u;  // two spill bins
#pragma unroll
                for (int r = 0; r < kCacheQ; ++r) {
                    bins[2 * r] = spill2;
                    bins[2 * r + 1] = spill2;
                    if (kThreads * r >= nquad) continue;  // (uniform) no thread holds a visible quad
                    if (tid + kThreads * r < nquad)
                        *reinterpret_cast<u32x4 *>(tsl + 4 * (tid + kThreads * r)) = vals[r];
                    uint32_t bb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bb[e] = 4 * (tid + kThreads * r) + e < nvis
                                    ? (uint32_t)value_bin_n(__uint_as_float(vals[r][e]), scale, bias, nbv)
                                    : (uint32_t)nbv;
                        // positions past the visible rows add nothing: thousands of them
                        // counted into the one spill bin would serialise on its atomics
                        if (bb[e] != (uint32_t)nbv) hist_add(bb[e], __uint_as_float(vals[r][e]));
                    }
                    bins[2 * r] = bb[0] | (bb[1] << 16);
                    bins[2 * r + 1] = bb[2] | (bb[3] << 16);
                }
            }
        } else {
            // the value bins of every team position are kept in LDS when they fit
            uint16_t *bins16 = reinterpret_cast<uint16_t *>(dyn + 2 * f.chunk);
            const bool keep = f.lds_bins;
            each([&](int t, float x) {
                const int bin = value_bin_n(x, scale, bias, nbv);
                hist_add((uint32_t)bin, x);
                if (keep) bins16[t] = (uint16_t)bin;
            });
        }
        if constexpr (MASK) {
            ninf = wave_sum_u32(ninf);
            if (lane == 0 && ninf) atomicAdd(&sm.hist[0], ninf);
        }
        __syncthreads();
        find_bin(sm.hist, nbv, f.keff, sm.wsum, &sm.bin, &sm.above);
        const int vb = sm.bin;
        const int need = f.keff - sm.above;
        const int cnt = (int)sm.hist[vb];
        // the attention list, in position order (wave counts summed in wave order)
        for (int j = 0; j * kThreads < n; ++j) {
            const int t = tid + kThreads * j;
            const bool in = t < n && value_bin_n(sc[t], scale, bias, nbv) >= vb;
            const uint64_t bal = __ballot(in);
            if (lane == 0) sm.wcnt[wave] = (int)__popcll(bal);
            __syncthreads();
            int base = na, tot = 0;
#pragma unroll
            for (int w = 0; w < kThreads / 64; ++w) {
                base += w < wave ? sm.wcnt[w] : 0;
                tot += sm.wcnt[w];
            }
            if (in) al[base + (int)__popcll(bal & ((1ull << lane) - 1ull))] = c0 + t;
            na += tot;
            __syncthreads();
        }
        // each wave's first tile of listed rows is requested now, so that the gather
        // overlaps the rest of the selection (waves holding window rows take theirs later);
        // the re-reading form requests it after its candidate loads, which would otherwise
        // wait behind the gather (the loads of a wave complete in order)
        auto early_gather = [&]() {
            if (win_w >= my_win && 32 * wave < na) {
                pick_tile_load(pre, wave);
                have_pre = true;
            }
            asm volatile("" ::: "memory");  // issue those loads here, not where they are used
        };
        if (cached) early_gather();
        // candidates as (key << 32 | ~position): larger means ahead in (key desc, position asc);
        // they take the histogram's place, which is no longer read
        uint64_t *cand = reinterpret_cast<uint64_t *>(sm.hist);
        if (tid == 0) {
            sm.kstar = 0u;
            sm.pstar = 0x7fffffff;
            sm.ncand = 0;
        }
        __syncthreads();
        if (cnt <= kCandCap) {
            // pass 2: the candidates (bin vb) into LDS.  Cached: two 16-bit bins per word;
            // adding 0x7fff - vb (0x8000 - vb) to a half sets its bit 15 exactly when the bin is
            // above (at least) vb, and bins stay <= nbv <= 4096, so no half carries into the next.
            if (cached) {
                const uint32_t kgt = (0x7fffu - (uint32_t)vb) * 0x10001u;
                const uint32_t kge = (0x8000u - (uint32_t)vb) * 0x10001u;
                uint32_t cmask = 0;  // bit 4r + e: element e of quad r is a candidate
#pragma unroll
                for (int r = 0; r < kCacheQ; ++r) {
                    const uint32_t a0 = bins[2 * r] + kgt, a1 = bins[2 * r + 1] + kgt;
                    const uint32_t b0 = bins[2 * r] + kge, b1 = bins[2 * r + 1] + kge;
                    const uint32_t e0 = (a0 ^ b0) & 0x80008000u, e1 = (a1 ^ b1) & 0x80008000u;
                    cmask |= ((e0 >> 15) & 1u | (e0 >> 30) & 2u | (e1 >> 13) & 4u | (e1 >> 28) & 8u) << (4 * r);
                }
                if (cmask) {  // few lanes: their candidates' scores are read back from LDS
                    int ci = atomicAdd(&sm.ncand, __builtin_popcount(cmask));
                    do {
                        const int bit = __builtin_ctz(cmask);
                        cmask &= cmask - 1u;
                        const int t = 4 * (tid + kThreads * (bit >> 2)) + (bit & 3);
                        cand[ci++] = ((uint64_t)order_key(tsl[t]) << 32) | (uint32_t)~(uint32_t)t;
                    } while (cmask);
                }
            } else {
                if (f.lds_bins) {
                    // candidate positions from the LDS bins (8 per 16-byte read), then their
                    // scores from the team buffer, one load per candidate, all in flight together
                    const uint16_t *bins16 = reinterpret_cast<const uint16_t *>(dyn + 2 * f.chunk);
                    int *cpos = reinterpret_cast<int *>(dyn + 2 * f.chunk) + f.bins_words;
                    for (int w8 = tid; 8 * w8 < nvis; w8 += kThreads) {
                        const u32x4 x = *reinterpret_cast<const u32x4 *>(bins16 + 8 * w8);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const int t = 8 * w8 + e;
                            const uint32_t bin = (x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                            if (t < nvis && bin == (uint32_t)vb) cpos[atomicAdd(&sm.ncand, 1)] = t;
                        }
                    }
                    __syncthreads();
                    for (int j = tid; j < cnt; j += kThreads) {
                        const int t = cpos[j];
                        cand[j] = ((uint64_t)order_key(ldf_agent(ts + t)) << 32) | (uint32_t)~(uint32_t)t;
                    }
                    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): nothing left in flight
                } else {
                    each([&](int t, float x) {
                        const int bin = value_bin_n(x, scale, bias, nbv);
                        if (bin == vb) cand[atomicAdd(&sm.ncand, 1)] = ((uint64_t)order_key(x) << 32) | (uint32_t)~(uint32_t)t;
                    });
                }
            }
            if (!cached) early_gather();
            __syncthreads();
            int ncand = cnt, nneed = need;
            refine_candidates(cand, ncand, nneed, reinterpret_cast<uint32_t *>(attn_lds), sm);
            rank_candidates(cand, ncand, nneed, sm);
            kstar = sm.kstar;
            pstar = sm.pstar;
        } else {
            radix_resolve(sm, [&](int t) { return ldf_agent(ts + t); }, nvis, scale, bias, vb, need, nbv);
            kstar = sm.kstar;
            pstar = sm.pstar;
        }
    }

    // ------------------------------------------------------------------ phase D
    int32_t *idx_row = f.topk_out + (size_t)q * f.keff;
    // a pick: every visible row without a cut, else key > kstar or key == kstar at a
    // position <= pstar
    auto picked = [&](int t) {
        const uint32_t k = order_key(sc[t]);
        return !select || k > kstar || (k == kstar && c0 + t <= pstar);
    };
    if (!select) {
        for (int p = tid; p < n; p += kThreads) al[p] = c0 + p;
        na = n;
        __syncthreads();
    }
    // partial states: one slot per (member, layer), member-major
    const int NL = LAYERS ? aa.L : 1;
    const int slot_bytes = f.slot_floats * 4;
    const rsrc_t part_r = make_rsrc(f.part + (size_t)q * f.team_size * NL * f.slot_floats,
                                    (uint32_t)(f.team_size * NL * slot_bytes));
    // Layer 0 (this step's own layer) attends here, with the rows requested during the
    // selection; further layers that share the top-k (their own queries, window rows and
    // sink, the same picked rows) follow in a block of their own below, so that the
    // one-layer step keeps this code as it is.
    {
        const float sl2 = aa.scale * kLog2e;
        uint16_t *tile = attn_lds + wave * 32 * LD;
        const int pick_tiles = (na + 31) / 32;
        auto is_pick = [&](int p) {
            if (p >= na) return false;
            if (!select) return true;
            const int pos = al[p];
            const uint32_t k = order_key(sc[pos - c0]);
            return k > kstar || (k == kstar && pos <= pstar);
        };
        AttnState<D> st;
        attn_init<D>(st);
        uint32_t npk = 0;  // picks among this wave's tiles
        // rows as the MFMA operands (quantised rows are dequantised here)
        auto as_rows = [&](const auto &raw, AttnRows<D> &rows) {
            if constexpr (QKV) {
                using Raw = std::decay_t<decltype(raw)>;
                if constexpr (std::is_same_v<Raw, KvRows<D, kKvE4M3>>)
                    kv_rows_convert<D, kKvE4M3>(raw, rows);
                else
                    kv_rows_convert<D, kKvE2M1>(raw, rows);
            } else {
                rows = raw;
            }
        };
        if (win_w < my_win) {
            AttnRows<D> rows;
            as_rows(wrows, rows);
            attn_tile_compute<D>(st, qb, rows, tile, aa.dv / 16, sl2, g, c);
        }
        // window tiles beyond the prefetched ones (more than 4 per member)
        for (int w = 4 + wave; w < my_win; w += 4) {
            WinRows raw;
            win_tile_load(raw, m + w * f.team_size, 0);
            AttnRows<D> rows;
            as_rows(raw, rows);
            attn_tile_compute<D>(st, qb, rows, tile, aa.dv / 16, sl2, g, c);
        }
        for (int tt = wave; tt < pick_tiles; tt += 4) {
            const int p0 = 32 * tt + c, p1 = 32 * tt + 16 + c;
            AttnRows<D> rows;
            if (tt == wave && have_pre) {
                as_rows(pre, rows);
            } else {
                PickRows raw;
                pick_tile_load(raw, tt);
                as_rows(raw, rows);
            }
            rows.valid[0] = __ballot(is_pick(p0));
            rows.valid[1] = __ballot(is_pick(p1));
            npk += __popcll(rows.valid[0] & 0xFFFFull) + __popcll(rows.valid[1] & 0xFFFFull);  // rows c of lanes c
            attn_tile_compute<D>(st, qb, rows, tile, aa.dv / 16, sl2, g, c);
        }
        if (lane == 0) sm.wpick[wave] = npk;
        __syncthreads();
        float *ow = reinterpret_cast<float *>(attn_lds);
        attn_wave_publish<D>(st, ow, wm, wl, wave, aa.dv, g, c);
        __syncthreads();
        // per-head factors of the 4 waves, once
        if (tid < kHeads) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w * kHeads + tid]);
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float mw = wm[w * kHeads + tid];
                const float fw = (mw == -INFINITY || M == -INFINITY) ? 0.f : exp2f(mw - M);
                hf[w * kHeads + tid] = fw;
                L += fw * wl[w * kHeads + tid];
            }
            hm[tid] = M;
            hl[tid] = L;
        }
        __syncthreads();
        // this member's state: O [16][dv] then (M, L) [16], 16-byte coherent stores
        const int qdv = aa.dv / 4;
        const uint32_t my_off = (uint32_t)(m * NL * slot_bytes);
        for (int e = tid; e < kHeads * qdv; e += kThreads) {
            const int h = fdiv(e, f.div_qdv);
            const int d = 4 * (e - h * qdv);
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&ow[(w * kHeads + h) * attn_ow_ld(aa.dv) + d]);
                O += hf[w * kHeads + h] * x;
            }
            st128_agent(part_r, my_off + (uint32_t)(h * aa.dv + d) * 4u, __builtin_bit_cast(u32x4, O));
        }
        if (tid < kHeads / 2) {
            const int h = 2 * tid;
            st128_agent(part_r, my_off + (uint32_t)(kHeads * aa.dv + 2 * h) * 4u,
                        u32x4{__float_as_uint(hm[h]), __float_as_uint(hl[h]), __float_as_uint(hm[h + 1]),
                              __float_as_uint(hl[h + 1])});
        }
    }
    // the further layers (each: its own queries and window rows, the shared picked rows back
    // from the cache), the same pass without the prefetched rows or the pick count
    for (int l = 1; l < NL; ++l) {
        __syncthreads();  // the previous layer's wave states in LDS have been read
        bf16x8 ql[D / 32];
        load_q_operands<D>(ql, aa.q + (size_t)l * aa.q_ls, (size_t)q, g, c);
        const float sl2 = aa.scale * kLog2e;
        uint16_t *tile = attn_lds + wave * 32 * LD;
        AttnState<D> st;
        attn_init<D>(st);
        auto compute = [&](const auto &raw, uint64_t v0, uint64_t v1, bool mask) {
            AttnRows<D> rows;
            if constexpr (QKV) {
                using Raw = std::decay_t<decltype(raw)>;
                if constexpr (std::is_same_v<Raw, KvRows<D, kKvE4M3>>)
                    kv_rows_convert<D, kKvE4M3>(raw, rows);
                else
                    kv_rows_convert<D, kKvE2M1>(raw, rows);
            } else {
                rows = raw;
            }
            if (mask) {
                rows.valid[0] = v0;
                rows.valid[1] = v1;
            }
            attn_tile_compute<D>(st, ql, rows, tile, aa.dv / 16, sl2, g, c);
        };
        for (int w = wave; w < my_win; w += 4) {
            WinRows raw;
            win_tile_load(raw, m + w * f.team_size, l);
            compute(raw, 0, 0, false);
        }
        for (int tt = wave; tt < (na + 31) / 32; tt += 4) {
            const int p0 = 32 * tt + c, p1 = 32 * tt + 16 + c;
            auto is_pick = [&](int p) {
                if (p >= na) return false;
                if (!select) return true;
                const int pos = al[p];
                const uint32_t k = order_key(sc[pos - c0]);
                return k > kstar || (k == kstar && pos <= pstar);
            };
            PickRows raw;
            pick_tile_load(raw, tt);
            compute(raw, __ballot(is_pick(p0)), __ballot(is_pick(p1)), true);
        }
        float *ow = reinterpret_cast<float *>(attn_lds);
        __syncthreads();
        attn_wave_publish<D>(st, ow, wm, wl, wave, aa.dv, g, c);
        __syncthreads();
        if (tid < kHeads) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w * kHeads + tid]);
            float L = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float mw = wm[w * kHeads + tid];
                const float fw = (mw == -INFINITY || M == -INFINITY) ? 0.f : exp2f(mw - M);
                hf[w * kHeads + tid] = fw;
                L += fw * wl[w * kHeads + tid];
            }
            hm[tid] = M;
            hl[tid] = L;
        }
        __syncthreads();
        const int qdv = aa.dv / 4;
        const uint32_t my_off = (uint32_t)((m * NL + l) * slot_bytes);
        for (int e = tid; e < kHeads * qdv; e += kThreads) {
            const int h = fdiv(e, f.div_qdv);
            const int d = 4 * (e - h * qdv);
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const f32x4 x = *reinterpret_cast<const f32x4 *>(&ow[(w * kHeads + h) * attn_ow_ld(aa.dv) + d]);
                O += hf[w * kHeads + h] * x;
            }
            st128_agent(part_r, my_off + (uint32_t)(h * aa.dv + d) * 4u, __builtin_bit_cast(u32x4, O));
        }
        if (tid < kHeads / 2) {
            const int h = 2 * tid;
            st128_agent(part_r, my_off + (uint32_t)(kHeads * aa.dv + 2 * h) * 4u,
                        u32x4{__float_as_uint(hm[h]), __float_as_uint(hl[h]), __float_as_uint(hm[h + 1]),
                              __float_as_uint(hl[h + 1])});
        }
    }
    // The member's merge slice (phase M): `items` (layer, head, dim quad) outputs, each summed
    // by lpi lanes, so waves [0, merge_waves) have merge work.
    const int qdv_m = aa.dv / 4;
    const int n_out_m = NL * kHeads * qdv_m;
    const int per_m = f.merge_per;  // ceil(n_out_m / team_size)
    const int items = max(0, min(m * per_m + per_m, n_out_m) - m * per_m);
    int lpi = 1;
    while (lpi * 2 * items <= kThreads && lpi < 16) lpi *= 2;
    const int merge_waves = (min(items * lpi, kThreads) + 63) / 64;
    // The member's picks go to the top-k list after barrier C, whose pick counts give their
    // offset.  The last wave writes them when it has no merge work; when every wave merges,
    // the writing is split into four contiguous ranges of the chunk's positions, one per
    // wave after its merge work, and each range's pick count is taken here, while the
    // partial-state stores complete.
    const int nlw = merge_waves < kThreads / 64 ? 1 : kThreads / 64;  // list waves
    const int lw0 = kThreads / 64 - nlw;                               // the first of them
    const int lq = nlw == 1 ? (n + 63) & ~63 : ((n + 255) >> 8) << 6;  // positions per range
    auto in_range = [&](int r, int p) { return p < n && p < (r + 1) * lq; };
    if (nlw > 1) {
        uint32_t cnt = 0;
        for (int p0 = wave * lq; p0 < min(n, (wave + 1) * lq); p0 += 64)
            cnt += (uint32_t)__popcll(__ballot(in_range(wave, p0 + lane) && picked(p0 + lane)));
        if (lane == 0) sm.wcnt[wave] = (int)cnt;
    }
    // barrier C: partial state published; the flag carries the member's pick count
    team_flag(slot_c, m, sm.wpick[0] + sm.wpick[1] + sm.wpick[2] + sm.wpick[3], 0u, (uint32_t)q, ep);
    team_poll(slot_c, f.team_size, (uint32_t)q, ep, f.spin_limit, f.err, sm.cnt);
    // every member has read the launch count (it passed barrier C): advance it
    if (m == 0 && tid == 0) st_agent(epoch, ep);

    // ------------------------------------------------------------------ phase M
    {
        // This member's slice of the (head, dim-quad) outputs.  Each output quad is summed
        // by a group of lpi <= 16 lanes (a power of two): every lane loads the O quad and
        // the (max, normaliser) pair of a stride of the slots, all in one round trip, and
        // the group combines its lanes with DPP exchanges.
        const int qdv = qdv_m;
        const int e0 = m * per_m;  // (layer, head, dim quad) outputs items from e0
        const int ls = __builtin_ctz((unsigned)lpi);  // lpi = 2^ls
        // rounds of kThreads / lpi items (one round unless lpi == 1 and items > kThreads)
        for (int i0 = 0; i0 < items; i0 += kThreads >> ls) {
            if (i0 + ((wave * 64) >> ls) >= items) continue;  // no item for this wave in this round
            const int item = i0 + (tid >> ls), sub = tid & (lpi - 1);
            const bool act = item < items;
            const int e = e0 + (act ? item : 0);
            const int ly = fdiv(e, f.div_hq);
            const int eh = e - ly * kHeads * qdv;
            const int h = fdiv(eh, f.div_qdv);
            const int d = 4 * (eh - h * qdv);
            const float *mlp = f.part + ((size_t)q * f.team_size * NL + ly) * f.slot_floats + kHeads * aa.dv + 2 * h;
            constexpr int kU = 8;
            f32x4 O = {0.f, 0.f, 0.f, 0.f};
            float M = -INFINITY, L = 0.f;
            for (int s0 = sub; s0 < f.team_size; s0 += kU * lpi) {
                u32x4 o[kU];
                uint64_t ml[kU];
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const int sl = s0 + u * lpi;
                    const bool ok = act && sl < f.team_size;
                    o[u] = ok ? ld128_agent(part_r, (uint32_t)((sl * NL + ly) * slot_bytes + (h * aa.dv + d) * 4))
                              : u32x4{0u, 0u, 0u, 0u};
                    ml[u] = ok ? ld64_agent(reinterpret_cast<const uint64_t *>(mlp + (size_t)sl * NL * f.slot_floats))
                               : pack2(-INFINITY, 0.f);
                }
                float Mn = M;
#pragma unroll
                for (int u = 0; u < kU; ++u) Mn = fmaxf(Mn, lo_f(ml[u]));
                const float a = M == -INFINITY ? 0.f : exp2f(M - Mn);
                O *= a;
                L *= a;
#pragma unroll
                for (int u = 0; u < kU; ++u) {
                    const float ms = lo_f(ml[u]);
                    const float w = ms == -INFINITY ? 0.f : exp2f(ms - Mn);
                    O += w * __builtin_bit_cast(f32x4, o[u]);
                    L += w * hi_f(ml[u]);
                }
                M = Mn;
            }
            // combine the group's lanes: partner lane^x for x = 8, 4, 2, 1 below lpi
            auto level = [&](auto xchg) {
                const float M2 = xchg(M), L2 = xchg(L);
                f32x4 O2;
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) O2[e4] = xchg(O[e4]);
                const float Mn = fmaxf(M, M2);
                const float a = M == -INFINITY ? 0.f : exp2f(M - Mn);
                const float bb = M2 == -INFINITY ? 0.f : exp2f(M2 - Mn);
                O = a * O + bb * O2;
                L = a * L + bb * L2;
                M = Mn;
            };
            if (lpi > 8) level([](float v) { return dpp_f<0x128>(v); });  // row_ror:8 = lane ^ 8
            if (lpi > 4) level([&](float v) {                                // lane ^ 4
                const float up = dpp_f<0x104>(v), dn = dpp_f<0x114>(v);       // row_shl:4, row_shr:4
                return (lane & 4) ? dn : up;
            });
            if (lpi > 2) level([](float v) { return dpp_f<0x4E>(v); });   // quad_perm [2,3,0,1]
            if (lpi > 1) level([](float v) { return dpp_f<0xB1>(v); });   // quad_perm [1,0,3,2]
            if (act && sub == 0) {
                uint16_t *dst = aa.out + (size_t)ly * aa.out_ls + ((size_t)q * kHeads + h) * aa.dv + d;
                *reinterpret_cast<u32x2 *>(dst) = attn_finish4(O, M, L, aa.sink ? aa.sink + ly * kHeads : nullptr, h);
            }
        }
    }
    // The member's picks into the top-k list, ascending, by the list waves (after their merge
    // work, if any): range r starts after the picks of the members before this one (their
    // counts came with barrier C) and of this member's earlier ranges.
    if (wave >= lw0) {
        const int r = wave - lw0;
        uint32_t pre = 0;
        for (int j = lane; j < m; j += 64) pre += sm.cnt[j];
        pre = wave_sum_u32(pre);
        for (int rr = 0; rr < r; ++rr) pre += (uint32_t)sm.wcnt[rr];
        // lane l takes lq / 64 consecutive positions of the range (their score reads all
        // issued together), the wave scan orders the lanes
        const int per = lq / 64;
        const int t0 = r * lq + lane * per, t1 = min(t0 + per, min(n, (r + 1) * lq));
        uint32_t mine = 0;
        for (int t = t0; t < t1; ++t) mine += picked(t) ? 1u : 0u;
        int o = (int)pre + (int)(wave_scan(mine) - mine);
        for (int t = t0; t < t1; ++t)
            if (picked(t)) {
                if (o < f.keff) idx_row[o] = c0 + t;
                ++o;
            }
        if (m == 0 && !select && r == nlw - 1)
            for (int j = nvis + lane; j < f.keff; j += 64) idx_row[j] = -1;
    }
}
}  // namespace

// The kernels of one index-code format (and level-two masking or not): launch, and
// co-resident workgroups per CU.
template <int FMT, bool MASK, bool QKV = false, bool LAYERS = false>
struct FusedKernels {
    template <int D, int DI, int HT>
    static hipError_t cfg(const FusedArgs &f, int grid, size_t dyn_bytes, hipStream_t stream) {
        if (f.cache_lds)
            hipLaunchKernelGGL((fused_decode_kernel<D, DI, FMT, HT, true, MASK, QKV, LAYERS>), dim3(grid),
                               dim3(kThreads), dyn_bytes, stream, f);
        else
            hipLaunchKernelGGL((fused_decode_kernel<D, DI, FMT, HT, false, MASK, QKV, LAYERS>), dim3(grid),
                               dim3(kThreads), dyn_bytes, stream, f);
        return hipGetLastError();
    }
    template <int D, int DI>
    static hipError_t di(const FusedArgs &f, int grid, size_t dyn, hipStream_t s) {
        switch (f.ia.Hi / 16) {
            case 1: return cfg<D, DI, 1>(f, grid, dyn, s);
            case 2: return cfg<D, DI, 2>(f, grid, dyn, s);
            case 3: return cfg<D, DI, 3>(f, grid, dyn, s);
            case 4: return cfg<D, DI, 4>(f, grid, dyn, s);
            default: return hipErrorInvalidValue;
        }
    }
    template <int D>
    static hipError_t d(const FusedArgs &f, int grid, size_t dyn, hipStream_t s) {
        return f.ia.Di == 64 ? di<D, 64>(f, grid, dyn, s) : di<D, 128>(f, grid, dyn, s);
    }
    static hipError_t launch(const FusedArgs &f, int grid, size_t dyn, hipStream_t s) {
        switch (f.aa.D) {
            case 64: return d<64>(f, grid, dyn, s);
            case 128: return d<128>(f, grid, dyn, s);
            case 192: return d<192>(f, grid, dyn, s);
            case 256: return d<256>(f, grid, dyn, s);
            default: return hipErrorInvalidValue;
        }
    }
    template <int D, int DI, int HT>
    static hipError_t occ(int *per_cu, size_t dyn, bool cached) {
        return cached ? hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            per_cu, fused_decode_kernel<D, DI, FMT, HT, true, MASK, QKV, LAYERS>, kThreads, dyn)
                      : hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            per_cu, fused_decode_kernel<D, DI, FMT, HT, false, MASK, QKV, LAYERS>, kThreads, dyn);
    }
    template <int D, int DI>
    static hipError_t occ_di(int HT, int *per_cu, size_t dyn, bool cached) {
        switch (HT) {
            case 1: return occ<D, DI, 1>(per_cu, dyn, cached);
            case 2: return occ<D, DI, 2>(per_cu, dyn, cached);
            case 3: return occ<D, DI, 3>(per_cu, dyn, cached);
            case 4: return occ<D, DI, 4>(per_cu, dyn, cached);
            default: return hipErrorInvalidValue;
        }
    }
    template <int D>
    static hipError_t occ_d(int DI, int HT, int *per_cu, size_t dyn, bool cached) {
        return DI == 64 ? occ_di<D, 64>(HT, per_cu, dyn, cached) : occ_di<D, 128>(HT, per_cu, dyn, cached);
    }
    // Workgroups of the kernel for (D, DI, HT, cached) that fit one CU with `dyn`
    // bytes of dynamic LDS (0 when the shape is not instantiated or the query fails).
    static int per_cu(int D, int DI, int HT, size_t dyn, bool cached) {
        int n = 0;
        hipError_t e = hipErrorInvalidValue;
        if (DI == 64 || DI == 128) {
            switch (D) {
                case 64: e = occ_d<64>(DI, HT, &n, dyn, cached); break;
                case 128: e = occ_d<128>(DI, HT, &n, dyn, cached); break;
                case 192: e = occ_d<192>(DI, HT, &n, dyn, cached); break;
                case 256: e = occ_d<256>(DI, HT, &n, dyn, cached); break;
                default: break;
            }
        }
        return e == hipSuccess ? n : 0;
    }
};

}  // namespace lit
