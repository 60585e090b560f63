// fused_decode.hip -- the whole sparse-attention step for decode-sized batches in one
// launch: indexer scores -> exact top-k -> gather attention -> merge.
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
//   A. Every member scores its chunk (MX-scaled fp8 MFMA, as in indexer.hip) and, when
//      the query sees more rows than it keeps, adds a 4096-bin histogram of the top 12
//      bits of the scores' order keys to the team histogram.
//   -- team barrier A --
//   B. Every member reads the team histogram and finds the bin b1 where the count from
//      the top reaches k.  It publishes how many of its scores lie above b1 and its
//      scores inside b1 (the candidates, in position order).
//   -- team barrier B --
//   S. Every member reads all candidates and finds, on its own, the exact k-th
//      (key, position): a 4096-bin histogram of the next 12 key bits, then ranks among
//      the few left (or, for heavy ties, the last 8 bits and a position scan).  From
//      the published counts it also knows where its picks start in the output list.
//   D. Every member writes its picks (ascending) to the top-k list, gathers those rows
//      and its share of the window rows, and runs the attention tiles (as in
//      attention.hip) into its partial state.
//   -- team barrier C --
//   M. Members merge the team's partial states (log-sum-exp) for a slice of the
//      (head, dim) outputs, add the sink, and write bf16.  The last member to finish
//      zeroes the team's control words.
// When the query keeps every visible row, barriers A and B and the histogram are
// skipped.
//
// Cross-workgroup data (histogram, candidates, counts, partial states, counters) moves
// through agent-scope atomic stores and loads, which are performed at the device's
// coherence point; a workgroup waits for its own stores to complete (vmcnt) before it
// bumps a barrier counter.  No agent-scope fence is used: on this device such a fence
// writes back or invalidates a whole XCD's L2.
//
// Every wait is a bounded spin: if a team does not assemble in time (workgroups not
// co-resident, e.g. another kernel holding CUs), the waiter sets the sticky error word
// and goes on, so the kernel always finishes; results are then undefined and the
// error word reports it.
#include <atomic>

#include "tile_ops.h"

namespace lit {

namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 16;
constexpr int kBins = 4096;
constexpr int kCandCap = 2048;  // candidates held in LDS (more are re-read from memory)

enum : int { kBarA = 0, kBarB = 1, kBarC = 2, kDone = 3, kCtrlWords = 8 };

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

// Arrive at a team barrier once this workgroup's stores are complete.
__device__ inline void team_arrive(uint32_t *ctr) {
    stores_done();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until the counter reaches `target` (bounded).
__device__ inline void team_wait(uint32_t *ctr, uint32_t target, uint32_t limit, uint32_t *err) {
    if (threadIdx.x == 0) {
        uint32_t n = 0;
        while (ld_agent(ctr) < target) {
            if (++n > limit) {
                __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
    }
    __syncthreads();
}

// Bin search from the top over `nbins` LDS counters (nbins a multiple of 256): the bin
// where the count from the top reaches `need`, and the count strictly above it.
__device__ inline void find_bin(const uint32_t *hist, int nbins, int need, uint32_t *wsum, int *out_bin,
                                int *out_above) {
    if (threadIdx.x == 0) {
        *out_bin = 0;
        *out_above = 0;
    }
    const int per = nbins / kThreads;
    const int hi = nbins - 1 - threadIdx.x * per;  // this thread's bins: hi, hi-1, ..., hi-per+1
    uint32_t mine = 0;
    for (int j = 0; j < per; ++j) mine += hist[hi - j];
    uint32_t total;
    const uint32_t incl = wg_scan(mine, wsum, &total);
    int above = (int)(incl - mine);
    if (above < need && need <= (int)incl) {
        for (int j = 0; j < per; ++j) {
            const int c = (int)hist[hi - j];
            if (above + c >= need) {
                *out_bin = hi - j;
                *out_above = above;
                break;
            }
            above += c;
        }
    }
    __syncthreads();
}

struct FusedLds {
    uint32_t hist[kBins];
    uint32_t wsum[kThreads / 64];
    float fred[kThreads / 64];
    int bin, above, ncand, npick, overflow;
    uint32_t kstar;
    int pstar;
};

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

// Workgroup max / min / sum (every thread gets the result).
__device__ inline float wg_max(float v, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
}
__device__ inline float wg_min(float v, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fminf(v, __shfl_xor(v, off));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int w = 1; w < kThreads / 64; ++w) r = fminf(r, red[w]);
    __syncthreads();
    return r;
}
__device__ inline uint32_t wg_sum(uint32_t v, uint32_t *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r += red[w];
    __syncthreads();
    return r;
}

// Linear value bin between the team's min and max: monotonic in the value, so every
// score in a higher bin is larger than every score in a lower one.
__device__ inline int value_bin(float v, float mn, float scale) {
    const float fb = fminf(fmaxf((v - mn) * scale, 0.f), (float)(kBins - 1));
    return (int)fb;
}

// Exact resolution by radix levels over the team's scores (heavy ties): among the
// scores in value bin vb, the need-th by (order key desc, position asc).  Threads take
// contiguous position ranges so the final tie cut can walk positions in order.
__device__ inline void radix_resolve(FusedLds &sm, const float *ts, int nvis, float mn, float scale, int vb,
                                     int need) {
    const int per = (nvis + kThreads - 1) / kThreads;
    const int t0 = threadIdx.x * per, t1 = min(t0 + per, nvis);
    auto in_bin = [&](float v) { return value_bin(v, mn, scale) == vb; };
    uint32_t prefix = 0u, pmask = 0u;
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int lv = 0; lv < 3; ++lv) {
        const int nb = 1 << widths[lv];
        for (int j = threadIdx.x; j < kBins; j += kThreads) sm.hist[j] = 0u;
        __syncthreads();
        for (int t = t0; t < t1; ++t) {
            const float v = ldf_agent(ts + t);
            const uint32_t k = order_key(v);
            if (in_bin(v) && (k & pmask) == prefix) atomicAdd(&sm.hist[(k >> shifts[lv]) & (nb - 1)], 1u);
        }
        __syncthreads();
        find_bin(sm.hist, nb < kThreads ? kThreads : nb, need, sm.wsum, &sm.bin, &sm.above);
        prefix |= (uint32_t)sm.bin << shifts[lv];
        pmask |= (uint32_t)(nb - 1) << shifts[lv];
        need -= sm.above;
        __syncthreads();
    }
    // equal keys: the need-th in position order
    uint32_t eq = 0;
    for (int t = t0; t < t1; ++t) {
        const float v = ldf_agent(ts + t);
        eq += in_bin(v) && order_key(v) == prefix;
    }
    uint32_t total;
    const uint32_t incl = wg_scan(eq, sm.wsum, &total);
    int before = (int)(incl - eq);
    if (before < need && need <= (int)incl) {
        for (int t = t0; t < t1; ++t) {
            const float v = ldf_agent(ts + t);
            if (in_bin(v) && order_key(v) == prefix && ++before == need) {
                sm.pstar = t;
                break;
            }
        }
    }
    if (threadIdx.x == 0) sm.kstar = prefix;
    __syncthreads();
}

template <int D, int DI, int HT>
__global__ __launch_bounds__(kThreads) void fused_decode_kernel(FusedArgs f) {
    constexpr int LD = D + 4;
    constexpr int kCache = 16;  // score pairs per thread kept in registers during selection
    __shared__ FusedLds sm;
    __shared__ __attribute__((aligned(16))) uint16_t attn_lds[4 * 32 * LD];  // rows / candidates / merge
    __shared__ float wm[4 * kHeads], wl[4 * kHeads];
    extern __shared__ float dyn[];  // chunk scores [chunk], then picks [chunk] (ints)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;

    // team / member of this workgroup (XCD-major order when the grid allows it)
    const int G = gridDim.x;
    const int lin = (G % 8 == 0) ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
    const int q = lin / f.team_size;
    const int m = lin % f.team_size;
    const IndexerArgs &ia = f.ia;
    const AttnArgs &aa = f.aa;
    const int b = q / ia.S;
    const int i = q % ia.S;
    const int nvis = min(ia.T, (ia.start_pos + i + 1) / ia.ratio);
    const bool select = nvis > f.keff;  // otherwise every visible row is picked
    const int c0 = m * f.chunk;
    const int c1 = min(c0 + f.chunk, nvis);
    const int n = max(0, c1 - c0);
    uint32_t *ctrl = f.ctrl + (size_t)q * kCtrlWords;
    float *ts = f.scores + (size_t)q * f.ld;  // the team's scores
    float *sc = dyn;
    int *picks = reinterpret_cast<int *>(dyn + f.chunk);

    // attention operands that do not depend on the selection: issued first
    bf16x8 qb[D / 32];
    load_q_operands<D>(qb, aa.q, (size_t)q, g, c);

    // ------------------------------------------------------------------ phase A
    {
        IdxQuery<DI, HT> qr;
        load_idx_query<DI, HT>(qr, ia, (size_t)q, true, g, c);
        for (int base = c0 + wave * 64; base < c1; base += 4 * 64) {
            IdxKeys kb[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                kb[u] = load_idx_keys<DI>(ia, (size_t)b * ia.T_cap + min(base + 16 * u + c, nvis - 1), g);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float s = idx_tile_score<DI, HT>(qr, kb[u]);
                const int t = base + 16 * u + c;
                if (g == 0 && t < c1) sc[t - c0] = s;
            }
        }
    }
    __syncthreads();
    if (select) {  // publish this chunk's scores (pairs; chunks start at even positions)
        uint64_t *dst = reinterpret_cast<uint64_t *>(ts + c0);
        for (int j = 2 * tid; j < n; j += 2 * kThreads)
            st64_agent(dst + j / 2, pack2(sc[j], j + 1 < n ? sc[j + 1] : 0.f));
        team_arrive(&ctrl[kBarA]);
    }

    // window rows of this member, prefetched by waves 3, 2, ... (tile w -> wave 3 - w)
    const int nwin = window_width(ia.S, ia.start_pos, aa.W);
    const int my_win = m < f.win_tiles ? (f.win_tiles - 1 - m) / f.team_size + 1 : 0;
    const int win_w = 3 - wave;  // this wave's prefetched window tile, if < my_win
    AttnRows<D> wrows;
    if (win_w < my_win) {
        const int j = m + win_w * f.team_size;
        const int p0 = 32 * j + c, p1 = 32 * j + 16 + c;
        const int s0 = p0 < nwin ? window_slot(ia.S, ia.start_pos, aa.W, aa.R, i, p0) : -1;
        const int s1 = p1 < nwin ? window_slot(ia.S, ia.start_pos, aa.W, aa.R, i, p1) : -1;
        attn_tile_load<D>(wrows, s0 >= 0 ? aa.win_kv + ((size_t)b * aa.R + s0) * D : nullptr,
                          s1 >= 0 ? aa.win_kv + ((size_t)b * aa.R + s1) * D : nullptr, g);
    }

    // ------------------------------------------------------------- phase S
    uint32_t kstar = 0u;  // a pick is key > kstar, or key == kstar with position <= pstar
    int pstar = 0x7fffffff;
    int off = c0;         // where this member's picks start in the output list
    if (select) {
        team_wait(&ctrl[kBarA], (uint32_t)f.team_size, f.spin_limit, f.err);
        const uint64_t *tp = reinterpret_cast<const uint64_t *>(ts);
        const int npair = (nvis + 1) / 2;
        const bool cached = npair <= kCache * kThreads;
        uint64_t vals[kCache];
        if (cached) {
#pragma unroll
            for (int r = 0; r < kCache; ++r) {
                const int pi = tid + r * kThreads;
                vals[r] = pi < npair ? ld64_agent(tp + pi) : 0ull;
            }
        }
        // visit every (pair index, pair) of the team's scores
        auto each = [&](auto &&fn) {
            if (cached) {
#pragma unroll
                for (int r = 0; r < kCache; ++r) {
                    const int pi = tid + r * kThreads;
                    if (pi < npair) fn(pi, vals[r]);
                }
            } else {
                for (int pi = tid; pi < npair; pi += kThreads) fn(pi, ld64_agent(tp + pi));
            }
        };
        // pass 1: team min / max
        float mx = -INFINITY, mn = INFINITY;
        each([&](int pi, uint64_t v) {
            mx = fmaxf(mx, lo_f(v));
            mn = fminf(mn, lo_f(v));
            if (2 * pi + 1 < nvis) {
                mx = fmaxf(mx, hi_f(v));
                mn = fminf(mn, hi_f(v));
            }
        });
        for (int j = tid; j < kBins; j += kThreads) sm.hist[j] = 0u;
        mx = wg_max(mx, sm.fred);
        mn = wg_min(mn, sm.fred);
        const float scale = mx > mn ? (float)kBins / (mx - mn) : 0.f;
        // pass 2: value histogram
        each([&](int pi, uint64_t v) {
            atomicAdd(&sm.hist[value_bin(lo_f(v), mn, scale)], 1u);
            if (2 * pi + 1 < nvis) atomicAdd(&sm.hist[value_bin(hi_f(v), mn, scale)], 1u);
        });
        __syncthreads();
        find_bin(sm.hist, kBins, f.keff, sm.wsum, &sm.bin, &sm.above);
        const int vb = sm.bin;
        const int need = f.keff - sm.above;
        const int cnt = (int)sm.hist[vb];
        // pass 3: the candidates (scores in bin vb) into LDS when they fit
        uint32_t *ckey = reinterpret_cast<uint32_t *>(attn_lds);
        int *cpos = reinterpret_cast<int *>(ckey + kCandCap);
        if (tid == 0) {
            sm.ncand = 0;
            sm.kstar = 0u;
            sm.pstar = 0x7fffffff;
        }
        __syncthreads();
        if (cnt <= kCandCap) {
            each([&](int pi, uint64_t v) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float x = h ? hi_f(v) : lo_f(v);
                    const int t = 2 * pi + h;
                    if (t < nvis && value_bin(x, mn, scale) == vb) {
                        const int sidx = atomicAdd(&sm.ncand, 1);
                        ckey[sidx] = order_key(x);
                        cpos[sidx] = t;
                    }
                }
            });
            __syncthreads();
            // rank every candidate by (key desc, position asc); the (need-1)-th is the cut
            for (int j = tid; j < cnt; j += kThreads) {
                const uint32_t kj = ckey[j];
                const int pj = cpos[j];
                int rank = 0;
                for (int o = 0; o < cnt; ++o) {
                    const uint32_t ko = ckey[o];
                    rank += ko > kj || (ko == kj && cpos[o] < pj);
                }
                if (rank == need - 1) {
                    sm.kstar = kj;
                    sm.pstar = pj;
                }
            }
            __syncthreads();
        } else {
            radix_resolve(sm, ts, nvis, mn, scale, vb, need);
        }
        kstar = sm.kstar;
        pstar = sm.pstar;
        // pass 4: picks at positions before this member's chunk
        uint32_t before = 0;
        each([&](int pi, uint64_t v) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = 2 * pi + h;
                const uint32_t k = order_key(h ? hi_f(v) : lo_f(v));
                before += t < c0 && (k > kstar || (k == kstar && t <= pstar));
            }
        });
        off = (int)wg_sum(before, sm.wsum);
    }

    // ------------------------------------------------------------------ phase D
    int32_t *idx_row = f.topk_out + (size_t)q * f.keff;
    {
        const int per = (n + kThreads - 1) / kThreads;
        const int t0 = tid * per, t1 = min(t0 + per, n);
        uint32_t mine = 0;
        for (int t = t0; t < t1; ++t) {
            const uint32_t k = order_key(sc[t]);
            mine += !select || k > kstar || (k == kstar && c0 + t <= pstar);
        }
        uint32_t total;
        const uint32_t incl = wg_scan(mine, sm.wsum, &total);
        int o = (int)(incl - mine);
        for (int t = t0; t < t1; ++t) {
            const uint32_t k = order_key(sc[t]);
            if (!select || k > kstar || (k == kstar && c0 + t <= pstar)) {
                picks[o] = c0 + t;
                if (off + o < f.keff) idx_row[off + o] = c0 + t;
                ++o;
            }
        }
        if (tid == 0) sm.npick = (int)total;
        if (m == 0 && !select)
            for (int j = nvis + tid; j < f.keff; j += kThreads) idx_row[j] = -1;
        __syncthreads();
    }
    {
        const float sl2 = aa.scale * kLog2e;
        uint16_t *tile = attn_lds + wave * 32 * LD;
        const int npick = sm.npick;
        const int pick_tiles = (npick + 31) / 32;
        AttnState<D> st;
        attn_init<D>(st);
        if (win_w < my_win) attn_tile_compute<D>(st, qb, wrows, tile, aa.dv / 16, sl2, g, c);
        // window tiles beyond the prefetched ones (more than 4 per member)
        for (int w = 4 + wave; w < my_win; w += 4) {
            const int j = m + w * f.team_size;
            const int p0 = 32 * j + c, p1 = 32 * j + 16 + c;
            const int s0 = p0 < nwin ? window_slot(ia.S, ia.start_pos, aa.W, aa.R, i, p0) : -1;
            const int s1 = p1 < nwin ? window_slot(ia.S, ia.start_pos, aa.W, aa.R, i, p1) : -1;
            AttnRows<D> rows;
            attn_tile_load<D>(rows, s0 >= 0 ? aa.win_kv + ((size_t)b * aa.R + s0) * D : nullptr,
                              s1 >= 0 ? aa.win_kv + ((size_t)b * aa.R + s1) * D : nullptr, g);
            attn_tile_compute<D>(st, qb, rows, tile, aa.dv / 16, sl2, g, c);
        }
        for (int tt = wave; tt < pick_tiles; tt += 4) {
            const int p0 = 32 * tt + c, p1 = 32 * tt + 16 + c;
            AttnRows<D> rows;
            attn_tile_load<D>(rows, p0 < npick ? aa.comp_kv + ((size_t)b * aa.T_cap + picks[p0]) * D : nullptr,
                              p1 < npick ? aa.comp_kv + ((size_t)b * aa.T_cap + picks[p1]) * D : nullptr, g);
            attn_tile_compute<D>(st, qb, rows, tile, aa.dv / 16, sl2, g, c);
        }
        __syncthreads();
        float *ow = reinterpret_cast<float *>(attn_lds);
        attn_wave_publish<D>(st, ow, wm, wl, wave, aa.dv, g, c);
        __syncthreads();
        // this member's state: O [16][dv] then (M, L) [16], as float pairs
        uint64_t *slot = reinterpret_cast<uint64_t *>(f.part + ((size_t)q * f.team_size + m) * f.slot_floats);
        const int half_dv = aa.dv / 2;
        for (int e = tid; e < kHeads * half_dv; e += kThreads) {
            const int h = e / half_dv;
            const int d = 2 * (e - h * half_dv);
            float O0, O1, M, L;
            attn_combine(ow, wm, wl, 4, h, d, aa.dv, O0, M, L);
            attn_combine(ow, wm, wl, 4, h, d + 1, aa.dv, O1, M, L);
            st64_agent(slot + (h * aa.dv + d) / 2, pack2(O0, O1));
        }
        if (tid < kHeads) {
            float O, M, L;
            attn_combine(ow, wm, wl, 4, tid, 0, aa.dv, O, M, L);
            st64_agent(slot + (kHeads * aa.dv) / 2 + tid, pack2(M, L));
        }
    }
    team_arrive(&ctrl[kBarC]);
    team_wait(&ctrl[kBarC], (uint32_t)f.team_size, f.spin_limit, f.err);

    // ------------------------------------------------------------------ phase M
    {
        // this member's slice of the (head, dim-pair) outputs
        const int half_dv = aa.dv / 2;
        const int n_out = kHeads * half_dv;
        const int per = (n_out + f.team_size - 1) / f.team_size;
        const int e0 = m * per, e1 = min(e0 + per, n_out);
        float *smax = reinterpret_cast<float *>(attn_lds);
        float *snrm = smax + f.team_size * kHeads;
        const uint64_t *tp = reinterpret_cast<const uint64_t *>(f.part + (size_t)q * f.team_size * f.slot_floats);
        const int slot_pairs = f.slot_floats / 2;
        for (int j = tid; j < f.team_size * kHeads; j += kThreads) {
            const int s = j / kHeads, h = j % kHeads;
            const uint64_t ml = ld64_agent(tp + (size_t)s * slot_pairs + (kHeads * aa.dv) / 2 + h);
            smax[j] = lo_f(ml);
            snrm[j] = hi_f(ml);
        }
        __syncthreads();
        for (int e = e0 + tid; e < e1; e += kThreads) {
            const int h = e / half_dv;
            const int d = 2 * (e - h * half_dv);
            float M = -INFINITY;
            for (int s = 0; s < f.team_size; ++s) M = fmaxf(M, smax[s * kHeads + h]);
            float O0 = 0.f, O1 = 0.f, L = 0.f;
            if (M != -INFINITY) {
                for (int s = 0; s < f.team_size; ++s) {
                    const float ms = smax[s * kHeads + h];
                    const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
                    const uint64_t o = ld64_agent(tp + (size_t)s * slot_pairs + (h * aa.dv + d) / 2);
                    O0 += w * lo_f(o);
                    O1 += w * hi_f(o);
                    L += w * snrm[s * kHeads + h];
                }
            }
            uint16_t *dst = aa.out + ((size_t)q * kHeads + h) * aa.dv + d;
            dst[0] = attn_finish(O0, M, L, aa.sink, h);
            dst[1] = attn_finish(O1, M, L, aa.sink, h);
        }
    }
    // the last member to finish zeroes the team's control words for the next launch
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&ctrl[kDone], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (uint32_t)f.team_size - 1u)
            for (int j = 0; j < kCtrlWords; ++j) st_agent(&ctrl[j], 0u);
    }
}

template <int D, int DI, int HT>
hipError_t launch_fused_cfg(const FusedArgs &f, int grid, size_t dyn_bytes, hipStream_t stream) {
    hipLaunchKernelGGL((fused_decode_kernel<D, DI, HT>), dim3(grid), dim3(kThreads), dyn_bytes, stream, f);
    return hipGetLastError();
}

template <int D, int DI>
hipError_t launch_fused_di(const FusedArgs &f, int grid, size_t dyn, hipStream_t s) {
    switch (f.ia.Hi / 16) {
        case 1: return launch_fused_cfg<D, DI, 1>(f, grid, dyn, s);
        case 2: return launch_fused_cfg<D, DI, 2>(f, grid, dyn, s);
        case 3: return launch_fused_cfg<D, DI, 3>(f, grid, dyn, s);
        case 4: return launch_fused_cfg<D, DI, 4>(f, grid, dyn, s);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_fused_d(const FusedArgs &f, int grid, size_t dyn, hipStream_t s) {
    return f.ia.Di == 64 ? launch_fused_di<D, 64>(f, grid, dyn, s) : launch_fused_di<D, 128>(f, grid, dyn, s);
}

// Compute units of a device (queried once per device).
int device_cus(int dev) {
    static std::atomic<int> cache[64];
    if (dev < 0 || dev >= 64) return 0;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev].store(v, std::memory_order_relaxed);
    return v;
}

// Co-resident workgroups of the fused kernel on the current device.
int max_resident(int D, int DI, int HT, size_t dyn) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int cus = device_cus(dev);
    if (cus <= 0) return 0;
    int per_cu = 0;
    hipError_t e = hipErrorInvalidValue;
#define LIT_OCC(DD, II, HH)                                                                              \
    if (D == DD && DI == II && HT == HH)                                                                 \
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_decode_kernel<DD, II, HH>, kThreads, dyn);
#define LIT_OCC_D(DD) LIT_OCC(DD, 64, 1) LIT_OCC(DD, 64, 2) LIT_OCC(DD, 64, 3) LIT_OCC(DD, 64, 4) \
                      LIT_OCC(DD, 128, 1) LIT_OCC(DD, 128, 2) LIT_OCC(DD, 128, 3) LIT_OCC(DD, 128, 4)
    LIT_OCC_D(64) LIT_OCC_D(128) LIT_OCC_D(192) LIT_OCC_D(256)
#undef LIT_OCC_D
#undef LIT_OCC
    if (e != hipSuccess) return 0;
    return cus * per_cu;
}

}  // namespace

FusedPlan plan_fused(int B, int S, int start_pos, int ratio, int Hi, int Di, int D, int dv, int W, int keff) {
    FusedPlan p{};
    p.ok = false;
    const int n_teams = B * S;
    const long T = ((long)start_pos + S) / ratio;
    if (n_teams <= 0 || keff <= 0 || T <= 0 || T > (1L << 24)) return p;
    if (D != 64 && D != 128 && D != 192 && D != 256) return p;
    if ((Di != 64 && Di != 128) || Hi % 16 || Hi > 64) return p;
    const int nwin = window_width(S, start_pos, W);
    p.win_tiles = (nwin + 31) / 32;
    int chunk = 256;
    size_t dyn = 0;
    int cap = 0;
    for (;; chunk *= 2) {
        if (chunk > 8192) return p;
        dyn = (size_t)chunk * 2 * sizeof(float);  // chunk scores + picks
        cap = max_resident(D, Di, Hi / 16, dyn);
        const long team = (T + chunk - 1) / chunk;
        if (cap > 0 && team <= kThreads && (long)n_teams * team <= cap) {
            p.team_size = (int)team;
            break;
        }
        if (cap <= 0) return p;
    }
    p.chunk = chunk;
    p.dyn_bytes = dyn;
    p.n_teams = n_teams;
    p.grid = n_teams * p.team_size;
    p.n_slots = p.team_size;
    // the merge stages two floats per (member, head) in the attention LDS buffer, and the
    // window tiles are spread one per member
    if ((size_t)p.n_slots * kHeads * 2 * sizeof(float) > (size_t)4 * 32 * (D + 4) * sizeof(uint16_t)) return p;
    p.ld = (T + 3) / 4 * 4;
    p.ok = true;
    (void)dv;
    return p;
}

size_t fused_state_bytes(const FusedPlan &p) {
    // error word + per-team control words
    return 256 + (size_t)p.n_teams * kCtrlWords * 4;
}

static int slot_floats(int dv) { return (kHeads * dv + 2 * kHeads + 63) / 64 * 64; }

size_t fused_ws_bytes(const FusedPlan &p, int dv) {
    return (size_t)p.n_teams * p.ld * 4 + 256 +                              // team scores
           (size_t)p.n_teams * p.team_size * slot_floats(dv) * 4 + 256;      // partial states
}

hipError_t launch_fused(FusedArgs f, const FusedPlan &p, void *ws, void *state, hipStream_t stream) {
    char *st = (char *)state;
    f.err = (uint32_t *)st;
    f.ctrl = (uint32_t *)(st + 256);
    char *rest = (char *)ws;
    auto bump = [&](size_t bytes) {
        char *r = rest;
        rest += (bytes + 255) / 256 * 256;
        return r;
    };
    f.scores = (float *)bump((size_t)p.n_teams * p.ld * 4);
    f.part = (float *)bump((size_t)p.n_teams * p.team_size * slot_floats(f.aa.dv) * 4);
    f.slot_floats = slot_floats(f.aa.dv);
    f.team_size = p.team_size;
    f.chunk = p.chunk;
    f.win_tiles = p.win_tiles;
    f.n_slots = p.n_slots;
    f.ld = p.ld;
    switch (f.aa.D) {
        case 64: return launch_fused_d<64>(f, p.grid, p.dyn_bytes, stream);
        case 128: return launch_fused_d<128>(f, p.grid, p.dyn_bytes, stream);
        case 192: return launch_fused_d<192>(f, p.grid, p.dyn_bytes, stream);
        case 256: return launch_fused_d<256>(f, p.grid, p.dyn_bytes, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace lit
