// topk.hip -- per-query top-k of the indexer scores, in position order.
//
// What is computed (DeepSeek-V4.1-Flash-NVFP4 inference/model.py, Indexer.forward):
// the k_eff = min(index_topk, end_pos/ratio) best-scoring visible rows of each query,
// listed in ascending row order, with -1 filling the slots of a query that sees fewer
// rows.  Ties go to the lower row.
//
// Design.  One 1024-thread workgroup per query row.  Scores become order-preserving
// 32-bit keys (larger float -> larger key, -0 folded onto +0) kept in VGPRs, blocked
// so that thread j owns a contiguous run of positions.  A three-pass radix select
// (11 + 11 + 10 bits, most significant first) finds the exact key of the k-th pick:
// each pass histograms the keys that still match the prefix into 2048 LDS bins, and
// a block-wide scan over the bins from the top finds the bin where the running count
// reaches the number still to pick.  A final pass counts, per thread, keys above the
// threshold and keys equal to it; one packed block scan turns those counts into
// output offsets, so each selected position lands in its ascending slot with no sort.
// Rows longer than 1024*ITEMS are processed in segments re-read from L2.
//
// Unmasked rows whose score arrays hold 1025..8192 positions take a lighter kernel
// instead, whatever the number of rows: one 256-thread workgroup per row, each thread
// owning 32 positions in VGPRs, and the value-bin selection of select_ops.h (one
// histogram pass, then the few scores of the cut's bin ranked exactly), so a row costs
// a few workgroup barriers rather than three radix passes of a 1024-thread workgroup.
// Arrays of 8193..32768 positions take the same kernel with 1024 threads.
#include "select_ops.h"

namespace lit {

namespace {

constexpr int kThreads = 1024;
// order key of -inf: the key every masked column takes (and a visible -inf score too)
constexpr uint32_t kMaskedKey = 0x007FFFFFu;

// Columns a query sees: its visible rows, or (level one) the blocks holding them.
__device__ inline int visible_columns(const TopkArgs &a, int i) {
    const int rows = min(a.T, (a.start_pos + i + 1) / a.ratio);
    return a.vis_block > 1 ? (rows + a.vis_block - 1) / a.vis_block : rows;
}

template <int ITEMS, bool CAND>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
    __shared__ int hist[2048];
    __shared__ uint32_t wsum[kThreads / 64];
    __shared__ int sel_bin;
    __shared__ int sel_above;
    __shared__ uint32_t keep[CAND ? kCandMaxBlocks / 32 : 1];  // level two: kept-block bitmap

    const int row = blockIdx.x;
    const int i = row % a.S;
    const int tid = threadIdx.x;
    const int n = visible_columns(a, i);
    int32_t *out = a.idx + (size_t)row * a.keff;
    const float *src = a.scores + (size_t)row * a.ld;

    if (n <= a.keff) {  // every visible column is picked
        for (int j = tid; j < a.keff; j += kThreads) out[j] = j < n ? j : -1;
        return;
    }

    if constexpr (CAND) {
        const int nb = (n + a.cand_bs - 1) / a.cand_bs;  // blocks this query can see
        for (int j = tid; j < (nb + 31) / 32; j += kThreads) keep[j] = 0u;
        __syncthreads();
        const int32_t *cl = a.cand + (size_t)row * a.cand_k;
        for (int j = tid; j < a.cand_k; j += kThreads) {
            const int blk = cl[j];
            if (blk >= 0 && blk < nb) atomicOr(&keep[blk >> 5], 1u << (blk & 31));
        }
        __syncthreads();
    }
    // masked columns (level two) take the key of -inf
    auto key_at = [&](int t, float v) -> uint32_t {
        if constexpr (CAND) {
            const int blk = t / a.cand_bs;
            if (!((keep[blk >> 5] >> (blk & 31)) & 1u)) return kMaskedKey;
        }
        return order_key(v);
    };

    constexpr int SEG = kThreads * ITEMS;
    const int nseg = (n + SEG - 1) / SEG;
    uint32_t keys[ITEMS];
    auto load = [&](int seg) -> int {
        const int base = seg * SEG + tid * ITEMS;
        const int cnt = max(0, min(ITEMS, n - base));
        if (cnt == ITEMS) {
#pragma unroll
            for (int u = 0; u < ITEMS; u += 4) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(src + base + u);
                keys[u] = key_at(base + u, v[0]);
                keys[u + 1] = key_at(base + u + 1, v[1]);
                keys[u + 2] = key_at(base + u + 2, v[2]);
                keys[u + 3] = key_at(base + u + 3, v[3]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < ITEMS; ++u) keys[u] = u < cnt ? key_at(base + u, src[base + u]) : 0u;
        }
        return cnt;
    };

    int cnt0 = 0;
    if (nseg == 1) cnt0 = load(0);

    uint32_t prefix = 0u, pmask = 0u;
    int remaining = a.keff;
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int j = tid; j < 2048; j += kThreads) hist[j] = 0;
        __syncthreads();
        // masked columns (level two) share one key: counted per thread and added once per
        // wave, since thousands of LDS atomics on one counter would serialise
        uint32_t nmask = 0;
        for (int seg = 0; seg < nseg; ++seg) {
            const int cnt = nseg == 1 ? cnt0 : load(seg);
#pragma unroll
            for (int u = 0; u < ITEMS; ++u)
                if (u < cnt && (keys[u] & pmask) == prefix) {
                    if (CAND && keys[u] == kMaskedKey)
                        ++nmask;
                    else
                        atomicAdd(&hist[(keys[u] >> shift) & (nbins - 1)], 1);
                }
        }
        if constexpr (CAND) {
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) nmask += (uint32_t)__shfl_xor((int)nmask, off);
            if ((tid & 63) == 0 && nmask) atomicAdd(&hist[(kMaskedKey >> shift) & (nbins - 1)], (int)nmask);
        }
        __syncthreads();
        // Thread j owns bins hi = nbins-1-2j and hi-1 (descending); the scan over
        // threads counts the keys in the bins above.
        int c_hi = 0, c_lo = 0;
        const int hi = nbins - 1 - 2 * tid;
        if (hi >= 1) {
            c_hi = hist[hi];
            c_lo = hist[hi - 1];
        }
        uint32_t total;
        const uint32_t incl = wg_scan<kThreads / 64>((uint32_t)(c_hi + c_lo), wsum, &total);
        const int above = (int)incl - c_hi - c_lo;
        if (hi >= 1) {
            if (above < remaining && remaining <= above + c_hi) {
                sel_bin = hi;
                sel_above = above;
            } else if (above + c_hi < remaining && remaining <= above + c_hi + c_lo) {
                sel_bin = hi - 1;
                sel_above = above + c_hi;
            }
        }
        __syncthreads();
        remaining -= sel_above;
        prefix |= (uint32_t)sel_bin << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
    }

    // prefix is now the exact key of the k-th pick; take every key above it and the
    // first `remaining` keys equal to it, in position order.
    const uint32_t thr = prefix;
    const int need_eq = remaining;
    int base_gt = 0, base_eq = 0;
    for (int seg = 0; seg < nseg; ++seg) {
        const int cnt = nseg == 1 ? cnt0 : load(seg);
        uint32_t ngt = 0, neq = 0;
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            if (u < cnt) {
                ngt += keys[u] > thr;
                neq += keys[u] == thr;
            }
        }
        const uint32_t packed = (ngt << 16) | neq;
        uint32_t total;
        const uint32_t excl = wg_scan<kThreads / 64>(packed, wsum, &total) - packed;
        int gt = base_gt + (int)(excl >> 16);
        int eq = base_eq + (int)(excl & 0xffffu);
        const int pos0 = seg * SEG + tid * ITEMS;
#pragma unroll
        for (int u = 0; u < ITEMS; ++u) {
            if (u < cnt) {
                if (keys[u] > thr) {
                    const int dst = gt + min(eq, need_eq);
                    if (dst < a.keff) out[dst] = pos0 + u;
                    ++gt;
                } else if (keys[u] == thr) {
                    if (eq < need_eq && gt + eq < a.keff) out[gt + eq] = pos0 + u;
                    ++eq;
                }
            }
        }
        base_gt += (int)(total >> 16);
        base_eq += (int)(total & 0xffffu);
    }
}

constexpr int kRowQ = 8;                // score quads per thread: rows of up to 8192 positions
constexpr int kRowCap = kCandCap / 2;   // candidates held in LDS (more take the radix levels)
constexpr int kRowBins2 = kBins - 2 * kRowCap;  // bins of the candidate refinement

// NT = 256: seven rows a compute unit (72 VGPRs; 16.5 KB of LDS, the row's whole LDS being
// the selection's histogram, which later holds the candidates in its first half and their
// refinement histogram in the second); NT = 1024 (rows of up to 32768 positions, few rows):
// one 16-wave workgroup a row.
template <int NT>
__global__ __launch_bounds__(NT, NT == 256 ? 7 : 1) void topk_rows_kernel(TopkArgs a) {
    __shared__ SelLdsT<NT> sm;
    __shared__ uint32_t mm[NT / 64][2];

    const int row = blockIdx.x;
    const int i = row % a.S;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = visible_columns(a, i);
    int32_t *out = a.idx + (size_t)row * a.keff;
    const float *src = a.scores + (size_t)row * a.ld;

    if (n <= a.keff) {  // every visible row is picked
        for (int j = tid; j < a.keff; j += NT) out[j] = j < n ? j : -1;
        return;
    }

    // quad r of thread tid holds positions 4 (tid + 256 r) .. +3, so each load of a wave
    // reads 1 KB of consecutive scores.  Positions past the row hold a copy of position
    // 0's score (a visible row: n > keff >= 1), which leaves the row's min and max
    // unchanged; their histogram counts are taken back below, and the validity nibbles
    // vn (bit 4r+e: position valid) keep them out of the candidates and picks.
    const float v0 = src[0];
    f32x4 v[kRowQ];
    uint32_t vn = 0u;
#pragma unroll
    for (int r = 0; r < kRowQ; ++r) {
        const int q = tid + NT * r;
        v[r] = *reinterpret_cast<const f32x4 *>(src + 4 * (4 * q < n ? q : 0));
        vn |= ((1u << min(max(n - 4 * q, 0), 4)) - 1u) << (4 * r);
    }
#pragma unroll
    for (int r = 0; r < kRowQ; ++r)
        if (((vn >> (4 * r)) & 0xFu) != 0xFu)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (!((vn >> (4 * r + e)) & 1u)) v[r][e] = v0;
    auto pos = [&](int r, int e) { return 4 * (tid + NT * r) + e; };

    // the row's min and max by order keys (-0 and +0 need not be told apart here: both give
    // the float 0), reduced over the workgroup through mm[]
    auto minmax = [&](bool skip_inf, uint32_t &kmax, uint32_t &kmin) {
        kmax = 0u;
        kmin = ~0u;
#pragma unroll
        for (int r = 0; r < kRowQ; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t u = __float_as_uint(v[r][e]);
                const uint32_t k = u ^ ((uint32_t)((int)u >> 31) | 0x80000000u);
                const bool inf = skip_inf && (u & 0x7fffffffu) == 0x7f800000u;
                kmax = inf ? kmax : max(kmax, k);
                kmin = inf ? kmin : min(kmin, k);
            }
        kmax = wave_max_u32(kmax);
        kmin = wave_min_u32(kmin);
        __syncthreads();  // mm[] of an earlier reduction has been read
        if (lane == 0) {
            mm[wave][0] = kmax;
            mm[wave][1] = kmin;
        }
        __syncthreads();
        kmax = 0u;
        kmin = ~0u;
        for (int w = 0; w < NT / 64; ++w) {
            kmax = max(kmax, mm[w][0]);
            kmin = min(kmin, mm[w][1]);
        }
    };
    for (int j = tid; j < kVBins / 4 + 1; j += NT)  // + the spill bin
        reinterpret_cast<u32x4 *>(sm.hist)[j] = u32x4{0u, 0u, 0u, 0u};
    uint32_t kmax, kmin;
    minmax(false, kmax, kmin);
    // the scores pass through an empty asm, so that later uses take their order keys again
    // rather than keeping these 32 alive
#pragma unroll
    for (int r = 0; r < kRowQ; ++r) asm volatile("" : "+v"(v[r]));
    float mx = key_float(kmax), mn = key_float(kmin);
    // An infinite end (level one of the two-level top-k pins one block at +inf) would stretch
    // the range to nothing: the range is then taken over the finite scores, and an infinity
    // lands in an end bin, which keeps the map monotone.  No finite score, a NaN, or a span
    // beyond the float range puts every score into one bin; the exact levels below decide.
    if (mx == INFINITY || mn == -INFINITY) {
        minmax(true, kmax, kmin);
        mx = key_float(kmax);
        mn = key_float(kmin);
    }
    const bool finite = kmax >= kmin && mx - mn < INFINITY;
    const float scale = finite && mx > mn ? (float)kVBins / (mx - mn) : 0.f;
    const float bias = finite ? -mn * scale : 0.f;

    // pass 1: the histogram of value bins.  Quads wholly past the row add nothing (a wave's
    // quads are consecutive, so this is a wave-uniform skip outside the boundary wave);
    // thousands of copies of one score would otherwise serialise on one bin's atomics.
#pragma unroll
    for (int r = 0; r < kRowQ; ++r)
        if (4 * (tid + NT * r) < n)
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&sm.hist[value_bin(v[r][e], scale, bias)], 1u);
    // the copies of position 0's score in the row's last, partial quad
    if (tid == 0 && (n & 3)) atomicSub(&sm.hist[value_bin(v0, scale, bias)], (uint32_t)(4 - (n & 3)));
    __syncthreads();
    find_bin<NT>(sm.hist, kVBins, a.keff, sm.wsum, &sm.bin, &sm.above);
    const int vb = sm.bin;
    const int need = a.keff - sm.above;
    const int cnt = (int)sm.hist[vb];
    __syncthreads();  // every thread has read hist[vb]: both paths below overwrite the histogram
    // per element (bit 4r+e): its bin is above vb (gm) or is vb (cm, the candidates).  The
    // bins are taken again from the scores rather than kept (16 registers fewer): the bin is
    // the clamped fma truncated, and for an integer c, truncation of a value x >= 0 is at
    // least c exactly when x is, so the float comparisons below decide the same.
    uint32_t gm = 0u, cm = 0u;
    {
        // opaque copies of the map, so that the compiler takes the bins again here instead
        // of keeping pass 1's 32 values alive across the bin search
        float rscale = scale, rbias = bias;
        asm volatile("" : "+v"(rscale), "+v"(rbias));
        const float fgt = (float)(vb + 1), fge = (float)vb;
#pragma unroll
        for (int r = 0; r < kRowQ; ++r) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = fminf(fmaxf(fmaf(v[r][e], rscale, rbias), 0.f), (float)(kVBins - 1));
                gm |= (uint32_t)(x >= fgt) << (4 * r + e);
                cm |= (uint32_t)(x >= fge && x < fgt) << (4 * r + e);
            }
            asm volatile("" : "+v"(gm), "+v"(cm));  // quad r's bins end here
        }
        gm &= vn;
        cm &= vn;
    }
    uint32_t kstar, pstar;
    if (cnt <= kRowCap) {
        // the scores of bin vb as (key << 32 | ~position), in the histogram's place; a
        // block scan over the threads' counts gives each its first slot
        uint64_t *cand = reinterpret_cast<uint64_t *>(sm.hist);
        uint32_t total;
        const uint32_t mine = (uint32_t)__popc(cm);
        int o = (int)(wg_scan<NT / 64, false>(mine, sm.wsum, &total) - mine);  // (a barrier follows the writes)
        if (cm) {
#pragma unroll
            for (int r = 0; r < kRowQ; ++r)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((cm >> (4 * r + e)) & 1u)
                        cand[o++] = ((uint64_t)order_key(v[r][e]) << 32) | (uint32_t)~(uint32_t)pos(r, e);
        }
        __syncthreads();
        int ncand = cnt, nneed = need;
        refine_candidates<NT, kRowCap, kRowBins2>(cand, ncand, nneed, sm.hist + 2 * kRowCap, sm);
        rank_candidates(cand, ncand, nneed, sm);
    } else {
        radix_resolve(sm, [&](int t) { return src[t]; }, n, scale, bias, vb, need);
    }
    kstar = sm.kstar;
    pstar = (uint32_t)sm.pstar;

    // output: a pick is key > kstar, or key == kstar at a position <= pstar: every element
    // above bin vb, and the candidates (bin vb) that pass the test.  The picks become a
    // bitmap over positions in LDS (the histogram is free again; word w covers positions 32w..32w+31,
    // assembled from 8 lanes' nibbles), and thread t then writes the picks of word t at the
    // offset one block scan gives it, in ascending order.
    uint32_t pm = gm;
    if (cm) {
#pragma unroll
        for (int r = 0; r < kRowQ; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if ((cm >> (4 * r + e)) & 1u) {
                    const uint32_t k = order_key(src[pos(r, e)]);
                    if (k > kstar || (k == kstar && (uint32_t)pos(r, e) <= pstar)) pm |= 1u << (4 * r + e);
                }
    }
    uint32_t *bm = sm.hist;
#pragma unroll
    for (int r = 0; r < kRowQ; ++r) {
        // OR over the 8 lanes: swap neighbours, swap pairs (DPP quad permutations), then
        // mirror within the half-row of 8 lanes
        const uint32_t nib = (pm >> (4 * r)) & 0xFu;
        int x = (int)(nib << (4 * (tid & 7)));
        x |= __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false);
        x |= __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false);
        x |= __builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false);
        if ((tid & 7) == 0) bm[NT / 8 * r + (tid >> 3)] = (uint32_t)x;
    }
    __syncthreads();
    uint32_t w = bm[tid];
    uint32_t total;
    int o = (int)(wg_scan<NT / 64, false>((uint32_t)__popc(w), sm.wsum, &total) - (uint32_t)__popc(w));
    while (w) {
        const int bit = __builtin_ctz(w);
        w &= w - 1u;
        if (o < a.keff) out[o] = 32 * tid + bit;
        ++o;
    }
}

__global__ __launch_bounds__(256) void block_max_kernel(const float *scores, long ld, int S, int start_pos,
                                                        int ratio, int T, int bs, float *bscores, long ldb) {
    const int row = blockIdx.y;
    const int i = row % S;
    const int j = blockIdx.x * 256 + threadIdx.x;
    const int nvis = min(T, (start_pos + i + 1) / ratio);
    const int nb = (nvis + bs - 1) / bs;
    if (j >= nb) return;
    const float *src = scores + (size_t)row * ld;
    float m = -INFINITY;
    const int t1 = min(j * bs + bs, nvis);
    for (int t = j * bs; t < t1; ++t) m = fmaxf(m, src[t]);
    // the block of the newest visible row is kept whatever its score
    bscores[(size_t)row * ldb + j] = j == (nvis - 1) / bs ? INFINITY : m;
}

}  // namespace

hipError_t launch_block_max(const float *scores, long ld, int B, int S, int start_pos, int ratio, int T, int bs,
                            float *bscores, long ldb, hipStream_t stream) {
    const int nblocks = (T + bs - 1) / bs;
    if (B <= 0 || S <= 0 || nblocks <= 0) return hipSuccess;
    dim3 grid((nblocks + 255) / 256, B * S);
    hipLaunchKernelGGL(block_max_kernel, grid, dim3(256), 0, stream, scores, ld, S, start_pos, ratio, T, bs,
                       bscores, ldb);
    return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, hipStream_t stream) {
    if (a.B <= 0 || a.S <= 0 || a.keff <= 0) return hipSuccess;
    dim3 grid(a.B * a.S), block(kThreads);
    const int cols = a.vis_block > 1 ? (a.T + a.vis_block - 1) / a.vis_block : a.T;
    if (a.masked) {
        if ((cols + a.cand_bs - 1) / a.cand_bs > kCandMaxBlocks) return hipErrorInvalidValue;
        if (cols <= kThreads * 4)
            hipLaunchKernelGGL((topk_kernel<4, true>), grid, block, 0, stream, a);
        else if (cols <= kThreads * 8)
            hipLaunchKernelGGL((topk_kernel<8, true>), grid, block, 0, stream, a);
        else if (cols <= kThreads * 16)
            hipLaunchKernelGGL((topk_kernel<16, true>), grid, block, 0, stream, a);
        else
            hipLaunchKernelGGL((topk_kernel<32, true>), grid, block, 0, stream, a);
        return hipGetLastError();
    }
    if (cols <= kSelThreads * 4 * kRowQ && cols > 1024) {  // rows of 1025..8192 positions
        hipLaunchKernelGGL(topk_rows_kernel<kSelThreads>, grid, dim3(kSelThreads), 0, stream, a);
        return hipGetLastError();
    }
    if (cols > kSelThreads * 4 * kRowQ && cols <= 1024 * 4 * kRowQ) {  // few rows of 8193..32768
        // positions: a 1024-thread workgroup each
        hipLaunchKernelGGL(topk_rows_kernel<1024>, grid, dim3(1024), 0, stream, a);
        return hipGetLastError();
    }
    if (cols <= kThreads * 4)
        hipLaunchKernelGGL((topk_kernel<4, false>), grid, block, 0, stream, a);
    else if (cols <= kThreads * 8)
        hipLaunchKernelGGL((topk_kernel<8, false>), grid, block, 0, stream, a);
    else if (cols <= kThreads * 16)
        hipLaunchKernelGGL((topk_kernel<16, false>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((topk_kernel<32, false>), grid, block, 0, stream, a);
    return hipGetLastError();
}

}  // namespace lit
