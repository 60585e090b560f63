// select_ops.h -- exact k-th selection over fp32 scores in one workgroup (256 threads, or
// 1024 for rows of up to 32768 positions), shared by the fused decode step and the row
// top-k kernel.
//
// The selection is exact: the k-th largest score by (order key desc, position asc), so
// equal scores go to the lower position.  Level one is a 4096-bin histogram of the
// values between the row's min and max (a monotone map: every score in a higher bin is
// larger than every score in a lower one), a bin search from the top finds the bin that
// holds the cut, and the few scores of that bin are ranked directly as 64-bit
// (key, ~position) composites -- after narrowing by histograms over their own range
// when there are many, or by radix levels over the order keys when there are more than
// an LDS buffer holds.
#pragma once

#include "tile_ops.h"

namespace lit {

constexpr int kSelThreads = 256;  // threads of a selecting workgroup
constexpr int kBins = 4096;       // radix-level histogram size (12-bit digits)
constexpr int kVBins = 4096;      // value bins of the first level (+ one spill bin)
constexpr int kCandCap = 2048;    // candidates held in LDS (more take the radix levels)
constexpr int kRankDirect = 128;  // candidates ranked directly (more are narrowed first)

// LDS of a selecting workgroup of NT threads.  The histogram doubles as the candidate buffer.
template <int NT>
struct SelLdsT {
    alignas(16) uint32_t hist[kBins + 4];  // + the spill bin of the value level
    uint64_t red64[NT / 64][2];
    uint32_t wsum[NT / 64];
    int bin, above, ncand;
    uint32_t kstar;
    int pstar;
};
using SelLds = SelLdsT<kSelThreads>;

// The float of an order key (inverse of order_key; -0 comes back as +0).
__device__ inline float key_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Bin search from the top over `nbins` LDS counters (256, 1024, 2048 or 4096): the bin where
// the count from the top reaches `need`, and the count strictly above it.  Thread t holds
// the contiguous bins [nbins - per*(t+1), nbins - per*t), read as 16-byte words.
template <int NT = kSelThreads>
__device__ inline void find_bin(const uint32_t *hist, int nbins, int need, uint32_t *wsum, int *out_bin,
                                int *out_above) {
    if (threadIdx.x == 0) {
        *out_bin = 0;
        *out_above = 0;
    }
    const int per = nbins / NT;
    const int lo = nbins - per * ((int)threadIdx.x + 1);
    uint32_t cnt[16];
    if (per == 1) {
        cnt[0] = hist[lo];
#pragma unroll
        for (int j = 1; j < 16; ++j) cnt[j] = 0u;
    } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const u32x4 x = 4 * v < per ? *reinterpret_cast<const u32x4 *>(hist + lo + 4 * v) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 4; ++e) cnt[4 * v + e] = x[e];
        }
    }
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) mine += cnt[j];
    uint32_t total;
    const uint32_t incl = wg_scan<NT / 64, false>(mine, wsum, &total);  // (a barrier closes this function)
    int above = (int)(incl - mine);
    if (above < need && need <= (int)incl) {
        int found = 0, fa = 0;
        bool done = false;
#pragma unroll
        for (int j = 15; j >= 0; --j) {
            if (!done && j < per && above + (int)cnt[j] >= need) {
                found = j;
                fa = above;
                done = true;
            }
            if (j < per) above += (int)cnt[j];
        }
        *out_bin = lo + found;
        *out_above = fa;
    }
    __syncthreads();
}

// Linear value bin between the team's min and max: monotonic in the value, so every
// score in a higher bin is larger than every score in a lower one.
// fma is monotone in v for scale >= 0, so bins are ordered like the scores; the clamp
// by max / min also sends a NaN (an infinite score times a zero scale) to bin 0.
__device__ inline int value_bin(float v, float scale, float bias) {
    return (int)fminf(fmaxf(fmaf(v, scale, bias), 0.f), (float)(kVBins - 1));
}
// The same over nbins bins (nbins <= kVBins).
__device__ inline int value_bin_n(float v, float scale, float bias, int nbins) {
    return (int)fminf(fmaxf(fmaf(v, scale, bias), 0.f), (float)(nbins - 1));
}

// Exact resolution by radix levels over a row's scores (heavy ties): among the scores in
// value bin vb, the need-th by (order key desc, position asc).  Threads take contiguous
// position ranges so the final tie cut can walk positions in order; score(t) reads the
// score at position t.
template <int NT, typename Score>
__device__ inline void radix_resolve(SelLdsT<NT> &sm, Score score, int nvis, float scale, float bias, int vb,
                                     int need, int nbins = kVBins) {
    const int per = (nvis + NT - 1) / NT;
    const int t0 = threadIdx.x * per, t1 = min(t0 + per, nvis);
    auto in_bin = [&](float v) { return value_bin_n(v, scale, bias, nbins) == vb; };
    uint32_t prefix = 0u, pmask = 0u;
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int lv = 0; lv < 3; ++lv) {
        const int nb = 1 << widths[lv];
        for (int j = threadIdx.x; j < kBins; j += NT) sm.hist[j] = 0u;
        __syncthreads();
        for (int t = t0; t < t1; ++t) {
            const float v = score(t);
            const uint32_t k = order_key(v);
            if (in_bin(v) && (k & pmask) == prefix) atomicAdd(&sm.hist[(k >> shifts[lv]) & (nb - 1)], 1u);
        }
        __syncthreads();
        find_bin<NT>(sm.hist, nb < NT ? NT : nb, need, sm.wsum, &sm.bin, &sm.above);
        prefix |= (uint32_t)sm.bin << shifts[lv];
        pmask |= (uint32_t)(nb - 1) << shifts[lv];
        need -= sm.above;
        __syncthreads();
    }
    // equal keys: the need-th in position order
    uint32_t eq = 0;
    for (int t = t0; t < t1; ++t) {
        const float v = score(t);
        eq += in_bin(v) && order_key(v) == prefix;
    }
    uint32_t total;
    const uint32_t incl = wg_scan<NT / 64>(eq, sm.wsum, &total);
    int before = (int)(incl - eq);
    if (before < need && need <= (int)incl) {
        for (int t = t0; t < t1; ++t) {
            const float v = score(t);
            if (in_bin(v) && order_key(v) == prefix && ++before == need) {
                sm.pstar = t;
                break;
            }
        }
    }
    if (threadIdx.x == 0) sm.kstar = prefix;
    __syncthreads();
}

// Narrows the candidates cand[0..cnt) (distinct (key, position) composites) while more
// than kRankDirect remain: an NB-bin histogram of the candidates over their own
// [min, max] range (a monotone map, so bins are ordered like the composites), the bin
// where the count from the top reaches need, and only that bin's candidates kept; need
// becomes the rank within them.  Clustered scores put hundreds of candidates into one
// value bin, and the direct rank costs cnt^2 comparisons.  cand holds at most CAP
// candidates; h2 is NB words of LDS (NB a multiple of 4 NT).
template <int NT, int CAP = kCandCap, int NB = kBins>
__device__ inline void refine_candidates(uint64_t *cand, int &cnt, int &need, uint32_t *h2, SelLdsT<NT> &sm) {
    constexpr int kPer = CAP / NT;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int round = 0; round < 8 && cnt > kRankDirect; ++round) {
        uint64_t cv[kPer];
        uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int j = tid + NT * r;
            cv[r] = j < cnt ? cand[j] : 0ull;
            if (j < cnt) {
                lo = min(lo, cv[r]);
                hi = max(hi, cv[r]);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const uint64_t l2 = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(lo >> 32), off) << 32) |
                                (uint32_t)__shfl_xor((int)(uint32_t)lo, off);
            const uint64_t h2v = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(hi >> 32), off) << 32) |
                                 (uint32_t)__shfl_xor((int)(uint32_t)hi, off);
            lo = min(lo, l2);
            hi = max(hi, h2v);
        }
        if (lane == 0) {
            sm.red64[wave][0] = lo;
            sm.red64[wave][1] = hi;
        }
        for (int j = tid; j < NB / 4; j += NT) reinterpret_cast<u32x4 *>(h2)[j] = u32x4{0u, 0u, 0u, 0u};
        __syncthreads();
        lo = ~0ull;
        hi = 0ull;
        for (int w = 0; w < NT / 64; ++w) {
            lo = min(lo, sm.red64[w][0]);
            hi = max(hi, sm.red64[w][1]);
        }
        const float s2 = (float)(NB - 1) / (float)(hi - lo);
        auto bin_of = [&](uint64_t v) { return min(NB - 1, (int)((float)(v - lo) * s2)); };
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            if (tid + NT * r < cnt) atomicAdd(&h2[bin_of(cv[r])], 1u);
        __syncthreads();
        find_bin<NT>(h2, NB, need, sm.wsum, &sm.bin, &sm.above);
        const int sb = sm.bin;
        need -= sm.above;
        if (tid == 0) sm.ncand = 0;
        __syncthreads();
#pragma unroll
        for (int r = 0; r < kPer; ++r)
            if (tid + NT * r < cnt && bin_of(cv[r]) == sb) cand[atomicAdd(&sm.ncand, 1)] = cv[r];
        __syncthreads();
        cnt = sm.ncand;
    }
}


// The direct rank: the candidate with need-1 ahead of it in (key desc, position asc) is
// the cut; it lands in sm.kstar / sm.pstar.
template <int NT>
__device__ inline void rank_candidates(const uint64_t *cand, int cnt, int need, SelLdsT<NT> &sm) {
    for (int j = threadIdx.x; j < cnt; j += NT) {
        const uint64_t cj = cand[j];
        int rank = 0;
        int o = 0;
        for (; o + 8 <= cnt; o += 8) {
            const u32x4 *p4 = reinterpret_cast<const u32x4 *>(cand + o);
            u32x4 x[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) x[v] = p4[v];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                rank += ((uint64_t)x[v][1] << 32 | x[v][0]) > cj;
                rank += ((uint64_t)x[v][3] << 32 | x[v][2]) > cj;
            }
        }
        for (; o < cnt; ++o) rank += cand[o] > cj;
        if (rank == need - 1) {
            sm.kstar = (uint32_t)(cj >> 32);
            sm.pstar = (int)~(uint32_t)cj;
        }
    }
    __syncthreads();
}

}  // namespace lit
