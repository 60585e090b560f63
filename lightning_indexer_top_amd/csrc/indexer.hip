// indexer.hip -- lightning-indexer scores on gfx950 MX-scaled fp8 MFMA.
//
// What is computed (DeepSeek-V4.1-Flash-NVFP4 inference/model.py, Indexer.forward;
// DeepSeek-V3.2-Exp inference/model.py, fp8_index):
//   score[b,i,t] = sum_h w[b,i,h] * relu( qhat[b,i,h,:] . khat[b,t,:] )
// with e4m3 (or fp4 e2m1, V4.1's own indexer precision) operands carrying one ue8m0
// scale per 32 values, and -inf for the rows a query cannot see yet
// (t >= (start_pos+i+1)/ratio).
//
// Mapping onto the chip.  The q.k contraction of 16 heads against 16 keys is one
// V_MFMA_SCALE_F32_16X16X128_F8F6F4: A = 16 query heads (rows), B = 16 keys
// (columns), K = 128 head dims, with the ue8m0 scales applied by the instruction.
// Measured operand layout (probed on gfx950): lane l = 16*g + c holds row/column c;
// its bytes 0-15 are K = 16g..16g+15 and bytes 16-31 are K = 64+16g..64+16g+15; the
// scale byte lane group g supplies covers K block 32g..32g+31.  So a lane loads row
// bytes [16g, 16g+16) and [64+16g, 64+16g+16) and the scale of block g -- memory
// order is K order.  Di = 64 uses only the low half (K 0..63, the high half zero).
// fp4 codes take the same instruction with 16 bytes (32 codes, one scale block) per
// lane: a 128-dim fp4 key is 64 bytes, one load per lane.
// C comes back as lane (g, c), register r = head 4g+r, key c; the ReLU, the head
// weights and the sum over the lane's 4 heads run in registers, and two cross-lane
// adds finish the head sum.  Four key tiles are scored together so that their MFMAs
// overlap and the cross-lane head sum of all four takes three exchanges.
//
// The key stream is the HBM-bound part at decode: every wave owns 16*U consecutive
// keys of one sequence, issues all their loads before the first MFMA, and writes 16*U
// fp32 scores.  Query heads stay in VGPRs.  For several queries per sequence
// (chunked prefill) a wave scores QG queries against the same keys, so the keys are
// read once per QG queries.
#include "tile_ops.h"

namespace lit {

namespace {

constexpr int kWaves = 4;  // waves per workgroup
constexpr int kU = 4;      // 16-key tiles per wave

template <int DI, int FMT, int HT, int QG>
__global__ __launch_bounds__(kWaves * 64) void indexer_scores_kernel(IndexerArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;

    const int n_groups = (a.S + QG - 1) / QG;
    const int b = blockIdx.y / n_groups;
    const int i0 = (blockIdx.y % n_groups) * QG;
    const int t0 = (blockIdx.x * kWaves + wave) * (16 * kU);
    if (t0 >= a.T) return;
    const int i_last = min(i0 + QG - 1, a.S - 1);
    const int vis_max = min(a.T, (a.start_pos + i_last + 1) / a.ratio);
    const size_t bs0 = (size_t)b * a.S;

    if (t0 >= vis_max) {  // nothing visible to any query of the group in this chunk
        if (g == 0) {
            for (int qq = 0; qq < QG; ++qq) {
                const int i = i0 + qq;
                if (i >= a.S) break;
                float *dst = a.scores + (bs0 + i) * a.ld;
                for (int u = 0; u < kU; ++u) {
                    const int t = t0 + 16 * u + c;
                    if (t < a.T && !a.visible_only) dst[t] = -INFINITY;
                }
            }
        }
        return;
    }

    // Keys first: they are the long-latency stream.
    IdxKeys kb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
        kb[u] = load_idx_keys<DI, FMT>(a, (size_t)b * a.T_cap + min(t0 + 16 * u + c, a.T - 1), g);

    IdxQuery<DI, FMT, HT> qs[QG];
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
        const int i = i0 + qq;
        load_idx_query<DI, FMT, HT>(qs[qq], a, bs0 + (i < a.S ? i : 0), i < a.S, g, c);
    }

    static_assert(kU == 4, "idx_score4 scores four tiles");
    const int t = t0 + 16 * g + c;  // lane group g receives tile g's scores
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
        const float s = idx_score4<DI, FMT, HT>(qs[qq], kb, g);
        const int i = i0 + qq;
        if (i < a.S && t < a.T) {
            const int vis = (a.start_pos + i + 1) / a.ratio;
            if (t < vis || !a.visible_only) a.scores[(bs0 + i) * a.ld + t] = t < vis ? s : -INFINITY;
        }
    }
}

// Many queries per sequence (chunked prefill): each wave keeps its 64 keys in VGPRs and
// streams kQB queries past them, the next query's operands loading while the current
// one is scored (two alternating buffers), so the key loads and the launch cost are
// spread over kQB queries instead of QG.  The four waves of a workgroup take 256
// consecutive keys and the same queries (their query loads coalesce in the cache).  16
// queries a block keep the staged form's LDS at 17.5 KB for 16 index heads of 64 dims, so
// more workgroups share a compute unit (measured at prefill-16k: 94 us against 108 us
// with 32 queries a block).
constexpr int kQB = 16;

template <int DI, int FMT, int HT>
__global__ __launch_bounds__(kWaves * 64) void indexer_scores_multi_kernel(IndexerArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;

    const int n_groups = (a.S + kQB - 1) / kQB;
    const int b = blockIdx.y / n_groups;
    const int i0 = (blockIdx.y % n_groups) * kQB;
    const int i1 = min(i0 + kQB, a.S);
    const int t0 = (blockIdx.x * kWaves + wave) * (16 * kU);
    if (t0 >= a.T) return;
    const int vis_max = min(a.T, (a.start_pos + i1) / a.ratio);
    const size_t bs0 = (size_t)b * a.S;
    const int t = t0 + 16 * g + c;  // lane group g receives tile g's scores

    if (t0 >= vis_max) {  // nothing visible to any query of the group in these keys
        if (g == 0)
            for (int i = i0; i < i1; ++i)
                for (int u = 0; u < kU; ++u) {
                    const int tt = t0 + 16 * u + c;
                    if (tt < a.T && !a.visible_only) a.scores[(bs0 + i) * a.ld + tt] = -INFINITY;
                }
        return;
    }

    IdxKeys kb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
        kb[u] = load_idx_keys<DI, FMT>(a, (size_t)b * a.T_cap + min(t0 + 16 * u + c, a.T - 1), g);

    static_assert(kU == 4, "idx_score4 scores four tiles");
    auto finish = [&](int i, float s) {
        if (t < a.T) {
            const int vis = (a.start_pos + i + 1) / a.ratio;
            if (t < vis || !a.visible_only) a.scores[(bs0 + i) * a.ld + t] = t < vis ? s : -INFINITY;
        }
    };
    IdxQuery<DI, FMT, HT> qa, qb;
    load_idx_query<DI, FMT, HT>(qa, a, bs0 + i0, true, g, c);
    for (int i = i0; i < i1; i += 2) {
        const bool second = i + 1 < i1;
        load_idx_query<DI, FMT, HT>(qb, a, bs0 + (second ? i + 1 : i), true, g, c);
        finish(i, idx_score4<DI, FMT, HT>(qa, kb, g));
        if (i + 2 < i1) load_idx_query<DI, FMT, HT>(qa, a, bs0 + i + 2, true, g, c);
        if (second) finish(i + 1, idx_score4<DI, FMT, HT>(qb, kb, g));
    }
}

// The same with the block's kQB queries staged in LDS first: the 256 threads copy their
// codes, scale bytes and head weights once (coalesced 16-byte loads), and every wave then
// reads its query operands from LDS, so the per-query latency is an LDS read instead of an
// L2 round trip.  For index heads small enough that kQB queries fit (HT*16 heads of
// idx_row_bytes + DI/32 + 4 bytes each, at most 2304 bytes a query).
template <int DI, int FMT, int HT>
constexpr int staged_query_bytes() {
    return HT * 16 * (idx_row_bytes(DI, FMT) + DI / 32 + 4);
}

template <int DI, int FMT, int HT>
__global__ __launch_bounds__(kWaves * 64) void indexer_scores_staged_kernel(IndexerArgs a) {
    constexpr int NH = HT * 16;
    constexpr int E = idx_row_bytes(DI, FMT);
    constexpr int NB = DI / 32;
    __shared__ __attribute__((aligned(16))) uint8_t qc[kQB][NH * E];   // codes
    __shared__ __attribute__((aligned(16))) float qw[kQB][NH];         // head weights
    __shared__ uint8_t qs[kQB][NH * NB];                               // scale bytes
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int c = lane & 15;

    const int n_groups = (a.S + kQB - 1) / kQB;
    const int b = blockIdx.y / n_groups;
    const int i0 = (blockIdx.y % n_groups) * kQB;
    const int i1 = min(i0 + kQB, a.S);
    const int nq = i1 - i0;
    const int tb0 = blockIdx.x * kWaves * 16 * kU;  // the block's first key
    if (tb0 >= a.T) return;
    const size_t bs0 = (size_t)b * a.S;

    // stage the block's queries (a whole workgroup returns together above, so every
    // thread reaches the barrier)
    {
        const uint8_t *src = a.q8 + (bs0 + i0) * NH * E;
        const int n16 = nq * NH * E / 16;
        for (int j = threadIdx.x; j < n16; j += kWaves * 64)
            reinterpret_cast<u32x4 *>(&qc[0][0])[j] = reinterpret_cast<const u32x4 *>(src)[j];
        const float *wsrc = a.w + (bs0 + i0) * NH;
        for (int j = threadIdx.x; j < nq * NH; j += kWaves * 64) (&qw[0][0])[j] = wsrc[j];
        const uint8_t *ssrc = a.q_sc + (bs0 + i0) * NH * NB;
        for (int j = threadIdx.x; j < nq * NH * NB; j += kWaves * 64) (&qs[0][0])[j] = ssrc[j];
    }
    __syncthreads();

    const int t0 = tb0 + wave * (16 * kU);
    if (t0 >= a.T) return;
    const int vis_max = min(a.T, (a.start_pos + i1) / a.ratio);
    const int t = t0 + 16 * g + c;  // lane group g receives tile g's scores
    if (t0 >= vis_max) {  // nothing visible to any query of the block in these keys
        if (g == 0)
            for (int i = i0; i < i1; ++i)
                for (int u = 0; u < kU; ++u) {
                    const int tt = t0 + 16 * u + c;
                    if (tt < a.T && !a.visible_only) a.scores[(bs0 + i) * a.ld + tt] = -INFINITY;
                }
        return;
    }

    IdxKeys kb[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
        kb[u] = load_idx_keys<DI, FMT>(a, (size_t)b * a.T_cap + min(t0 + 16 * u + c, a.T - 1), g);

    static_assert(kU == 4, "idx_score4 scores four tiles");
    auto load_q = [&](IdxQuery<DI, FMT, HT> &q, int qi) {
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const int h = 16 * ht + c;
            q.a[ht] = mx_operand<DI, FMT>(&qc[qi][h * E], g);
            q.s[ht] = g < NB ? (int)qs[qi][h * NB + g] : 127;
#pragma unroll
            for (int r = 0; r < 4; ++r) q.w[ht][r] = qw[qi][16 * ht + 4 * g + r];
        }
    };
    for (int i = i0; i < i1; ++i) {
        IdxQuery<DI, FMT, HT> qv;
        load_q(qv, i - i0);
        const float s = idx_score4<DI, FMT, HT>(qv, kb, g);
        if (t < a.T) {
            const int vis = (a.start_pos + i + 1) / a.ratio;
            if (t < vis || !a.visible_only) a.scores[(bs0 + i) * a.ld + t] = t < vis ? s : -INFINITY;
        }
    }
}

// 16 index heads of 64 e4m3 dims (the chunked-prefill shape): two queries' heads against 32
// keys per V_MFMA_SCALE_F32_32X32X64_F8F6F4 (operand layout and epilogue in tile_ops.h).
// Seven waves a SIMD (at most 72 VGPRs, no spill; the unconstrained build takes 77 and six
// waves): the kernel issues VALU about 60% of its time and waits on memory the rest, so one
// more wave per SIMD hides more of the waits.
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(7))) void indexer_scores_mx32_kernel(IndexerArgs a) {
    constexpr int NH = 16, E = 64, NB = 2;
    __shared__ __attribute__((aligned(16))) uint8_t qc[kQB][NH * E];   // codes
    __shared__ __attribute__((aligned(16))) float qw[kQB][NH];         // head weights
    __shared__ uint8_t qs[kQB][NH * NB];                               // scale bytes
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 5;
    const int c = lane & 31;

    const int n_groups = (a.S + kQB - 1) / kQB;
    const int b = blockIdx.y / n_groups;
    const int i0 = (blockIdx.y % n_groups) * kQB;
    const int i1 = min(i0 + kQB, a.S);
    const int nq = i1 - i0;
    const int tb0 = blockIdx.x * kWaves * 64;  // the block's first key
    if (tb0 >= a.T) return;
    const size_t bs0 = (size_t)b * a.S;

    // this wave's 64 keys (columns c of two 32-key operands), requested before the query
    // staging so that the two round trips overlap (the barrier below waits for both)
    const int t0 = tb0 + wave * 64;
    const int vis_max = min(a.T, (a.start_pos + i1) / a.ratio);
    i32x8 kb[2] = {};
    int ks[2] = {127, 127};
    if (t0 < vis_max) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const size_t row = (size_t)b * a.T_cap + min(t0 + 32 * m + c, a.T - 1);
            kb[m] = mx32_operand(a.k8 + row * E, g);
            ks[m] = a.k_sc[row * NB + g];
        }
    }

    // stage the block's queries (a whole workgroup returns together above, so every
    // thread reaches the barrier)
    {
        const uint8_t *src = a.q8 + (bs0 + i0) * NH * E;
        const int n16 = nq * NH * E / 16;
        for (int j = threadIdx.x; j < n16; j += kWaves * 64)
            reinterpret_cast<u32x4 *>(&qc[0][0])[j] = reinterpret_cast<const u32x4 *>(src)[j];
        const float *wsrc = a.w + (bs0 + i0) * NH;
        for (int j = threadIdx.x; j < nq * NH; j += kWaves * 64) (&qw[0][0])[j] = wsrc[j];
        const uint8_t *ssrc = a.q_sc + (bs0 + i0) * NH * NB;
        for (int j = threadIdx.x; j < nq * NH * NB; j += kWaves * 64) (&qs[0][0])[j] = ssrc[j];
    }
    __syncthreads();

    if (t0 >= a.T) return;
    if (t0 >= vis_max) {  // nothing visible to any query of the block in these keys
        const int tt = t0 + lane;
        if (tt < a.T && !a.visible_only)
            for (int i = i0; i < i1; ++i) a.scores[(bs0 + i) * a.ld + tt] = -INFINITY;
        return;
    }
    const int h = c & 15;
    for (int qa = 0; qa < nq; qa += 2) {
        // rows 0-15: query qa's heads, rows 16-31: query qa+1's (query qa again past the
        // block's end; that half's scores are not stored)
        const int qb = min(qa + 1, nq - 1);
        const int qr = c < 16 ? qa : qb;
        const i32x8 av = mx32_operand(&qc[qr][h * E], g);
        const int as = qs[qr][h * NB + g];
        const Mx32Weights wt = mx32_weights(&qw[qa][0], &qw[qb][0], g);
        f32x16 acc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m)
            acc[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, kb[m], f32x16{}, 0, 0, 0, as, 0, ks[m]);
        float sc[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) sc[m] = mx32_pair_scores(acc[m], wt);
        // the two queries' visible counts on the scalar unit (a lane-dependent numerator would
        // make this a vector division)
        const int va = __builtin_amdgcn_readfirstlane((a.start_pos + i0 + qa + 1) / a.ratio);
        const int vb = __builtin_amdgcn_readfirstlane((a.start_pos + i0 + qa + 2) / a.ratio);
        if (qa + g < nq) {
            const int vis = g ? vb : va;
            float *dst = a.scores + (bs0 + i0 + qa + g) * a.ld;
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                const int t = t0 + 32 * m + c;
                if (t < (a.visible_only ? vis : a.T)) dst[t] = t < vis ? sc[m] : -INFINITY;
            }
        }
    }
}

template <int DI, int FMT, int HT>
hipError_t launch_staged(const IndexerArgs &a, hipStream_t stream) {
    const int keys_per_block = kWaves * 16 * kU;
    dim3 grid((a.T + keys_per_block - 1) / keys_per_block, a.B * ((a.S + kQB - 1) / kQB));
    hipLaunchKernelGGL((indexer_scores_staged_kernel<DI, FMT, HT>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <int DI, int FMT, int HT>
hipError_t launch_multi(const IndexerArgs &a, hipStream_t stream) {
    if constexpr (DI == 64 && FMT == kFmtE4M3 && HT == 1) {
        dim3 grid((a.T + kWaves * 64 - 1) / (kWaves * 64), a.B * ((a.S + kQB - 1) / kQB));
        hipLaunchKernelGGL(indexer_scores_mx32_kernel, grid, dim3(kWaves * 64), 0, stream, a);
        return hipGetLastError();
    }
    if constexpr (staged_query_bytes<DI, FMT, HT>() <= 2304) return launch_staged<DI, FMT, HT>(a, stream);
    const int keys_per_block = kWaves * 16 * kU;
    dim3 grid((a.T + keys_per_block - 1) / keys_per_block, a.B * ((a.S + kQB - 1) / kQB));
    hipLaunchKernelGGL((indexer_scores_multi_kernel<DI, FMT, HT>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <int DI, int FMT, int HT, int QG>
hipError_t launch_cfg(const IndexerArgs &a, hipStream_t stream) {
    const int keys_per_block = kWaves * 16 * kU;
    dim3 grid((a.T + keys_per_block - 1) / keys_per_block, a.B * ((a.S + QG - 1) / QG));
    hipLaunchKernelGGL((indexer_scores_kernel<DI, FMT, HT, QG>), grid, dim3(kWaves * 64), 0, stream, a);
    return hipGetLastError();
}

template <int DI, int FMT>
hipError_t launch_di(const IndexerArgs &a, hipStream_t stream) {
    const int HT = a.Hi / 16;
    const bool multi = a.S > 1;
    if (a.S >= kQB) {
        switch (HT) {
            case 1: return launch_multi<DI, FMT, 1>(a, stream);
            case 2: return launch_multi<DI, FMT, 2>(a, stream);
            case 3: return launch_multi<DI, FMT, 3>(a, stream);
            case 4: return launch_multi<DI, FMT, 4>(a, stream);
            default: return hipErrorInvalidValue;
        }
    }
    switch (HT) {
        case 1: return multi ? launch_cfg<DI, FMT, 1, 4>(a, stream) : launch_cfg<DI, FMT, 1, 1>(a, stream);
        case 2: return multi ? launch_cfg<DI, FMT, 2, 2>(a, stream) : launch_cfg<DI, FMT, 2, 1>(a, stream);
        case 3: return launch_cfg<DI, FMT, 3, 1>(a, stream);
        case 4: return launch_cfg<DI, FMT, 4, 1>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_indexer_scores(const IndexerArgs &a, hipStream_t stream) {
    if (a.T <= 0 || a.B <= 0 || a.S <= 0) return hipSuccess;
    if (a.fmt == kFmtE2M1) {
        if (a.Di == 64) return launch_di<64, kFmtE2M1>(a, stream);
        if (a.Di == 128) return launch_di<128, kFmtE2M1>(a, stream);
        return hipErrorInvalidValue;
    }
    if (a.Di == 64) return launch_di<64, kFmtE4M3>(a, stream);
    if (a.Di == 128) return launch_di<128, kFmtE4M3>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace lit
