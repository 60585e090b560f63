// tile_ops.h -- wave-level building blocks shared by the standalone kernels and the
// fused decode kernel: the MX-scaled fp8 indexer tile, the 32-row gather-attention
// tile with its online softmax, and workgroup scans.
#pragma once

#include "lit_internal.h"

namespace lit {

// Orders this wave's earlier LDS writes before its later LDS reads (the lanes of a wave
// exchange data through a wave-private LDS region; no workgroup barrier is involved).
__device__ inline void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Cross-lane exchanges without LDS traffic.  V_PERMLANE16_SWAP / V_PERMLANE32_SWAP swap a
// register's odd 16-lane rows with another's even rows (its upper 32 lanes with another's
// lower 32).  Swapping x with itself leaves, in lane i, x of lane i and of lane i ^ 16
// (i ^ 32) in the two results: the first holds the partner's value in lanes with bit 4
// (bit 5) set, the second in the others.  The 2-element results are bit-cast whole.
__device__ inline uint64_t swap16_pair(uint32_t x) {
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_permlane16_swap(x, x, false, false));
}
__device__ inline uint64_t swap32_pair(uint32_t x) {
    return __builtin_bit_cast(uint64_t, __builtin_amdgcn_permlane32_swap(x, x, false, false));
}
// Max / sum over the four lanes i, i^16, i^32, i^48 (every one of them gets it).
__device__ inline float group4_max(float x) {
    uint64_t p = swap16_pair(__float_as_uint(x));
    x = fmaxf(__uint_as_float((uint32_t)p), __uint_as_float((uint32_t)(p >> 32)));
    p = swap32_pair(__float_as_uint(x));
    return fmaxf(__uint_as_float((uint32_t)p), __uint_as_float((uint32_t)(p >> 32)));
}
__device__ inline float group4_sum(float x) {
    uint64_t p = swap16_pair(__float_as_uint(x));
    x = __uint_as_float((uint32_t)p) + __uint_as_float((uint32_t)(p >> 32));
    p = swap32_pair(__float_as_uint(x));
    return __uint_as_float((uint32_t)p) + __uint_as_float((uint32_t)(p >> 32));
}
// Reduction over the 64 lanes of a wave with a commutative, associative op on 32-bit
// values, every lane getting the result: quad permutations and the mirrors within 8 and 16
// lanes (DPP), then the two swaps.  Every lane of the wave must be active.
template <typename Op>
__device__ inline uint32_t wave_reduce(uint32_t v, Op op) {
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));   // quad_perm 1,0,3,2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));   // quad_perm 2,3,0,1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xf, 0xf, false));  // row_half_mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xf, 0xf, false));  // row_mirror
    uint64_t p = swap16_pair(v);
    v = op((uint32_t)p, (uint32_t)(p >> 32));
    p = swap32_pair(v);
    return op((uint32_t)p, (uint32_t)(p >> 32));
}
__device__ inline uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce(v, [](uint32_t x, uint32_t y) { return max(x, y); });
}
__device__ inline uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce(v, [](uint32_t x, uint32_t y) { return min(x, y); });
}
__device__ inline uint32_t wave_sum_u32(uint32_t v) {
    return wave_reduce(v, [](uint32_t x, uint32_t y) { return x + y; });
}
__device__ inline float wave_max_f(float v) {
    return __uint_as_float(wave_reduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
    }));
}
__device__ inline float wave_min_f(float v) {
    return __uint_as_float(wave_reduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(fminf(__uint_as_float(x), __uint_as_float(y)));
    }));
}
__device__ inline float wave_sum_f(float v) {
    return __uint_as_float(wave_reduce(__float_as_uint(v), [](uint32_t x, uint32_t y) {
        return __float_as_uint(__uint_as_float(x) + __uint_as_float(y));
    }));
}

// ---------------------------------------------------------------------------
// Indexer tile (V_MFMA_SCALE_F32_16X16X128_F8F6F4).
//
// Operand layouts measured on gfx950, lane l = 16g + c holding row/column c:
//   e4m3: bytes 0-15 are K = 16g..16g+15, bytes 16-31 are K = 64+16g..64+16g+15, and
//         the scale byte lane group g supplies covers K block 32g..32g+31.  A lane
//         loads row bytes [16g, 16g+16) and [64+16g, 64+16g+16): memory order is K
//         order.  A 64-dim row uses only the low half (K 0..63).
//   e2m1: the first 4 registers are K = 32g..32g+31 (two codes a byte), with the
//         scale of block g.  A lane loads row bytes [16g, 16g+16) -- one 16-byte load
//         per key -- and a 64-dim row (32 bytes) fills lane groups 0 and 1, the other
//         two carrying zeros.
// C comes back as lane (g, c), register r = A row 4g+r, B column c.
// ---------------------------------------------------------------------------
template <int DI, int FMT>
__device__ inline i32x8 mx_operand(const uint8_t *row, int g) {
    i32x8 v;
    if constexpr (FMT == kFmtE2M1) {
        // a 64-dim row: lane groups 2 and 3 re-read group 0 and 1's bytes (in bounds)
        // and zero them, so no lane's load is conditional
        const u32x4 x = *reinterpret_cast<const u32x4 *>(row + 16 * (DI == 128 ? g : (g & 1)));
        const bool live = DI == 128 || g < 2;
        v[0] = live ? (int)x[0] : 0; v[1] = live ? (int)x[1] : 0;
        v[2] = live ? (int)x[2] : 0; v[3] = live ? (int)x[3] : 0;
        v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
    } else {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(row + 16 * g);
        u32x4 hi = {0u, 0u, 0u, 0u};
        if (DI == 128) hi = *reinterpret_cast<const u32x4 *>(row + 64 + 16 * g);
        v[0] = (int)lo[0]; v[1] = (int)lo[1]; v[2] = (int)lo[2]; v[3] = (int)lo[3];
        v[4] = (int)hi[0]; v[5] = (int)hi[1]; v[6] = (int)hi[2]; v[7] = (int)hi[3];
    }
    return v;
}

// One query's index heads as MFMA A operands: HT tiles of 16 heads, their scale bytes,
// and the head weights of the 4 C rows each lane receives.
template <int DI, int FMT, int HT>
struct IdxQuery {
    i32x8 a[HT];
    int s[HT];
    float w[HT][4];
};

template <int DI, int FMT, int HT>
__device__ inline void load_idx_query(IdxQuery<DI, FMT, HT> &q, const IndexerArgs &a, size_t qi,
                                      bool valid, int g, int c) {
    constexpr int NB = DI / 32;
    constexpr int E = idx_row_bytes(DI, FMT);
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const size_t head = qi * a.Hi + 16 * ht + c;
        if (valid) {
            q.a[ht] = mx_operand<DI, FMT>(a.q8 + head * E, g);
            q.s[ht] = g < NB ? (int)a.q_sc[head * NB + g] : 127;
        } else {
            q.a[ht] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            q.s[ht] = 127;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) q.w[ht][r] = valid ? a.w[qi * a.Hi + 16 * ht + 4 * g + r] : 0.f;
    }
}

// Keys of one 16-key tile as MFMA B operands (key c of the tile per lane column).
struct IdxKeys {
    i32x8 b;
    int s;
};

template <int DI, int FMT>
__device__ inline IdxKeys load_idx_keys(const IndexerArgs &a, size_t row, int g) {
    constexpr int NB = DI / 32;
    IdxKeys k;
    k.b = mx_operand<DI, FMT>(a.k8 + row * idx_row_bytes(DI, FMT), g);
    k.s = g < NB ? (int)a.k_sc[row * NB + g] : 127;
    return k;
}

// ReLU as an integer max on the float's bits: a negative float is a negative int, so
// one v_max_i32 (no NaN canonicalisation, which fmaxf costs under IEEE mode); -0 maps
// to +0.
__device__ inline float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ---------------------------------------------------------------------------
// 16 index heads of 64 e4m3 dims (the chunked-prefill indexer shape):
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 takes two queries' 16 heads as its 32 rows and 32 keys
// as its columns.  Its 64-deep K is exactly a head's dims, where the 16x16x128 form carries
// a zero half, so a query needs half the MFMA passes.  Operand layout, measured with an
// on-GPU probe: lane 32g + r holds row r, its bytes 0-15 belong to K block 0 and bytes
// 16-31 to K block 1, and lane group g supplies block g's scale; a lane therefore loads row
// bytes [16g, 16g+16) and [32+16g, 32+16g+16) and the row's scale byte g (the order of K
// within a block is the same for both operands, so it does not matter).  The result comes
// back as lane 32g + c, register 4i + r = row 8i + 4g + r, column c: rows 0-15 are the first
// query's heads.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ inline i32x8 mx32_operand(const uint8_t *row, int g) {
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(row + 16 * g);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(row + 32 + 16 * g);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// The head weights of the rows lane group g receives: heads 4g+r and 8+4g+r of each query.
struct Mx32Weights {
    f32x4 a0, a1, b0, b1;
};
__device__ inline Mx32Weights mx32_weights(const float *wa, const float *wb, int g) {
    Mx32Weights w;
    w.a0 = *reinterpret_cast<const f32x4 *>(wa + 4 * g);
    w.a1 = *reinterpret_cast<const f32x4 *>(wa + 8 + 4 * g);
    w.b0 = *reinterpret_cast<const f32x4 *>(wb + 4 * g);
    w.b1 = *reinterpret_cast<const f32x4 *>(wb + 8 + 4 * g);
    return w;
}

// The two queries' scores of one 32-key tile from its MFMA result: the head-weighted ReLU
// sum, query A's score of key c in lane c, query B's in lane 32 + c.  Lanes 32 apart hold
// the two halves of each query's heads: swapping the upper half of the A partials with the
// lower half of the B partials and adding finishes both sums.
__device__ inline float mx32_pair_scores(const f32x16 &acc, const Mx32Weights &w) {
    float sa = 0.f, sb = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        sa += w.a0[r] * relu_bits(acc[r]);
        sa += w.a1[r] * relu_bits(acc[4 + r]);
        sb += w.b0[r] * relu_bits(acc[8 + r]);
        sb += w.b1[r] * relu_bits(acc[12 + r]);
    }
    const uint64_t x = __builtin_bit_cast(
        uint64_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(sa), __float_as_uint(sb), false, false));
    return __uint_as_float((uint32_t)x) + __uint_as_float((uint32_t)(x >> 32));
}

// Scores of four 16-key tiles for one query.  All 4*HT MFMAs are issued first; each
// lane then holds, per tile, the head-weighted ReLU sum over its 4 heads of every head
// tile, and the sum over the four lane groups takes three lane swaps and three adds:
// across lanes 32 apart each lane keeps two tiles and sends two, across lanes 16 apart it
// keeps one and sends one.  Lane (g, c) returns the score of key c of tile g.
template <int DI, int FMT, int HT>
__device__ inline float idx_score4(const IdxQuery<DI, FMT, HT> &q, const IdxKeys (&k)[4], int g) {
    // operand type codes of the instruction: 0 = e4m3, 4 = e2m1
    constexpr int kType = FMT == kFmtE2M1 ? 4 : 0;
    f32x4 acc[4][HT];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
            acc[u][ht] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                q.a[ht], k[u].b, f32x4{0.f, 0.f, 0.f, 0.f}, kType, kType, 0, q.s[ht], 0, k[u].s);
    float part[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        part[u] = 0.f;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht)
#pragma unroll
            for (int r = 0; r < 4; ++r) part[u] += q.w[ht][r] * relu_bits(acc[u][ht][r]);
    }
    // Lane group g ends with tile g's scores.  Swapping the upper half of tile 0's partials
    // with the lower half of tile 2's (and 1 with 3) and adding puts the sum over lane
    // groups {0, 2} / {1, 3} of tile 0 (1) in lanes 0-31 and of tile 2 (3) in lanes 32-63;
    // swapping the odd 16-lane rows of the first sum with the even rows of the second and
    // adding completes tile g in row g.
    const uint64_t a = __builtin_bit_cast(
        uint64_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false));
    const uint64_t b = __builtin_bit_cast(
        uint64_t, __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false));
    const float k02 = __uint_as_float((uint32_t)a) + __uint_as_float((uint32_t)(a >> 32));
    const float k13 = __uint_as_float((uint32_t)b) + __uint_as_float((uint32_t)(b >> 32));
    const uint64_t c2 = __builtin_bit_cast(
        uint64_t, __builtin_amdgcn_permlane16_swap(__float_as_uint(k02), __float_as_uint(k13), false, false));
    return __uint_as_float((uint32_t)c2) + __uint_as_float((uint32_t)(c2 >> 32));
}

// ---------------------------------------------------------------------------
// Gather-attention tile (V_MFMA_F32_16X16X32_BF16), 16 heads.
//
// Logits: A = 16 gathered rows (lane (g, c): row c, dims 32s+8g..+7), B = Q^T (lane
// (g, c): head c, same dims) -> lane (g, h) holds head h's logits for rows 4g+r.  Two
// such halves give rows 4g..4g+3 and 16+4g..16+4g+3, which as bf16 are the B operand
// (P^T, k-slots in that row order) of O^T = V^T P^T; V^T comes from an LDS copy of
// the rows read column-wise with the same row order.  O^T lands as lane (g, h),
// register r = dim 16dt+4g+r of head h: every lane owns one head throughout.
// ---------------------------------------------------------------------------
template <int D>
struct AttnState {
    float m;  // running max of log2-domain logits of head c
    float l;  // this lane's share of the running normaliser
    f32x4 o[D / 16];
};

__device__ inline bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

template <int D>
__device__ inline void attn_init(AttnState<D> &st) {
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) st.o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
__device__ inline void load_q_operands(bf16x8 (&qb)[D / 32], const uint16_t *q, size_t bs, int g, int c) {
    const uint16_t *qrow = q + (bs * 16 + c) * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
        qb[s] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qrow + 32 * s + 8 * g));
}

// Loads of one tile's rows (issued early, consumed by attn_tile_compute).
template <int D>
struct AttnRows {
    u32x4 r[2][D / 32];
    uint64_t valid[2];
};

template <int D>
__device__ inline void attn_tile_load(AttnRows<D> &t, const uint16_t *rp0, const uint16_t *rp1, int g) {
    t.valid[0] = __ballot(rp0 != nullptr);
    t.valid[1] = __ballot(rp1 != nullptr);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        t.r[0][s] = rp0 ? *reinterpret_cast<const u32x4 *>(rp0 + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
        t.r[1][s] = rp1 ? *reinterpret_cast<const u32x4 *>(rp1 + 32 * s + 8 * g) : u32x4{0u, 0u, 0u, 0u};
    }
}

// The same loads from addresses that are always valid: a lane whose row is not part of
// the tile (v0 / v1 false) points at a stand-in row its wave attends anyway, so the data
// is finite and its probability 0 adds nothing.  Unconditional loads let the compiler
// leave them in flight where they are issued (a load under a branch is waited for at
// the join).
template <int D>
__device__ inline void attn_tile_load_rows(AttnRows<D> &t, const uint16_t *rp0, bool v0, const uint16_t *rp1,
                                           bool v1, int g) {
    t.valid[0] = __ballot(v0);
    t.valid[1] = __ballot(v1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        t.r[0][s] = *reinterpret_cast<const u32x4 *>(rp0 + 32 * s + 8 * g);
        t.r[1][s] = *reinterpret_cast<const u32x4 *>(rp1 + 32 * s + 8 * g);
    }
}

// Raw buffer loads.  A buffer resource covers `bytes` (< 2^31) from `base`; a load at an
// offset at or past that count returns zeros and touches no memory, so a lane without a
// row loads from offset kOffNone instead of branching around its load.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOffNone = 0x80000000u;
__device__ inline rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// One tile's rows from a bf16 source by buffer loads: lane (g, c) reads dims 32s+8g..+7
// of the rows at byte offsets off0 / off1 (kOffNone: no row, zeros).
template <int D>
__device__ inline void attn_tile_load_buf(AttnRows<D> &t, rsrc_t src, uint32_t off0, uint32_t off1, int g) {
    t.valid[0] = __ballot(off0 != kOffNone);
    t.valid[1] = __ballot(off1 != kOffNone);
    const uint32_t o0 = off0 + 16u * g, o1 = off1 + 16u * g;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        t.r[0][s] = __builtin_amdgcn_raw_buffer_load_b128(src, (int)(o0 + 64u * s), 0, 0);
        t.r[1][s] = __builtin_amdgcn_raw_buffer_load_b128(src, (int)(o1 + 64u * s), 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Quantised KV rows, dequantised on gather into the bf16 operand layout above (lane
// (g, c) holds dims 32s+8g..32s+8g+7 of its row for each s).
//   kKvE4M3: D e4m3 bytes a row, one ue8m0 scale byte per 32 dims.  A lane reads 8 code
//            bytes and the scale of block s per piece; V_CVT_SCALEF32_PK_BF16_FP8 applies
//            the scale (the instruction uses only the exponent of its f32 scale, which a
//            power of two is exactly; measured on gfx950).
//   kKvE2M1: D/2 bytes a row (two e2m1 codes a byte, element 2j low), one e4m3 scale byte
//            per 16 dims.  A lane reads 4 code bytes and the scale of group 2s + g/2.  The
//            e4m3 scale is no power of two, so the codes become f32 pairs, are multiplied
//            by the decoded scale, and the products -- exact in bf16: at most 6
//            significant bits, magnitudes within 2^-10 .. 2688 -- are truncated to bf16.
// Indexing a 2-element result of these conversion builtins gave the first element twice
// in this compiler; the results are therefore bit-cast whole.
// ---------------------------------------------------------------------------
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ inline float ue8m0_f32(uint32_t sb) {
    // 2^(sb-127); sb = 0 is the subnormal 2^-127
    return __uint_as_float(sb ? sb << 23 : 0x00400000u);
}

// Raw codes and scale byte of 8 dims (32s+8g..) of one row: loads only.
template <int D, int KF>
struct KvPiece {
    uint32_t w[KF == kKvE4M3 ? 2 : 1];
    uint32_t sb;
};

template <int D, int KF>
__device__ inline KvPiece<D, KF> kv_piece_load(const uint8_t *codes, const uint8_t *scales, size_t row, int s,
                                               int g) {
    KvPiece<D, KF> p;
    if constexpr (KF == kKvE4M3) {
        const u32x2 w = *reinterpret_cast<const u32x2 *>(codes + row * D + 32 * s + 8 * g);
        p.w[0] = w[0];
        p.w[1] = w[1];
        p.sb = scales[row * (D / 32) + s];
    } else {
        p.w[0] = *reinterpret_cast<const uint32_t *>(codes + row * (D / 2) + 16 * s + 4 * g);
        p.sb = scales[row * (D / 16) + 2 * s + (g >> 1)];
    }
    return p;
}

// The piece as 4 packed bf16 pairs (no loads).
template <int D, int KF>
__device__ inline u32x4 kv_piece_convert(const KvPiece<D, KF> &p) {
    u32x4 out;
    if constexpr (KF == kKvE4M3) {
        const float sf = ue8m0_f32(p.sb);
        out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p.w[0], sf, false));
        out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p.w[0], sf, true));
        out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p.w[1], sf, false));
        out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(p.w[1], sf, true));
    } else {
        const uint32_t w = p.w[0];
        const uint64_t sp = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(p.sb, 1.f, false));
        const float sf = __uint_as_float((uint32_t)sp);
        uint64_t pr[4];  // byte k's two codes as f32
        pr[0] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 0));
        pr[1] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 1));
        pr[2] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 2));
        pr[3] = __builtin_bit_cast(uint64_t, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.f, 3));
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = __float_as_uint(__uint_as_float((uint32_t)pr[k]) * sf);
            const uint32_t hi = __float_as_uint(__uint_as_float((uint32_t)(pr[k] >> 32)) * sf);
            out[k] = (lo >> 16) | (hi & 0xFFFF0000u);
        }
    }
    return out;
}

// 8 dims of row `row` (dims 32s+8g..) of a quantised source, as 4 packed bf16 pairs.
template <int D, int KF>
__device__ inline u32x4 kv_piece(const uint8_t *codes, const uint8_t *scales, size_t row, int s, int g) {
    return kv_piece_convert<D, KF>(kv_piece_load<D, KF>(codes, scales, row, s, g));
}

// A tile's quantised rows as loaded (converted when the tile is computed, so that the
// loads stay in flight meanwhile).
template <int D, int KF>
struct KvRows {
    KvPiece<D, KF> p[2][D / 32];
    uint64_t valid[2];
};

// Unconditional loads of rows row0 / row1 (a lane off the tile passes a stand-in row its
// wave attends anyway, with v0 / v1 false).
template <int D, int KF>
__device__ inline void kv_rows_load(KvRows<D, KF> &t, const uint8_t *codes, const uint8_t *scales, size_t row0,
                                    bool v0, size_t row1, bool v1, int g) {
    t.valid[0] = __ballot(v0);
    t.valid[1] = __ballot(v1);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        t.p[0][s] = kv_piece_load<D, KF>(codes, scales, row0, s, g);
        t.p[1][s] = kv_piece_load<D, KF>(codes, scales, row1, s, g);
    }
}

template <int D, int KF>
__device__ inline void kv_rows_convert(const KvRows<D, KF> &t, AttnRows<D> &r) {
    r.valid[0] = t.valid[0];
    r.valid[1] = t.valid[1];
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        r.r[0][s] = kv_piece_convert<D, KF>(t.p[0][s]);
        r.r[1][s] = kv_piece_convert<D, KF>(t.p[1][s]);
    }
}

// One tile's rows from a quantised source (row0 / row1 < 0: not part of the tile).
template <int D, int KF>
__device__ inline void kv_tile_load(AttnRows<D> &t, const uint8_t *codes, const uint8_t *scales, long row0,
                                    long row1, int g) {
    t.valid[0] = __ballot(row0 >= 0);
    t.valid[1] = __ballot(row1 >= 0);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
        t.r[0][s] = row0 >= 0 ? kv_piece<D, KF>(codes, scales, (size_t)row0, s, g) : u32x4{0u, 0u, 0u, 0u};
        t.r[1][s] = row1 >= 0 ? kv_piece<D, KF>(codes, scales, (size_t)row1, s, g) : u32x4{0u, 0u, 0u, 0u};
    }
}

// A tile's logits (two 16-row halves) and which of its rows are listed.
struct AttnLogits {
    f32x4 sc[2];
    uint64_t valid[2];
};

// First half of a 32-row tile: the logits S^T = rows x Q^T, and the rows copied into this
// wave's LDS region (`tile`, 32 rows x (D+4) bf16) for the V^T reads.  Once it returns, the
// row registers may take the next tile's loads.
template <int D>
__device__ inline AttnLogits attn_tile_logits(const bf16x8 (&qb)[D / 32], const AttnRows<D> &t, uint16_t *tile,
                                              int g, int c) {
    constexpr int KS = D / 32;
    constexpr int LD = D + 4;
    AttnLogits lg;
    lg.valid[0] = t.valid[0];
    lg.valid[1] = t.valid[1];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        lg.sc[half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            lg.sc[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(t.r[half][s]), qb[s], lg.sc[half], 0, 0, 0);
        uint16_t *dst = tile + (16 * half + c) * LD + 8 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            *reinterpret_cast<u32x2 *>(dst + 32 * s) = u32x2{t.r[half][s][0], t.r[half][s][1]};
            *reinterpret_cast<u32x2 *>(dst + 32 * s + 4) = u32x2{t.r[half][s][2], t.r[half][s][3]};
        }
    }
    return lg;
}

// ---------------------------------------------------------------------------
// Coalesced row gather, for a wave that walks many tiles.  In the MFMA operand layout 16
// neighbouring lanes hold 16 different rows, and the vector cache serves every lane's 16
// bytes as an access of its own (one access a lane a clock bounds such a gather).  Here
// piece e of a tile -- row e / P, 16-byte piece e % P, P = D / 8 -- is loaded by lane e % 64
// of load e / 64, so neighbouring lanes read consecutive bytes of one row; the pieces are
// staged into the wave's LDS tile (row stride LDR bf16) and the logits' row operands are
// read back from there.
// ---------------------------------------------------------------------------
template <int D>
struct RowPieces {
    static constexpr int P = D / 8;        // 16-byte pieces a row
    static constexpr int N = 32 * P / 64;  // loads a lane makes for a tile
    u32x4 v[N];
    uint64_t valid;                        // bit r: tile row r is listed
};

// A tile's loads.  Lane r < 32 passes row r's byte offset in `src` (kOffNone: no row,
// zeros are read).
template <int D>
__device__ inline void row_pieces_load(RowPieces<D> &rp, rsrc_t src, uint32_t off, int lane) {
    constexpr int P = RowPieces<D>::P;
    rp.valid = __ballot(lane < 32 && off != kOffNone);
#pragma unroll
    for (int j = 0; j < RowPieces<D>::N; ++j) {
        const int e = 64 * j + lane;
        const uint32_t o = (uint32_t)__shfl((int)off, e / P);
        rp.v[j] = __builtin_amdgcn_raw_buffer_load_b128(src, (int)(o + 16u * (uint32_t)(e % P)), 0, 0);
    }
}

// The pieces into the wave's LDS tile (rows LDR bf16 apart, LDR a multiple of 8).
template <int D, int LDR>
__device__ inline void row_pieces_stage(const RowPieces<D> &rp, uint16_t *tile, int lane) {
    constexpr int P = RowPieces<D>::P;
#pragma unroll
    for (int j = 0; j < RowPieces<D>::N; ++j) {
        const int e = 64 * j + lane;
        *reinterpret_cast<u32x4 *>(tile + (e / P) * LDR + 8 * (e % P)) = rp.v[j];
    }
}

// attn_tile_logits with the row operands read from the staged LDS tile.
template <int D, int LDR>
__device__ inline AttnLogits attn_tile_logits_lds(const bf16x8 (&qb)[D / 32], uint64_t valid, const uint16_t *tile,
                                                  int g, int c) {
    constexpr int KS = D / 32;
    AttnLogits lg;
    lg.valid[0] = valid & 0xffffull;
    lg.valid[1] = (valid >> 16) & 0xffffull;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint16_t *src = tile + (16 * half + c) * LDR + 8 * g;
        lg.sc[half] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            lg.sc[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(*reinterpret_cast<const u32x4 *>(src + 32 * s)), qb[s], lg.sc[half], 0, 0, 0);
    }
    return lg;
}

// Second half: online softmax of the logits and O^T += V^T P^T with V^T read transposed
// from the LDS copy (rows LD bf16 apart).  ndt = dv/16 output tiles are accumulated.  The V^T tiles are read in
// groups of RG (all D/16 at once by default: one LDS latency per tile; fewer keep fewer
// registers live).
template <int D, int RG = D / 16, int LD = D + 4>
__device__ inline void attn_tile_update(AttnState<D> &st, const AttnLogits &lg, uint16_t *tile, int ndt, float sl2,
                                        int g, int c) {
    constexpr int NT = D / 16;
    float x[8];
    float tmax = -INFINITY;
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool v = (lg.valid[half] >> (4 * g + r)) & 1ull;
            const float val = v ? lg.sc[half][r] * sl2 : -INFINITY;
            x[4 * half + r] = val;
            tmax = fmaxf(tmax, val);
        }
    tmax = group4_max(tmax);
    // Lazy rescale: the reference max st.m moves (and O and l are rescaled) only when the
    // tile's max exceeds it by more than 8 in log2 units, so probabilities stay <= 2^8
    // (exact in fp32, and within bf16 range for P) and most tiles skip the rescale.  The
    // final normalisation uses the same reference, so the result is unchanged in exact
    // arithmetic.  Exponents are <= 8 here; v_exp_f32 is used directly (its flush of
    // results below 2^-126 is far under the bf16 output's resolution).
    const bool move = tmax > st.m + 8.f;  // also the first finite tile (st.m = -inf)
    if (__ballot(move)) {
        const float alpha = !move ? 1.f : (st.m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.m - tmax));
        st.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) st.o[dt] *= alpha;
        st.m = move ? tmax : st.m;
    }
    bf16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const float pk = x[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(x[k] - st.m);
        psum += pk;
        pb[k] = (__bf16)pk;
    }
    st.l += psum;

    wave_lds_sync();  // the rows this wave wrote are readable by its other lanes
    // V^T operand by DS_READ_B64_TR_B16.  Within a 16-lane group, output lane i's element k
    // is element i&3 of the 8 bytes addressed by lane 4k + (i>>2) (probed on gfx950).  So lane
    // (g, c) addresses row 4g + (c>>2), dims 16dt + 4(c&3), and receives dim 16dt + c of rows
    // 4g..4g+3; a second read 16 rows down gives rows 16+4g..16+4g+3.
    lds_v4s *v0 = (lds_v4s *)((lds_u16 *)tile + (4 * g + (c >> 2)) * LD + 4 * (c & 3));
    lds_v4s *v1 = (lds_v4s *)((lds_u16 *)tile + (16 + 4 * g + (c >> 2)) * LD + 4 * (c & 3));
    // Every column tile of a group is read (all within the row's D dims) before the group's
    // first product, so the reads' LDS latency is paid once per group rather than once per
    // output tile; only the ndt tiles of dv are accumulated.
    static_assert(NT % RG == 0, "groups of whole column tiles");
#pragma unroll
    for (int d0 = 0; d0 < NT; d0 += RG) {
        v4s lo[RG], hi[RG];
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            lo[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(v0 + 4 * (d0 + u));
            hi[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(v1 + 4 * (d0 + u));
        }
#pragma unroll
        for (int u = 0; u < RG; ++u) {
            if (d0 + u < ndt) {
                const bf16x8 va = __builtin_bit_cast(
                    bf16x8, (v8s){lo[u][0], lo[u][1], lo[u][2], lo[u][3], hi[u][0], hi[u][1], hi[u][2], hi[u][3]});
                st.o[d0 + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, st.o[d0 + u], 0, 0, 0);
            }
        }
    }
    wave_lds_sync();  // reads done before the next tile overwrites the region
}

// One 32-row tile: logits, online softmax, P.V.
template <int D>
__device__ inline void attn_tile_compute(AttnState<D> &st, const bf16x8 (&qb)[D / 32], const AttnRows<D> &t,
                                         uint16_t *tile, int ndt, float sl2, int g, int c) {
    const AttnLogits lg = attn_tile_logits<D>(qb, t, tile, g, c);
    attn_tile_update<D>(st, lg, tile, ndt, sl2, g, c);
}

// Finish a wave: the normaliser summed over the wave (m is already uniform per head).
template <int D>
__device__ inline void attn_wave_total(AttnState<D> &st) {
    st.l = group4_sum(st.l);
}

// Row stride (floats) of the wave states in LDS: dv plus 4, so that the 16 heads of a wave
// start in different banks (dv itself is a multiple of 64 floats for the usual head sizes,
// which would put every head row in the same bank).
__host__ __device__ constexpr int attn_ow_ld(int dv) { return dv + 4; }

// A wave's finished state into LDS: ow [nwaves][16][attn_ow_ld(dv)] floats, wm / wl
// [nwaves][16].  Lane (g, c) holds dims 16dt+4g..16dt+4g+3 of head c: one 16-byte store per dt.
template <int D>
__device__ inline void attn_wave_publish(AttnState<D> &st, float *ow, float *wm, float *wl, int wave,
                                         int dv, int g, int c) {
    attn_wave_total<D>(st);
    if (g == 0) {
        wm[wave * 16 + c] = st.m;
        wl[wave * 16 + c] = st.l;
    }
    float *row = ow + (wave * 16 + c) * attn_ow_ld(dv) + 4 * g;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
        if (16 * dt < dv) *reinterpret_cast<f32x4 *>(row + 16 * dt) = st.o[dt];
}

// Combine the n waves' states of head h at dim d (log-sum-exp).
__device__ inline void attn_combine(const float *ow, const float *wm, const float *wl, int n, int h, int d,
                                    int dv, float &O, float &M, float &L) {
    M = -INFINITY;
    for (int w = 0; w < n; ++w) M = fmaxf(M, wm[w * 16 + h]);
    O = 0.f;
    L = 0.f;
    if (M == -INFINITY) return;
    for (int w = 0; w < n; ++w) {
        const float mw = wm[w * 16 + h];
        const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
        O += f * ow[(w * 16 + h) * attn_ow_ld(dv) + d];
        L += f * wl[w * 16 + h];
    }
}

// Final normalisation with an optional sink logit (natural-log units), bf16 bits out.
__device__ inline uint16_t attn_finish(float O, float M, float L, const float *sink, int h) {
    if (sink) {
        const float s2 = sink[h] * kLog2e;
        const float M2 = fmaxf(M, s2);
        if (M2 != -INFINITY) {
            const float f = M == -INFINITY ? 0.f : exp2f(M - M2);
            O *= f;
            L = L * f + exp2f(s2 - M2);
        }
    }
    const float val = L > 0.f ? O / L : 0.f;
    return __builtin_bit_cast(uint16_t, (__bf16)val);
}

// The same for four consecutive dims: one reciprocal of the normaliser, and the four
// bf16 results packed for one 8-byte store.
__device__ inline u32x2 attn_finish4(f32x4 O, float M, float L, const float *sink, int h) {
    if (sink) {
        const float s2 = sink[h] * kLog2e;
        const float M2 = fmaxf(M, s2);
        if (M2 != -INFINITY) {
            const float f = M == -INFINITY ? 0.f : exp2f(M - M2);
            O *= f;
            L = L * f + exp2f(s2 - M2);
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint16_t r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = __builtin_bit_cast(uint16_t, (__bf16)(O[e] * inv));
    return u32x2{(uint32_t)r[0] | ((uint32_t)r[1] << 16), (uint32_t)r[2] | ((uint32_t)r[3] << 16)};
}

// ---------------------------------------------------------------------------
// Wave and workgroup scans.  The wave scan uses DPP lane shifts within rows of 16
// lanes and the row broadcasts of 64-lane waves (no LDS traffic).
// ---------------------------------------------------------------------------
__device__ inline uint32_t wave_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Inclusive scan over the workgroup (ascending thread id); *total gets the sum.  Every
// thread of the workgroup must call it; NW = waves per workgroup (a constant, so that no
// launch-size load -- and with it a wait on every outstanding load -- is emitted).
// wsum needs NW entries.  TAIL = false leaves out the closing barrier (which keeps a
// following scan from overwriting wsum while it is still read) for callers that reach a
// barrier of their own before wsum is written again.
template <int NW, bool TAIL = true>
__device__ inline uint32_t wg_scan(uint32_t v, uint32_t *wsum, uint32_t *total) {
    const int lane = threadIdx.x & 63;
    const int wid = threadIdx.x >> 6;
    v = wave_scan(v);
    if (lane == 63) wsum[wid] = v;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const uint32_t x = wsum[w];
        before += w < wid ? x : 0u;
        all += x;
    }
    *total = all;
    if constexpr (TAIL) __syncthreads();
    return v + before;
}

// Order-preserving 32-bit key of a float: a larger float gives a larger key; -0 ranks
// as +0.
__device__ inline uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace lit
