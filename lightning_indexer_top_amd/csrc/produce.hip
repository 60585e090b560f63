// produce.hip -- the cache writes of a decode step or a chunk: the compressor's slot fill
// and softmax pooling into compressed-KV rows, and the window-KV ring slots.
//
// What is computed (DeepSeek-V4.1-Flash-NVFP4 inference/model.py):
//   Compressor.forward, decode: the new token's kv and gate score (after the wkv / wgate
//     projections, which are outside the path) fill slot start_pos % ratio of the
//     sequence's state; when the group completes, the latent is the softmax-gated sum
//     over the slots (per feature, fp32), cast to bf16, RMS-normalised (RMSNorm.forward:
//     fp32 math, bf16 result).  Ratio 1 has no state: the latent is the norm of the
//     token's kv.
//   Attention._compress_kv: the latent's last rd dims are rotated at the group's first
//     position (apply_rotary_emb: adjacent pairs as complex numbers), the result rounded
//     to bf16, quantised to fp4 in groups of 16 with e4m3 scales and written to cache
//     row start_pos / ratio.
//   Attention._window_kv, decode: the token's window KV row is rotated at start_pos,
//     quantised to e4m3 with a ue8m0 scale per 32 and written to ring slot start_pos % R.
//   A chunk of S tokens is the S decode steps in order: at start_pos 0 that is the pages'
//     prefill branches (Compressor.forward: whole groups pooled at once, the remainder left
//     in the state; _window_kv: the ring seeded with the chunk's last rows).  One
//     workgroup per completed group (its slots from the state for positions before the
//     chunk, else from the chunk) and per surviving window row.
// Quantiser decisions are exact: the fp4 scale is the smallest e4m3 value s with
// 6 s >= amax and a code compares |x| with the midpoints times s (products exact in
// fp32); the e4m3 scale is the smallest 2^e with amax <= 448 * 2^e and a code rounds
// x / 2^e (exact) to the nearest e4m3 value, ties to the even code.
//
// Mapping: one workgroup per sequence and written row, one thread per feature (D <= 256).
// A row moves a few hundred bytes; the kernels are launch-bound, not bandwidth-bound.
#include "lit_internal.h"

namespace lit {

namespace {

constexpr int kThreads = 256;

__device__ inline float bf16_round(float x) { return (float)(__bf16)x; }

// e4m3 value of a positive code c (1..126), exact.
__device__ inline float e4m3_pos_value(int c) {
    const int e = c >> 3, m = c & 7;
    return e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
}

// e4m3 code of y, |y| <= 448, nearest with ties to the even code (v_rndne).
__device__ inline uint32_t e4m3_encode(float y) {
    const float a = fminf(fabsf(y), 448.f);
    uint32_t code;
    if (a < 0x1p-6f) {
        code = (uint32_t)__builtin_rintf(a * 512.f);  // subnormal steps of 2^-9; 8 is 2^-6
    } else {
        int e = ilogbf(a);
        int q = (int)__builtin_rintf((ldexpf(a, -e) - 1.f) * 8.f);
        if (q == 8) {
            ++e;
            q = 0;
        }
        code = (uint32_t)(((e + 7) << 3) | q);
    }
    return code | (signbit(y) ? 0x80u : 0u);
}

// Reduction over groups of `width` adjacent lanes (width a power of two, <= 64).
__device__ inline float group_max(float v, int width) {
    for (int off = width / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, width));
    return v;
}

__device__ inline float block_sum(float v, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float s = 0.f;
    for (int w = 0; w < kThreads / 64; ++w) s += red[w];
    __syncthreads();
    return s;
}

// Rotate the last rd of D bf16 values in LDS at table row pos, rounding to bf16.
__device__ inline void rope_lds(float *x, int D, int rd, const float *freqs, int pos) {
    const int j = threadIdx.x;
    if (j < rd / 2) {
        const float a = x[D - rd + 2 * j], b = x[D - rd + 2 * j + 1];
        const float c = freqs[((size_t)pos * (rd / 2) + j) * 2], s = freqs[((size_t)pos * (rd / 2) + j) * 2 + 1];
        // the complex product, each term rounded on its own (no fused multiply-add)
        x[D - rd + 2 * j] = bf16_round(__fsub_rn(__fmul_rn(a, c), __fmul_rn(b, s)));
        x[D - rd + 2 * j + 1] = bf16_round(__fadd_rn(__fmul_rn(a, s), __fmul_rn(b, c)));
    }
    __syncthreads();
}

// One group's cache row: the latent pooled over its `ratio` slots (slot(r, d) gives slot r's
// kv and score of feature d), RMS-normalised, optionally stored (pre-rotation, bf16), rotated
// at `pos` and quantised into compressed row `row` of sequence b.
template <typename Slot>
__device__ inline void write_group(const ProduceArgs &p, int b, Slot slot, int pos, int row, uint16_t *lat,
                                   float *x, float *red) {
    const int d = threadIdx.x;
    const bool live = d < p.D;
    float v = 0.f;
    if (live) {
        if (p.ratio == 1) {
            v = bf16_round(slot(0, d).x);
        } else {
            float m = -INFINITY;
            for (int r = 0; r < p.ratio; ++r) m = fmaxf(m, slot(r, d).y);
            float z = 0.f, acc = 0.f;
            for (int r = 0; r < p.ratio; ++r) {
                const float2 ks = slot(r, d);
                const float e = expf(ks.y - m);
                z += e;
                acc += e * ks.x;
            }
            v = bf16_round(acc / z);  // kv.to(dtype)
        }
    }
    // RMSNorm (fp32), bf16 result
    const float ss = block_sum(v * v, red);
    const float rn = 1.f / sqrtf(ss / (float)p.D + p.eps);
    const float y = live ? bf16_round(p.norm_w[d] * (v * rn)) : 0.f;
    if (lat && live) lat[d] = __builtin_bit_cast(uint16_t, (__bf16)y);
    x[d] = y;
    __syncthreads();
    rope_lds(x, p.D, p.rd, p.freqs, pos);
    // fp4 with an e4m3 scale per 16 dims
    const float xv = live ? x[d] : 0.f;
    const float amax = group_max(fabsf(xv), 16);
    int lo = 1, hi = 126;  // smallest positive e4m3 value s with 6 s >= amax
    while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (6.f * e4m3_pos_value(mid) >= amax) hi = mid; else lo = mid + 1;
    }
    const float s = e4m3_pos_value(lo);
    const float a = fabsf(xv);
    uint32_t c = (a > 0.25f * s) + (a >= 0.75f * s) + (a > 1.25f * s) + (a >= 1.75f * s) + (a > 2.5f * s) +
                 (a >= 3.5f * s) + (a > 5.f * s);
    c |= xv < 0.f ? 8u : 0u;
    const uint32_t other = (uint32_t)__shfl_xor((int)c, 1);
    const size_t rw = (size_t)b * p.T_cap + row;
    if (live && (d & 1) == 0) p.codes[rw * (p.D / 2) + d / 2] = (uint8_t)(c | (other << 4));
    if (live && (d & 15) == 0) p.scales[rw * (p.D / 16) + d / 16] = (uint8_t)lo;
}

__global__ __launch_bounds__(kThreads) void compress_append_kernel(ProduceArgs p) {
    __shared__ float x[kThreads];
    __shared__ float red[kThreads / 64];
    const int b = blockIdx.x;
    const int d = threadIdx.x;
    const bool done = (p.start_pos + 1) % p.ratio == 0;
    const float *kv = p.kv + (size_t)b * p.D, *sc = p.score + (size_t)b * p.D;
    float *ks = p.kv_state + (size_t)b * p.ratio * p.D;
    float *gs = p.score_state + (size_t)b * p.ratio * p.D;
    if (p.ratio > 1) {
        const int slot = p.start_pos % p.ratio;
        if (d < p.D) {
            ks[(size_t)slot * p.D + d] = kv[d];
            gs[(size_t)slot * p.D + d] = sc[d];
        }
        if (!done) return;
    }
    // (each thread reads back only its own feature's slots)
    auto slot = [&](int r, int dd) {
        return p.ratio == 1 ? make_float2(kv[dd], sc[dd])
                            : make_float2(ks[(size_t)r * p.D + dd], gs[(size_t)r * p.D + dd]);
    };
    write_group(p, b, slot, p.start_pos + 1 - p.ratio, p.start_pos / p.ratio,
                p.latent ? p.latent + (size_t)b * p.D : nullptr, x, red);
}

// A chunk: workgroup (b, j) writes the j-th group completed in the chunk (group g_lo + j); the
// first also leaves every slot holding the last chunk token of its residue in the state, after
// reading the slots its group took from there (no other group reads the state).
__global__ __launch_bounds__(kThreads) void compress_chunk_kernel(ProduceArgs p, int g_lo, int n_rows) {
    __shared__ float x[kThreads];
    __shared__ float red[kThreads / 64];
    const int b = blockIdx.x;
    const int j = blockIdx.y;
    const int d = threadIdx.x;
    const float *kv = p.kv + (size_t)b * p.S * p.D, *sc = p.score + (size_t)b * p.S * p.D;
    float *ks = p.ratio > 1 ? p.kv_state + (size_t)b * p.ratio * p.D : nullptr;
    float *gs = p.ratio > 1 ? p.score_state + (size_t)b * p.ratio * p.D : nullptr;
    if (j < n_rows) {
        const int g = g_lo + j;
        // slot r of group g is position g * ratio + r: from the state before the chunk
        auto slot = [&](int r, int dd) {
            const int t = g * p.ratio + r - p.start_pos;
            return t < 0 ? make_float2(ks[(size_t)r * p.D + dd], gs[(size_t)r * p.D + dd])
                         : make_float2(kv[(size_t)t * p.D + dd], sc[(size_t)t * p.D + dd]);
        };
        write_group(p, b, slot, g * p.ratio, g, p.latent ? p.latent + ((size_t)b * n_rows + j) * p.D : nullptr, x,
                    red);
    }
    // (a thread reads and writes only its own feature's state entries, in program order)
    if (j == 0 && p.ratio > 1 && d < p.D) {
        for (int r = 0; r < p.ratio; ++r) {
            // the last chunk position with residue r
            const int last = p.start_pos + p.S - 1;
            const int pr = last - ((last - r) % p.ratio + p.ratio) % p.ratio;
            if (pr >= p.start_pos) {
                ks[(size_t)r * p.D + d] = kv[(size_t)(pr - p.start_pos) * p.D + d];
                gs[(size_t)r * p.D + d] = sc[(size_t)(pr - p.start_pos) * p.D + d];
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void window_append_kernel(ProduceArgs p) {
    __shared__ float x[kThreads];
    const int b = blockIdx.x;
    const int d = threadIdx.x;
    const bool live = d < p.D;
    x[d] = live ? (float)__builtin_bit_cast(__bf16, p.win_in[(size_t)b * p.D + d]) : 0.f;
    __syncthreads();
    rope_lds(x, p.D, p.rd, p.freqs, p.start_pos);
    const float xv = live ? x[d] : 0.f;
    const float amax = group_max(fabsf(xv), 32);
    int e = -127;
    if (amax > 0.f) {
        e = ilogbf(amax) - 9;
        while (amax > 448.f * ldexpf(1.f, e)) ++e;
    }
    const size_t slot = (size_t)b * p.R + p.start_pos % p.R;
    if (live) p.codes[slot * p.D + d] = (uint8_t)e4m3_encode(ldexpf(xv, -e));
    if (live && (d & 31) == 0) p.scales[slot * (p.D / 32) + d / 32] = (uint8_t)(e + 127);
}


// A chunk into the ring: workgroup (b, j) writes the j-th of the chunk's last min(S, R) rows
// (earlier rows would be overwritten within the chunk), at its own position's slot.
__global__ __launch_bounds__(kThreads) void window_chunk_kernel(ProduceArgs p, int first) {
    __shared__ float x[kThreads];
    const int b = blockIdx.x;
    const int t = first + blockIdx.y;
    const int pos = p.start_pos + t;
    const int d = threadIdx.x;
    const bool live = d < p.D;
    x[d] = live ? (float)__builtin_bit_cast(__bf16, p.win_in[((size_t)b * p.S + t) * p.D + d]) : 0.f;
    __syncthreads();
    rope_lds(x, p.D, p.rd, p.freqs, pos);
    const float xv = live ? x[d] : 0.f;
    const float amax = group_max(fabsf(xv), 32);
    int e = -127;
    if (amax > 0.f) {
        e = ilogbf(amax) - 9;
        while (amax > 448.f * ldexpf(1.f, e)) ++e;
    }
    const size_t slot = (size_t)b * p.R + pos % p.R;
    if (live) p.codes[slot * p.D + d] = (uint8_t)e4m3_encode(ldexpf(xv, -e));
    if (live && (d & 31) == 0) p.scales[slot * (p.D / 32) + d / 32] = (uint8_t)(e + 127);
}

}  // namespace

hipError_t launch_compress_append(const ProduceArgs &p, hipStream_t stream) {
    if (p.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(compress_append_kernel, dim3(p.B), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_window_append(const ProduceArgs &p, hipStream_t stream) {
    if (p.B <= 0) return hipSuccess;
    hipLaunchKernelGGL(window_append_kernel, dim3(p.B), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

int compress_chunk_rows(int start_pos, int S, int ratio) {
    if (ratio < 1 || start_pos < 0 || S < 0) return 0;
    return (start_pos + S) / ratio - start_pos / ratio;
}

hipError_t launch_compress_chunk(const ProduceArgs &p, hipStream_t stream) {
    if (p.B <= 0 || p.S <= 0) return hipSuccess;
    const int n = compress_chunk_rows(p.start_pos, p.S, p.ratio);
    if (n == 0 && p.ratio == 1) return hipSuccess;
    hipLaunchKernelGGL(compress_chunk_kernel, dim3(p.B, n > 0 ? n : 1), dim3(kThreads), 0, stream, p,
                       p.start_pos / p.ratio, n);
    return hipGetLastError();
}

hipError_t launch_window_chunk(const ProduceArgs &p, hipStream_t stream) {
    if (p.B <= 0 || p.S <= 0) return hipSuccess;
    const int n = p.S < p.R ? p.S : p.R;
    hipLaunchKernelGGL(window_chunk_kernel, dim3(p.B, n), dim3(kThreads), 0, stream, p, p.S - n);
    return hipGetLastError();
}

}  // namespace lit
