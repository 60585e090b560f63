// abi_driver.cpp -- drives the host side of liblit.so's C ABI (include/lit.h): argument
// validation, refusals and workspace / state sizing, over valid, edge-case and invalid
// shapes.  Built host-only with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py; no call reaches a kernel launch, so no GPU is needed.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/lit.h"

static int failures = 0;
#define EXPECT(cond)                                                        \
    do {                                                                    \
        if (!(cond)) {                                                      \
            std::fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                                     \
        }                                                                   \
    } while (0)

static void *const A = reinterpret_cast<void *>(0x10000);    // aligned stand-in, never read
static void *const MIS = reinterpret_cast<void *>(0x10001);  // misaligned stand-in

static lit_step_args step(int B, int S, int start_pos, int ratio, int Hi, int Di, int k, int D, int W) {
    lit_step_args s;
    std::memset(&s, 0, sizeof s);
    s.B = B; s.S = S; s.start_pos = start_pos; s.ratio = ratio; s.Hi = Hi; s.Di = Di; s.index_topk = k;
    s.T_cap = (start_pos + S) / (ratio > 0 ? ratio : 1);
    s.q8 = (const uint8_t *)A; s.q_sc = (const uint8_t *)A; s.w = (const float *)A;
    s.k8 = (const uint8_t *)A; s.k_sc = (const uint8_t *)A;
    s.H = 16; s.D = D; s.dv = D; s.W = W; s.R = W + S;
    s.q = (const uint16_t *)A; s.win_kv = (const uint16_t *)A; s.comp_kv = (const uint16_t *)A;
    s.scale = 0.1f; s.topk_idx = (int32_t *)A; s.out = (uint16_t *)A;
    return s;
}

int main() {
    for (int c = -1; c < 9; ++c) EXPECT(lit_status_str(c) != nullptr);
    EXPECT(lit_abi_version() == LIT_ABI_VERSION);
    for (int S = 0; S < 5; ++S)
        for (int p = 0; p < 40; p += 3)
            for (int r = -1; r < 5; ++r) {
                const int kw = lit_topk_width(S, p, r, 16);
                EXPECT(kw >= 0 && kw <= 16);
                (void)lit_window_width(S, p, 8);
                (void)lit_compress_writes_row(p, r);
                (void)lit_candidate_blocks_width(S, p, r, 8, 4);
                (void)lit_topk_workspace_bytes(2, S, p, r > 0 ? r : 1, 16);
                (void)lit_candidate_blocks_workspace_bytes(2, S, p, r > 0 ? r : 1, 4);
            }
    (void)lit_sparse_attn_workspace_bytes(8, 1, 16, 192, 128, 2048);
    (void)lit_sparse_attn_layers_workspace_bytes(3, 8, 1, 16, 192, 128, 2048);
    // indexer refusals
    const uint8_t *u = (const uint8_t *)A;
    float *f = (float *)A;
    EXPECT(lit_indexer_scores(u, u, f, u, u, 1, 1, 16, 48, 512, 1023, 2, f, 512, nullptr) == LIT_E_SHAPE);
    EXPECT(lit_indexer_scores(u, u, f, u, u, 1, 1, 80, 64, 512, 1023, 2, f, 512, nullptr) == LIT_E_UNSUPPORTED);
    EXPECT(lit_indexer_scores(u, u, f, nullptr, u, 1, 1, 16, 64, 512, 1023, 2, f, 512, nullptr) == LIT_E_NULL);
    EXPECT(lit_indexer_scores((const uint8_t *)MIS, u, f, u, u, 1, 1, 16, 64, 512, 1023, 2, f, 512, nullptr) ==
           LIT_E_ALIGN);
    EXPECT(lit_indexer_scores(u, u, f, u, u, 0, 1, 16, 64, 512, 1023, 2, f, 512, nullptr) == LIT_OK);
    EXPECT(lit_indexer_scores_fmt(7, u, u, f, u, u, 1, 1, 16, 64, 512, 1023, 2, f, 512, nullptr) ==
           LIT_E_UNSUPPORTED);
    // top-k refusals
    int32_t *ip = (int32_t *)A;
    EXPECT(lit_topk(f, 510, 1, 1, 1023, 2, 64, ip, A, 1 << 20, nullptr) == LIT_E_SHAPE);
    EXPECT(lit_topk(f, 514, 1, 1, 1023, 2, 64, ip, A, 1 << 20, nullptr) == LIT_E_ALIGN);
    EXPECT(lit_topk(nullptr, 512, 1, 1, 1023, 2, 64, ip, A, 1 << 20, nullptr) == LIT_E_NULL);
    EXPECT(lit_topk(f, 512, 1, 1, 1023, 0, 64, ip, A, 1 << 20, nullptr) == LIT_E_SHAPE);
    // window and attention refusals
    EXPECT(lit_window_indices(1, 1, 5, 4, 0, ip, nullptr) != LIT_OK);
    const uint16_t *h = (const uint16_t *)A;
    uint16_t *o = (uint16_t *)A;
    EXPECT(lit_sparse_attn(h, 1, 1, 8, 128, 128, h, 128, ip, 128, h, 512, ip, 64, nullptr, 0.1f, o, A, 1 << 20,
                           nullptr) == LIT_E_UNSUPPORTED);  // 8 heads
    EXPECT(lit_sparse_attn(h, 1, 1, 16, 96, 96, h, 128, ip, 128, h, 512, ip, 64, nullptr, 0.1f, o, A, 1 << 20,
                           nullptr) == LIT_E_UNSUPPORTED);  // D = 96
    EXPECT(lit_sparse_attn(h, 1, 1, 16, 128, 256, h, 128, ip, 128, h, 512, ip, 64, nullptr, 0.1f, o, A, 1 << 20,
                           nullptr) == LIT_E_SHAPE);        // dv > D
    EXPECT(lit_sparse_attn(nullptr, 1, 1, 16, 128, 128, h, 128, ip, 128, h, 512, ip, 64, nullptr, 0.1f, o, A,
                           1 << 20, nullptr) == LIT_E_NULL);
    // producer refusals
    EXPECT(lit_compress_append(1, 48, 2, 1, f, f, f, f, f, 1e-6f, f, 4, 16, (uint8_t *)A,
                               (uint8_t *)A, 4, nullptr, nullptr) == LIT_E_SHAPE);
    EXPECT(lit_window_append(1, 64, 0, h, f, 4, 16, (uint8_t *)A, (uint8_t *)A, 0, nullptr) == LIT_E_SHAPE);
    // step sizing over the workloads' shapes, edge cases and refusals
    const lit_step_args shapes[] = {
        step(1, 1, 1023, 2, 16, 64, 64, 128, 128),   step(4, 1, 4095, 1, 16, 64, 64, 128, 128),
        step(8, 1, 16383, 2, 64, 128, 2048, 192, 128), step(1, 4096, 12288, 2, 16, 64, 512, 128, 128),
        step(2, 1, 131071, 4, 64, 128, 2048, 128, 128), step(1, 1, 2, 4, 16, 64, 64, 128, 128),
        step(1, 70, 0, 2, 16, 64, 16, 64, 16),        step(0, 1, 100, 2, 16, 64, 64, 128, 128),
    };
    for (const lit_step_args &s0 : shapes) {
        lit_step_args s = s0;
        (void)lit_sparse_step_workspace_bytes(&s);
        (void)lit_sparse_step_state_bytes(&s);
        s.flags = LIT_STEP_UNFUSED;
        (void)lit_sparse_step_workspace_bytes(&s);
        s.layers = 3;
        (void)lit_sparse_step_workspace_bytes(&s);
        lit_step_args bad = s0;
        bad.Di = 48;
        EXPECT(lit_sparse_step(&bad, A, 1 << 20, nullptr) != LIT_OK);
        bad = s0;
        bad.index_topk = -1;
        EXPECT(lit_sparse_step(&bad, A, 1 << 20, nullptr) != LIT_OK || s0.B == 0);
        bad = s0;
        bad.R = 1;
        EXPECT(lit_sparse_step(&bad, A, 1 << 20, nullptr) != LIT_OK || s0.B == 0);
        bad = s0;
        EXPECT(lit_sparse_step(&bad, nullptr, 0, nullptr) != LIT_OK || s0.B == 0);
    }
    EXPECT(lit_sparse_step(nullptr, A, 1 << 20, nullptr) == LIT_E_NULL);
    EXPECT(lit_sparse_step_noalloc(nullptr, nullptr, nullptr) == LIT_E_NULL);
    {
        lit_step_args big = step(1, 4096, 12288, 2, 16, 64, 512, 128, 128);  // workspace beyond the scratch
        big.R = 4223;
        EXPECT(lit_sparse_step_noalloc(&big, nullptr, nullptr) == LIT_E_WORKSPACE);
    }
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("abi driver ok\n");
    return 0;
}
