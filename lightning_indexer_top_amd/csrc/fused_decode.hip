// fused_decode.hip -- plan, workspace / state layout and dispatch of the fused decode
// kernel (fused_kernel.h): the team shape (chunk, team size) that fits every workgroup
// on the device at once, where the team's scores live during selection, and the
// launch of the kernel form (fused_forms.hip) of the call's index-code format, masking,
// KV format and layer count.
#include <atomic>

#include "fused_kernel.h"

namespace lit {

namespace {

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

// The forms by their traits (LIT_FUSED_FORMS).
struct FusedForm {
    int fmt;
    bool mask, qkv, layers;
    hipError_t (*launch)(const FusedArgs &, int, size_t, hipStream_t);
    int (*per_cu)(int, int, int, size_t, bool);
};
#define LIT_FUSED_ENTRY(name, fmt, mask, qkv, layers) {fmt, mask, qkv, layers, launch_fused_##name, fused_per_cu_##name},
constexpr FusedForm kForms[] = {LIT_FUSED_FORMS(LIT_FUSED_ENTRY)};
#undef LIT_FUSED_ENTRY

const FusedForm *find_form(int fmt, bool mask, bool qkv, bool layers) {
    for (const FusedForm &f : kForms)
        if (f.fmt == fmt && f.mask == mask && f.qkv == qkv && f.layers == layers) return &f;
    return nullptr;
}

// Co-resident workgroups of the fused kernel on the current device.
int max_resident(int fmt, bool masked, bool qkv, bool layers, int D, int DI, int HT, size_t dyn, bool cached) {
    const FusedForm *form = find_form(fmt, masked, qkv, layers);
    if (!form) return 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    const int cus = device_cus(dev);
    if (cus <= 0) return 0;
    return cus * form->per_cu(D, DI, HT, dyn, cached);
}

}  // namespace

FusedPlan plan_fused(int fmt, bool masked, bool qkv, bool layers, int B, int S, int start_pos, int ratio, int Hi,
                     int Di, int D, int dv, int W, int keff) {
    FusedPlan p{};
    p.ok = false;
    const int n_teams = B * S;
    const long T = ((long)start_pos + S) / ratio;
    if (n_teams <= 0 || keff <= 0 || T <= 0 || T > (1L << 24)) return p;
    if (D != 64 && D != 128 && D != 192 && D != 256) return p;
    if ((Di != 64 && Di != 128) || Hi % 16 || Hi > 64) return p;
    const int nwin = window_width(S, start_pos, W);
    p.win_tiles = (nwin + 31) / 32;
    p.cache_lds = T <= (long)kCacheQ * 4 * kThreads;
    int chunk = 256;
    size_t dyn = 0;
    int cap = 0;
    for (;; chunk *= 2) {
        if (chunk > 8192) return p;
        // chunk scores + picks, and the team's scores when they fit the register cache, else
        // (when they fit) 16-bit value bins of every team position
        dyn = (size_t)chunk * 2 * sizeof(float) + (p.cache_lds ? (size_t)kCacheQ * 4 * kThreads * sizeof(float) : 0);
        p.lds_bins = false;
        if (!p.cache_lds) {
            // the bins (padded to 16 bytes), then kCandCap candidate positions
            const size_t with_bins = dyn + (size_t)(T + 7) / 8 * 16 + (size_t)kCandCap * 4;
            if (max_resident(fmt, masked, qkv, layers, D, Di, Hi / 16, with_bins, false) > 0) {
                dyn = with_bins;
                p.lds_bins = true;
            }
        }
        cap = max_resident(fmt, masked, qkv, layers, D, Di, Hi / 16, dyn, p.cache_lds);
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
    // value bins of the selection: about two visible rows a bin, at least 256, at most 4096
    p.vbins = T <= 1024 ? 256 : T <= 4096 ? 1024 : 4096;
    p.ok = true;
    (void)dv;
    return p;
}

size_t fused_state_bytes(const FusedPlan &p) {
    // error word, then one fixed-size region per query
    return 256 + (size_t)p.n_teams * kQState;
}

static int slot_floats(int dv) { return (kHeads * dv + 2 * kHeads + 63) / 64 * 64; }  // 16-byte multiple

size_t fused_ws_bytes(const FusedPlan &p, int dv, int layers) {
    return (size_t)p.n_teams * p.ld * 4 + 256 +                                      // team scores
           (size_t)p.n_teams * p.team_size * layers * slot_floats(dv) * 4 + 256;     // partial states
}

size_t fused_part_bytes_per_query(const FusedPlan &p, int dv, int layers) {
    return (size_t)p.team_size * (size_t)(layers > 0 ? layers : 1) * slot_floats(dv) * 4;
}

hipError_t launch_fused(FusedArgs f, const FusedPlan &p, void *ws, void *state, hipStream_t stream,
                        uint32_t *err_word) {
    char *st = (char *)state;
    f.err = err_word ? err_word : (uint32_t *)st;
    f.qstate = st + 256;
    char *rest = (char *)ws;
    auto bump = [&](size_t bytes) {
        char *r = rest;
        rest += (bytes + 255) / 256 * 256;
        return r;
    };
    f.scores = (float *)bump((size_t)p.n_teams * p.ld * 4);
    f.part = (float *)bump((size_t)p.n_teams * p.team_size * f.aa.L * slot_floats(f.aa.dv) * 4);
    f.slot_floats = slot_floats(f.aa.dv);
    f.team_size = p.team_size;
    f.chunk = p.chunk;
    f.win_tiles = p.win_tiles;
    f.vbins = p.vbins;
    f.n_slots = p.n_slots;
    f.merge_per = (f.aa.L * kHeads * (f.aa.dv / 4) + p.team_size - 1) / p.team_size;
    f.div_team = fast_div((uint32_t)p.team_size);
    f.div_S = fast_div((uint32_t)f.ia.S);
    f.div_ratio = fast_div((uint32_t)f.ia.ratio);
    f.div_R = fast_div((uint32_t)(f.aa.R > 0 ? f.aa.R : 1));
    f.div_qdv = fast_div((uint32_t)(f.aa.dv / 4));
    f.div_hq = fast_div((uint32_t)(kHeads * (f.aa.dv / 4)));
    f.div_cbs = fast_div((uint32_t)(f.cand_bs > 0 ? f.cand_bs : 1));
    f.ld = p.ld;
    f.cache_lds = p.cache_lds;
    f.lds_bins = p.lds_bins;
    f.bins_words = (int)((p.ld + 7) / 8 * 4);  // 32-bit words of the padded bins
    const FusedForm *form = find_form(f.ia.fmt, f.cand != nullptr, f.aa.win_fmt != kKvBf16 || f.aa.comp_fmt != kKvBf16,
                                      f.aa.L > 1);
    if (!form) return hipErrorInvalidValue;
    return form->launch(f, p.grid, p.dyn_bytes, stream);
}

}  // namespace lit
