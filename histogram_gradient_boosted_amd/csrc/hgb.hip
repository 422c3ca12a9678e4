// hgb: C ABI of the level histogram build (see include/hgb.h for the contract).
//
// Host side of the library: the context, argument validation, per-call launch
// planning and the staging of small plans to the device.  The kernels live in
// hgb_kernels.h.
#include "hgb.h"
#include "hgb_kernels.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

using namespace hgb;

namespace {

// gfx950: 160 KiB of LDS per CU; every fill runs one 1024-thread block per CU.
constexpr int64_t kFillLdsBudget = 160 * 1024;
constexpr int kRootThreads = 1024;
constexpr int kLevelThreads = 1024;
// Fill items per CU: the root gets one equal share per CU (equal items finish
// together, and fewer items mean fewer merges of partial histograms); other
// levels, with nodes of very different sizes, get several smaller items per
// CU for balance.
constexpr int64_t kRootItemsPerCu = 1;
constexpr int64_t kLevelItemsPerCu = 4;
// Keep a row-major copy of the bins when a row takes at most this many bytes.
constexpr int64_t kRowMajorMaxRowBytes = 512;
// Default fixed-point precision of begin_tree (bits below the largest value).
constexpr int kDefaultPrecision = 30;
constexpr int kStages = 4;

struct Stage {
    void* host = nullptr;
    void* dev = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
};

}  // namespace

struct hgb_ctx {
    int device = 0;
    int n_cu = 256;
    hipStream_t stream = nullptr;
    std::string err;

    // dataset plane: feature-major bins, plus a row-major copy when rows are
    // narrow enough for a row to sit in a cache line or two
    void* bins = nullptr;
    void* bins_rm = nullptr;
    int64_t rm_stride = 0;   // bytes per row of the row-major copy (multiple of 16)
    int bin_bytes = 0;
    int64_t n = 0;
    int F = 0, B = 0, S = 0, has_missing = 0;
    bool have_data = false;

    // gradient plane
    int2* q = nullptr;
    int64_t q_cap = 0;
    int precision = kDefaultPrecision;
    int k_g = 0, k_h = 0;
    bool have_tree = false;

    // level scratch
    int2* gh = nullptr;
    int64_t gh_cap = 0;
    FeatureBest* best = nullptr;
    int64_t best_cap = 0;
    long long* totals = nullptr;
    int64_t totals_cap = 0;

    // small device words: [0..1] max patterns, [2] error flags
    uint32_t* dev_words = nullptr;
    uint32_t* host_words = nullptr;   // pinned

    Stage stage[kStages];
    int stage_next = 0;

    // HGB_DEBUG_PLAN=1 in the environment prints each fill plan to stderr
    bool debug_plan = false;
    // HGB_FILL_TUNE="key=value,..." overrides the fill planner (developer
    // tuning): root_lc, root_tile, root_ipc, level_lc, level_tile, level_ipc
    // (ipc = items per CU), align (rows an item boundary is a multiple of);
    // -1 keeps the planner's choice.
    int tune[7] = {-1, -1, -1, -1, -1, -1, -1};

    // optional per-kernel timing
    bool prof = false;
    std::vector<hipEvent_t> ev_pool;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_pending[HGB_KERNEL_COUNT];
    double prof_ms[HGB_KERNEL_COUNT] = {};
    int64_t prof_launches[HGB_KERNEL_COUNT] = {};
};

namespace {

hgb_status fail(hgb_ctx* c, hgb_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    c->err = buf;
    return st;
}

#define HGB_HIP(c, expr)                                                                   \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess)                                                              \
            return fail((c), HGB_E_DEVICE, "%s failed: %s", #expr, hipGetErrorString(e_)); \
    } while (0)

#define HGB_LAUNCHED(c, what)                                                              \
    do {                                                                                   \
        hipError_t e_ = hipGetLastError();                                                 \
        if (e_ != hipSuccess)                                                              \
            return fail((c), HGB_E_DEVICE, "launch of %s failed: %s", what,                \
                        hipGetErrorString(e_));                                            \
    } while (0)

template <typename T>
hgb_status grow(hgb_ctx* c, T** p, int64_t* cap, int64_t need)
{
    if (need <= *cap) return HGB_OK;
    if (*p) {
        HGB_HIP(c, hipStreamSynchronize(c->stream));
        HGB_HIP(c, hipFree(*p));
        *p = nullptr;
        *cap = 0;
    }
    int64_t want = std::max<int64_t>(need, 1024);
    HGB_HIP(c, hipMalloc((void**)p, sizeof(T) * (size_t)want));
    *cap = want;
    return HGB_OK;
}

// Copy `bytes` of host data to a device staging buffer on the stream.  The
// stage is released (event recorded) by stage_release after its consumers have
// been enqueued; a stage is reused only once that event has completed.
hgb_status stage_upload(hgb_ctx* c, const void* src, size_t bytes, Stage** out)
{
    Stage& s = c->stage[c->stage_next];
    c->stage_next = (c->stage_next + 1) % kStages;
    if (s.pending) {
        HGB_HIP(c, hipEventSynchronize(s.ev));
        s.pending = false;
    }
    if (bytes > s.cap) {
        if (s.host) HGB_HIP(c, hipHostFree(s.host));
        if (s.dev) HGB_HIP(c, hipFree(s.dev));
        s.host = s.dev = nullptr;
        size_t want = std::max<size_t>(bytes, 4096);
        HGB_HIP(c, hipHostMalloc(&s.host, want, hipHostMallocDefault));
        HGB_HIP(c, hipMalloc(&s.dev, want));
        s.cap = want;
    }
    if (!s.ev) HGB_HIP(c, hipEventCreateWithFlags(&s.ev, hipEventDisableTiming));
    if (bytes) {
        std::memcpy(s.host, src, bytes);
        HGB_HIP(c, hipMemcpyAsync(s.dev, s.host, bytes, hipMemcpyHostToDevice, c->stream));
    }
    *out = &s;
    return HGB_OK;
}

hgb_status stage_release(hgb_ctx* c, Stage* s)
{
    HGB_HIP(c, hipEventRecord(s->ev, c->stream));
    s->pending = true;
    return HGB_OK;
}

hipEvent_t pool_event(hgb_ctx* c)
{
    if (!c->ev_pool.empty()) {
        hipEvent_t e = c->ev_pool.back();
        c->ev_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Brackets the launches of one kernel class with events when timing is on.
struct ProfScope {
    hgb_ctx* c;
    int kernel;
    hipEvent_t start = nullptr;
    ProfScope(hgb_ctx* ctx, int k) : c(ctx), kernel(k)
    {
        if (!c->prof) return;
        start = pool_event(c);
        if (start && hipEventRecord(start, c->stream) != hipSuccess) {
            c->ev_pool.push_back(start);
            start = nullptr;
        }
    }
    ~ProfScope()
    {
        if (!start) return;
        hipEvent_t stop = pool_event(c);
        if (stop && hipEventRecord(stop, c->stream) == hipSuccess) {
            c->ev_pending[kernel].emplace_back(start, stop);
        } else {
            c->ev_pool.push_back(start);
            if (stop) c->ev_pool.push_back(stop);
        }
    }
};

int grid_for(int64_t work, int threads, int cap)
{
    int64_t g = (work + threads - 1) / threads;
    return (int)std::max<int64_t>(1, std::min<int64_t>(g, cap));
}

// ---------------------------------------------------------------------------
// Fill planning
// ---------------------------------------------------------------------------

enum FillKind { kFillRoot = 0, kFillCols = 1, kFillRowsKind = 2 };

// Launch shape of one build_level fill.
struct FillPlan {
    FillKind kind;
    int acc;            // kWide / kPacked
    int lc;             // log2 of the privatized copy count
    int tile;           // features per item (root, cols: NF; rows: features per load)
    int lt;             // rows: bytes loaded per row
    int threads;
    int64_t step_rows;  // rows a block consumes per step
    int drain;          // packed: steps between drains of the copies (0: wide)
    size_t lds_bytes;
};

// LDS bytes per feature of a tile: the copies, plus the packed accumulator.
int64_t feature_lds(int acc, int S, int lc)
{
    return (int64_t)tile_words(acc, 1, S, lc) * 8;
}

// Packed sums stay exact while every copy-slot sees at most
// kPackedRowsPerCopy rows between drains.  Copy c is used by threads / C
// threads, each taking `per_thread` rows per step; the root kernel may add up
// to kRootRows - 1 tail rows on one copy after its last step.  Returns the
// steps between drains (0: not even one step fits).
int packed_drain_steps(int threads, int lc, int per_thread)
{
    const int64_t per_copy_step = (int64_t)(threads >> lc) * per_thread;
    return (int)((kPackedRowsPerCopy - (kRootRows - 1)) / per_copy_step);
}

// Cost model of the fill per cell (seconds), from microbenchmarks on the
// MI355X: random-bin ds_add_u64 runs at kLdsOps[lc] lanes per clock per CU
// with 2^lc lane-interleaved copies; bins stream from HBM at ~6 TB/s and the
// (g, h) pair, re-read by every feature tile of a row chunk, mostly from L2 at
// ~15 TB/s.  The two overlap imperfectly.
double fill_cost(int acc, int lc, int tile, int w)
{
    static const double kLdsOps[5] = {4.3, 4.75, 5.4, 6.9, 8.4};
    const double lds = (acc == kWide ? 2.0 : 1.0) / (kLdsOps[lc] * 2.4e9 * 256);
    const double mem = w / 6.0e12 + (8.0 / tile) / 15.0e12;
    return std::max(lds, mem) + 0.25 * std::min(lds, mem);
}

FillPlan plan_fill(const hgb_ctx* c, bool root, bool rm)
{
    FillPlan p{};
    const int S = c->S;
    const int w = c->bin_bytes;
    p.kind = root ? kFillRoot : (rm ? kFillRowsKind : kFillCols);
    p.threads = root ? kRootThreads : kLevelThreads;
    auto per_thread_of = [&](int tile) {
        return p.kind == kFillRoot ? kRootRows : (p.kind == kFillCols ? cols_entries(tile) : kLevelEntries);
    };
    const int64_t budget = kFillLdsBudget;
    const int want_acc = c->precision <= kPackedMaxBits ? kPacked : kWide;
    // Candidate tiles: NF in {1, 2, 4, 8} features (root, cols), or the
    // features of one 16/8/4/2-byte row load (rows).
    double best = 1e300;
    bool found = false;
    for (int acc : {want_acc, (int)kWide}) {
        if (found) break;   // fall back to wide sums only when packed cannot fit
        for (int lc = 4; lc >= 0; --lc) {
            const int64_t per_feature = feature_lds(acc, S, lc);
            const int force_lc = c->tune[root ? 0 : 3];
            if (force_lc >= 0 && lc != force_lc) continue;
            for (int k = 0; k < 4; ++k) {
                int tile, lt = 0;
                if (p.kind == kFillRowsKind) {
                    lt = 16 >> k;
                    if (lt < w) continue;
                    tile = lt / w;
                } else {
                    tile = 8 >> k;
                }
                const int force_tile = c->tune[root ? 1 : 4];
                if (force_tile > 0 && tile != force_tile) continue;
                if (tile * per_feature > budget) continue;
                if (p.kind == kFillRoot && w == 2 && tile > 4) continue;   // register-bound
                if (acc == kPacked && packed_drain_steps(p.threads, lc, per_thread_of(tile)) == 0) continue;
                // a tile much wider than the matrix wastes nothing but LDS
                const int eff = std::min(tile, c->F);
                const double cost = fill_cost(acc, lc, eff, w);
                if (cost < best) {
                    best = cost;
                    found = true;
                    p.acc = acc;
                    p.lc = lc;
                    p.tile = tile;
                    p.lt = lt;
                }
            }
        }
    }
    if (!found) {   // one wide feature of one copy always fits (S <= HGB_MAX_SLOTS)
        p.acc = kWide;
        p.lc = 0;
        p.tile = 1;
        p.lt = p.kind == kFillRowsKind ? w : 0;
    }
    if (p.kind != kFillRowsKind) {
        // rows loads cover exactly `tile` features; the others take min(NF, F)
        while (p.tile > 1 && (p.tile >> 1) >= c->F) p.tile >>= 1;
    }
    p.lds_bytes = (size_t)(p.tile * feature_lds(p.acc, S, p.lc));
    p.step_rows = (int64_t)p.threads * per_thread_of(p.tile);
    p.drain = p.acc == kPacked ? packed_drain_steps(p.threads, p.lc, per_thread_of(p.tile)) : 0;
    return p;
}

template <typename K>
hgb_status set_lds(hgb_ctx* c, K kernel, size_t bytes)
{
    HGB_HIP(c, hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)bytes));
    return HGB_OK;
}

struct FillArgs {
    const int2* gh;
    const int32_t* row_index;
    const FillItem* items;
    int n_items;
    int vec_ok;
    int drain;
    int64_t* hist;
};

template <typename BinT, int ACC>
hgb_status launch_fill_acc(hgb_ctx* c, const FillPlan& p, const FillArgs& a)
{
    const unsigned grid = (unsigned)(8 * ((a.n_items + 7) / 8));
    unsigned long long* hist = (unsigned long long*)a.hist;
    const BinT* bins = (const BinT*)c->bins;
    hgb_status st = HGB_OK;
#define HGB_LAUNCH(kern, ...)                                                            \
    do {                                                                                 \
        st = set_lds(c, kern, p.lds_bytes);                                              \
        if (st != HGB_OK) return st;                                                     \
        kern<<<grid, p.threads, p.lds_bytes, c->stream>>>(__VA_ARGS__);                  \
    } while (0)
    if (p.kind == kFillRoot) {
#define HGB_ROOT(NF) HGB_LAUNCH((k_fill_root<BinT, NF, ACC>), bins, c->n, c->F, c->S, p.lc, a.gh, a.items, a.n_items, a.vec_ok, a.drain, hist)
        switch (p.tile) {
        case 1: HGB_ROOT(1); break;
        case 2: HGB_ROOT(2); break;
        case 3: HGB_ROOT(3); break;
        case 4: HGB_ROOT(4); break;
        case 5: HGB_ROOT(5); break;
        case 6: HGB_ROOT(6); break;
        case 7: HGB_ROOT(7); break;
        default: HGB_ROOT(8); break;
        }
#undef HGB_ROOT
    } else if (p.kind == kFillCols) {
        switch (p.tile) {
        case 1: HGB_LAUNCH((k_fill_cols<BinT, 1, ACC>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        case 2: HGB_LAUNCH((k_fill_cols<BinT, 2, ACC>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        case 4: HGB_LAUNCH((k_fill_cols<BinT, 4, ACC>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        default: HGB_LAUNCH((k_fill_cols<BinT, 8, ACC>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        }
    } else {
        const uint8_t* rm = (const uint8_t*)c->bins_rm;
        switch (p.lt) {
        case 16: HGB_LAUNCH((k_fill_rows<BinT, 16, ACC>), rm, c->rm_stride, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        case 8: HGB_LAUNCH((k_fill_rows<BinT, 8, ACC>), rm, c->rm_stride, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        case 4: HGB_LAUNCH((k_fill_rows<BinT, 4, ACC>), rm, c->rm_stride, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        default: HGB_LAUNCH((k_fill_rows<BinT, 2, ACC>), rm, c->rm_stride, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.n_items, a.drain, hist); break;
        }
    }
#undef HGB_LAUNCH
    HGB_LAUNCHED(c, "fill");
    return HGB_OK;
}

hgb_status launch_fill(hgb_ctx* c, const FillPlan& p, const FillArgs& a)
{
    if (c->bin_bytes == 1)
        return p.acc == kPacked ? launch_fill_acc<uint8_t, kPacked>(c, p, a)
                                : launch_fill_acc<uint8_t, kWide>(c, p, a);
    return p.acc == kPacked ? launch_fill_acc<uint16_t, kPacked>(c, p, a)
                            : launch_fill_acc<uint16_t, kWide>(c, p, a);
}

}  // namespace

extern "C" {

int hgb_available(void)
{
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) return 0;
    return n > 0 ? 1 : 0;
}

hgb_status hgb_create(int device, void* hip_stream, hgb_ctx** out)
{
    if (!out) return HGB_E_INVALID;
    *out = nullptr;
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return HGB_E_DEVICE;
    if (device < 0 || device >= n) return HGB_E_INVALID;
    if (hipSetDevice(device) != hipSuccess) return HGB_E_DEVICE;
    hgb_ctx* c = new hgb_ctx();
    c->device = device;
    if (const char* e = std::getenv("HGB_DEBUG_PLAN")) c->debug_plan = e[0] == '1';
    if (const char* e = std::getenv("HGB_FILL_TUNE")) {
        static const char* keys[7] = {"root_lc", "root_tile", "root_ipc", "level_lc", "level_tile", "level_ipc", "align"};
        std::string spec(e);
        size_t pos = 0;
        while (pos < spec.size()) {
            size_t end = spec.find(',', pos);
            if (end == std::string::npos) end = spec.size();
            const std::string kv = spec.substr(pos, end - pos);
            const size_t eq = kv.find('=');
            if (eq != std::string::npos)
                for (int k = 0; k < 7; ++k)
                    if (kv.compare(0, eq, keys[k]) == 0) c->tune[k] = std::atoi(kv.c_str() + eq + 1);
            pos = end + 1;
        }
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
        c->n_cu = prop.multiProcessorCount;
    c->stream = (hipStream_t)hip_stream;
    if (hipMalloc((void**)&c->dev_words, 64) != hipSuccess ||
        hipHostMalloc((void**)&c->host_words, 64, hipHostMallocDefault) != hipSuccess ||
        hipMemset(c->dev_words, 0, 64) != hipSuccess) {
        hgb_destroy(c);
        return HGB_E_DEVICE;
    }
    *out = c;
    return HGB_OK;
}

void hgb_destroy(hgb_ctx* c)
{
    if (!c) return;
    // Best-effort teardown: errors here have nowhere to go.
    (void)hipSetDevice(c->device);
    (void)hipStreamSynchronize(c->stream);
    for (Stage& s : c->stage) {
        if (s.ev) (void)hipEventDestroy(s.ev);
        if (s.host) (void)hipHostFree(s.host);
        if (s.dev) (void)hipFree(s.dev);
    }
    for (auto& v : c->ev_pending)
        for (auto& pr : v) {
            (void)hipEventDestroy(pr.first);
            (void)hipEventDestroy(pr.second);
        }
    for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
    (void)hipFree(c->bins);
    (void)hipFree(c->bins_rm);
    (void)hipFree(c->q);
    (void)hipFree(c->gh);
    (void)hipFree(c->best);
    (void)hipFree(c->totals);
    (void)hipFree(c->dev_words);
    (void)hipHostFree(c->host_words);
    delete c;
}

const char* hgb_last_error(const hgb_ctx* c)
{
    return c ? c->err.c_str() : "null context";
}

hgb_status hgb_sync(hgb_ctx* c)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    HGB_HIP(c, hipSetDevice(c->device));
    HGB_HIP(c, hipMemcpyAsync(c->host_words + 2, c->dev_words + 2, 4, hipMemcpyDeviceToHost,
                              c->stream));
    HGB_HIP(c, hipStreamSynchronize(c->stream));
    uint32_t flags = c->host_words[2];
    if (flags) {
        k_clear_u32<<<1, 64, 0, c->stream>>>(c->dev_words + 2, 1);
        HGB_LAUNCHED(c, "k_clear_u32");
        HGB_HIP(c, hipStreamSynchronize(c->stream));
        if (flags & kErrRowIndex)
            return fail(c, HGB_E_INVALID, "a row index outside [0, n_rows) was skipped");
    }
    return HGB_OK;
}

hgb_status hgb_upload_bins(hgb_ctx* c, const void* bins, int bin_bytes, int on_device,
                           int32_t n_rows, int32_t n_features, int32_t n_bins,
                           int32_t has_missing)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!bins || n_rows <= 0 || n_features <= 0 || n_bins <= 0)
        return fail(c, HGB_E_INVALID, "upload_bins: empty matrix or null pointer");
    if (bin_bytes != 1 && bin_bytes != 2)
        return fail(c, HGB_E_INVALID, "upload_bins: bin_bytes must be 1 or 2");
    if (n_features > 0xffff) return fail(c, HGB_E_UNSUPPORTED, "upload_bins: more than 65535 features");
    const int S = n_bins + (has_missing ? 1 : 0);
    const int max_value = bin_bytes == 1 ? 255 : 65535;
    if (S - 1 > max_value)
        return fail(c, HGB_E_INVALID, "upload_bins: %d slots do not fit %d-byte bins", S, bin_bytes);
    if (S > HGB_MAX_SLOTS)
        return fail(c, HGB_E_UNSUPPORTED, "upload_bins: %d slots exceed the LDS plan (%d)", S,
                    HGB_MAX_SLOTS);
    HGB_HIP(c, hipSetDevice(c->device));
    c->have_tree = false;
    c->have_data = false;
    const int64_t total = (int64_t)n_rows * n_features;
    const size_t bytes = (size_t)total * bin_bytes;
    HGB_HIP(c, hipStreamSynchronize(c->stream));
    if (c->bins) {
        HGB_HIP(c, hipFree(c->bins));
        c->bins = nullptr;
    }
    if (c->bins_rm) {
        HGB_HIP(c, hipFree(c->bins_rm));
        c->bins_rm = nullptr;
    }
    HGB_HIP(c, hipMalloc(&c->bins, bytes));
    HGB_HIP(c, hipMemcpyAsync(c->bins, bins, bytes,
                              on_device ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                              c->stream));
    k_clear_u32<<<1, 64, 0, c->stream>>>(c->dev_words, 1);
    HGB_LAUNCHED(c, "k_clear_u32");
    const int grid = grid_for(total, 256, 4096);
    if (bin_bytes == 1)
        k_bins_max<uint8_t><<<grid, 256, 0, c->stream>>>((const uint8_t*)c->bins, total, c->dev_words);
    else
        k_bins_max<uint16_t><<<grid, 256, 0, c->stream>>>((const uint16_t*)c->bins, total, c->dev_words);
    HGB_LAUNCHED(c, "k_bins_max");
    HGB_HIP(c, hipMemcpyAsync(c->host_words, c->dev_words, 4, hipMemcpyDeviceToHost, c->stream));
    HGB_HIP(c, hipStreamSynchronize(c->stream));
    if (c->host_words[0] >= (uint32_t)S)
        return fail(c, HGB_E_INVALID, "upload_bins: stored value %u is not a slot (S = %d)",
                    c->host_words[0], S);
    if ((int64_t)n_features * bin_bytes <= kRowMajorMaxRowBytes) {
        const int64_t stride = ((int64_t)n_features * bin_bytes + 15) / 16 * 16;
        HGB_HIP(c, hipMalloc(&c->bins_rm, (size_t)(stride * n_rows)));
        HGB_HIP(c, hipMemsetAsync(c->bins_rm, 0, (size_t)(stride * n_rows), c->stream));
        c->rm_stride = stride;
        dim3 tgrid((unsigned)((n_rows + 63) / 64), (unsigned)((n_features + 63) / 64));
        if (bin_bytes == 1)
            k_transpose<uint8_t><<<tgrid, 256, 0, c->stream>>>((const uint8_t*)c->bins,
                                                              (uint8_t*)c->bins_rm, n_rows, n_features, stride);
        else
            k_transpose<uint16_t><<<tgrid, 256, 0, c->stream>>>((const uint16_t*)c->bins,
                                                               (uint8_t*)c->bins_rm, n_rows, n_features, stride);
        HGB_LAUNCHED(c, "k_transpose");
    }
    c->bin_bytes = bin_bytes;
    c->n = n_rows;
    c->F = n_features;
    c->B = n_bins;
    c->S = S;
    c->has_missing = has_missing ? 1 : 0;
    c->have_data = true;
    return HGB_OK;
}

hgb_status hgb_begin_tree(hgb_ctx* c, const float* grad, const float* hess)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_data) return fail(c, HGB_E_STATE, "begin_tree before upload_bins");
    if (!grad || !hess) return fail(c, HGB_E_INVALID, "begin_tree: null gradient pointer");
    HGB_HIP(c, hipSetDevice(c->device));
    c->have_tree = false;
    hgb_status st = grow(c, &c->q, &c->q_cap, c->n);
    if (st != HGB_OK) return st;
    k_clear_u32<<<1, 64, 0, c->stream>>>(c->dev_words, 2);
    HGB_LAUNCHED(c, "k_clear_u32");
    const int vec = ((uintptr_t)grad % 16 == 0 && (uintptr_t)hess % 16 == 0) ? 1 : 0;
    {
        ProfScope ps(c, HGB_KERNEL_QUANTIZE);
        k_grad_hess_max<<<grid_for((c->n + 3) / 4, 256, 1024), 256, 0, c->stream>>>(grad, hess, c->n,
                                                                                 vec, c->dev_words);
    }
    HGB_LAUNCHED(c, "k_grad_hess_max");
    HGB_HIP(c, hipMemcpyAsync(c->host_words, c->dev_words, 8, hipMemcpyDeviceToHost, c->stream));
    HGB_HIP(c, hipStreamSynchronize(c->stream));
    const uint32_t pg = c->host_words[0], ph = c->host_words[1];
    if (pg >= 0x7f800000u) return fail(c, HGB_E_NONFINITE, "begin_tree: NaN or Inf gradient");
    if (ph >= 0x7f800000u)
        return fail(c, HGB_E_NONFINITE, "begin_tree: NaN, Inf or negative hessian");
    int k[2];
    const uint32_t pat[2] = {pg, ph};
    for (int i = 0; i < 2; ++i) {
        float m;
        std::memcpy(&m, &pat[i], 4);
        if (m == 0.0f) {
            k[i] = 0;
        } else {
            int e = 0;
            (void)std::frexp((double)m, &e);
            k[i] = c->precision - e;
        }
    }
    c->k_g = k[0];
    c->k_h = k[1];
    {
        ProfScope ps(c, HGB_KERNEL_QUANTIZE);
        k_quantize<<<grid_for((c->n + 3) / 4, 256, 8192), 256, 0, c->stream>>>(
            grad, hess, c->n, vec, std::ldexp(1.0, k[0]), std::ldexp(1.0, k[1]), c->q);
    }
    HGB_LAUNCHED(c, "k_quantize");
    c->have_tree = true;
    return HGB_OK;
}

hgb_status hgb_set_precision(hgb_ctx* c, int32_t bits)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (bits < 1 || bits > 30)
        return fail(c, HGB_E_INVALID, "set_precision: bits must be in [1, 30]");
    c->precision = bits;
    c->have_tree = false;
    return HGB_OK;
}

hgb_status hgb_get_scales(const hgb_ctx* c, int32_t* k_g, int32_t* k_h)
{
    if (!c || !k_g || !k_h) return HGB_E_INVALID;
    if (!c->have_tree) return HGB_E_STATE;
    *k_g = c->k_g;
    *k_h = c->k_h;
    return HGB_OK;
}

hgb_status hgb_build_level(hgb_ctx* c, const int32_t* row_index, const int32_t* node_offsets,
                           int32_t n_nodes, int64_t* hist, const int32_t* out_slot)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_tree) return fail(c, HGB_E_STATE, "build_level before begin_tree");
    if (!hist) return fail(c, HGB_E_INVALID, "build_level: null histogram buffer");
    if (n_nodes < 1 || n_nodes > 65535)
        return fail(c, HGB_E_INVALID, "build_level: n_nodes must be in [1, 65535]");
    // The root is row_index == NULL with node_offsets == NULL.  With offsets
    // given, row_index may be NULL only when every node is empty.
    const bool root = !row_index && !node_offsets;
    if (row_index && !node_offsets)
        return fail(c, HGB_E_INVALID, "build_level: node_offsets required with row_index");
    if (root && n_nodes != 1)
        return fail(c, HGB_E_INVALID, "build_level: the root (no row index) is one node");
    std::vector<int64_t> begin(n_nodes), count(n_nodes);
    if (root) {
        begin[0] = 0;
        count[0] = c->n;
    } else {
        if (node_offsets[0] != 0) return fail(c, HGB_E_INVALID, "build_level: offsets must start at 0");
        for (int i = 0; i < n_nodes; ++i) {
            if (node_offsets[i + 1] < node_offsets[i])
                return fail(c, HGB_E_INVALID, "build_level: offsets decrease at node %d", i);
            begin[i] = node_offsets[i];
            count[i] = (int64_t)node_offsets[i + 1] - node_offsets[i];
        }
        if (!row_index && node_offsets[n_nodes] != 0)
            return fail(c, HGB_E_INVALID, "build_level: row_index is NULL but the nodes hold rows");
    }
    std::vector<int32_t> slots(n_nodes);
    for (int i = 0; i < n_nodes; ++i) {
        slots[i] = out_slot ? out_slot[i] : i;
        if (slots[i] < 0) return fail(c, HGB_E_INVALID, "build_level: negative output slot");
    }
    {
        std::vector<int32_t> sorted = slots;
        std::sort(sorted.begin(), sorted.end());
        if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
            return fail(c, HGB_E_INVALID, "build_level: two nodes share an output slot");
    }
    HGB_HIP(c, hipSetDevice(c->device));
    const int64_t total = root ? c->n : (int64_t)node_offsets[n_nodes];
    // The root reads rows in order; other levels read through the row index,
    // from the row-major copy when there is one.
    const bool rm = !root && c->bins_rm != nullptr;
    const FillPlan plan0 = plan_fill(c, root, rm);
    const int64_t node_elems = (int64_t)c->F * c->S * 2;

    // Feature tiles (f0, width).  Root tiles have exactly the kernel's width:
    // full tiles of plan.tile, then the remainder split into powers of two,
    // each width its own launch.  Level tiles are plan.tile wide, the last one
    // possibly narrower (those kernels take the width at run time).
    std::vector<std::pair<int, int>> tiles;
    FillPlan plan = plan0;
    if (root) {
        // equal tiles when a divisor of F close to the planned width exists
        for (int d = plan.tile; d >= 1 && 2 * d > plan.tile; --d)
            if (c->F % d == 0) {
                plan.tile = d;
                break;
            }
    }
    {
        int f0 = 0;
        for (; f0 + plan.tile <= c->F; f0 += plan.tile) tiles.emplace_back(f0, plan.tile);
        if (f0 < c->F) {
            if (root) {
                for (int wdt = plan.tile >> 1; wdt >= 1; wdt >>= 1)
                    if (f0 + wdt <= c->F) {
                        tiles.emplace_back(f0, wdt);
                        f0 += wdt;
                    }
            } else {
                tiles.emplace_back(f0, c->F - f0);
            }
        }
    }
    const int n_tiles = (int)tiles.size();
    for (const auto& t : tiles)
        if (t.second < 1 || (root && t.second > 8) || t.first + t.second > c->F)
            return fail(c, HGB_E_DEVICE, "build_level: internal error in the tile plan");

    // Rows per item: about (items per CU) x (CUs) items of equal size over the
    // level, a multiple of 8 rows (the root's vector groups).
    int64_t ipc = root ? kRootItemsPerCu : kLevelItemsPerCu;
    if (c->tune[root ? 2 : 5] > 0) ipc = c->tune[root ? 2 : 5];
    const int64_t target = ipc * c->n_cu;
    // Item boundaries on 128-row multiples keep the root's bin and (g, h)
    // loads cache-line aligned.
    int64_t align = 128;
    if (c->tune[6] > 0) align = (c->tune[6] + 7) / 8 * 8;
    int64_t ch = (total * n_tiles + target - 1) / target;
    ch = std::max<int64_t>((ch + align - 1) / align * align, align);

    // Item order decides which items share an L2 (the kernel gives each XCD a
    // contiguous run).  Root and row-major levels: (node, chunk, tile) -- the
    // tiles of one row chunk read the same rows.  Feature-major levels:
    // (tile, chunk, node) -- the nodes of one tile read the same columns.
    // groups[w]: the items of root tiles of width w (one launch each; root
    // widths are 1, 2, 4 or 8).  Level items all go to groups[0].
    std::vector<FillItem> groups[9];
    std::vector<int32_t> zero_slots;
    std::vector<int64_t> nchunks(n_nodes);
    int64_t max_ch = 0;
    for (int i = 0; i < n_nodes; ++i) {
        nchunks[i] = (count[i] + ch - 1) / ch;
        max_ch = std::max(max_ch, nchunks[i]);
        if (count[i] == 0 || nchunks[i] > 1) zero_slots.push_back(slots[i]);
    }
    size_t n_items = 0;
    auto push = [&](int i, int64_t j, int t) {
        FillItem it{};
        it.out_slot = slots[i];
        it.row_begin = (int32_t)(begin[i] + j * ch);
        it.row_end = (int32_t)std::min<int64_t>(begin[i] + (j + 1) * ch, begin[i] + count[i]);
        it.f0_nf = tiles[t].first | (tiles[t].second << 16);
        it.atomic_merge = nchunks[i] > 1 ? 1 : 0;
        groups[root ? tiles[t].second : 0].push_back(it);
        ++n_items;
    };
    if (plan.kind != kFillCols) {
        for (int i = 0; i < n_nodes; ++i)
            for (int64_t j = 0; j < nchunks[i]; ++j)
                for (int t = 0; t < n_tiles; ++t) push(i, j, t);
    } else {
        for (int t = 0; t < n_tiles; ++t)
            for (int64_t j = 0; j < max_ch; ++j)
                for (int i = 0; i < n_nodes; ++i)
                    if (j < nchunks[i]) push(i, j, t);
    }
    if (n_items > (size_t)INT32_MAX / 8)
        return fail(c, HGB_E_UNSUPPORTED, "build_level: too many fill items");
    if (c->debug_plan)
        std::fprintf(stderr,
                     "[hgb] fill kind %d acc %d copies %d tile %d lt %d drain %d chunk %lld items %zu lds %zu\n",
                     (int)plan.kind, plan.acc, 1 << plan.lc, plan.tile, plan.lt, plan.drain, (long long)ch,
                     n_items, plan.lds_bytes);
    const int2* gh = c->q;
    if (!root) {
        hgb_status st = grow(c, &c->gh, &c->gh_cap, std::max<int64_t>(total, 1));
        if (st != HGB_OK) return st;
        if (total > 0) {
            ProfScope ps(c, HGB_KERNEL_GATHER);
            k_gather<<<grid_for(total, 256, 8192), 256, 0, c->stream>>>(c->q, row_index, total, c->n,
                                                                        c->gh, c->dev_words + 2);
            HGB_LAUNCHED(c, "k_gather");
        }
        gh = c->gh;
    }
    if (!zero_slots.empty()) {
        Stage* s = nullptr;
        hgb_status st = stage_upload(c, zero_slots.data(), zero_slots.size() * sizeof(int32_t), &s);
        if (st != HGB_OK) return st;
        dim3 grid(grid_for(node_elems, 256, 1024), (unsigned)zero_slots.size());
        {
            ProfScope ps(c, HGB_KERNEL_ZERO);
            k_zero_slices<<<grid, 256, 0, c->stream>>>(hist, (const int32_t*)s->dev, node_elems);
        }
        HGB_LAUNCHED(c, "k_zero_slices");
        st = stage_release(c, s);
        if (st != HGB_OK) return st;
    }
    for (int wdt = 8; wdt >= 0; --wdt) {
        std::vector<FillItem>& items = groups[wdt];
        if (items.empty()) continue;
        Stage* s = nullptr;
        hgb_status st = stage_upload(c, items.data(), items.size() * sizeof(FillItem), &s);
        if (st != HGB_OK) return st;
        FillPlan gp = plan;
        if (root && wdt > 0) {
            gp.tile = wdt;
            gp.lds_bytes = (size_t)(wdt * feature_lds(plan.acc, c->S, plan.lc));
        }
        FillArgs a;
        a.gh = gh;
        a.row_index = row_index;
        a.items = (const FillItem*)s->dev;
        a.n_items = (int)items.size();
        // 8-row vector loads of the root need rows aligned to 8 (chunk starts
        // are multiples of 8)
        a.vec_ok = (c->n % 8 == 0) ? 1 : 0;
        a.drain = std::max(plan.drain, 1);
        a.hist = hist;
        ProfScope ps(c, HGB_KERNEL_FILL);
        st = launch_fill(c, gp, a);
        if (st != HGB_OK) return st;
        st = stage_release(c, s);
        if (st != HGB_OK) return st;
    }
    return HGB_OK;
}

hgb_status hgb_subtract_siblings(hgb_ctx* c, const int64_t* parent, int64_t* child,
                                 const uint8_t* built_is_right, const int32_t* parent_slot,
                                 int32_t n_pairs)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_data) return fail(c, HGB_E_STATE, "subtract_siblings before upload_bins");
    if (n_pairs < 0 || n_pairs > 65535)
        return fail(c, HGB_E_INVALID, "subtract_siblings: n_pairs out of range");
    if (n_pairs == 0) return HGB_OK;
    if (!parent || !child || !built_is_right)
        return fail(c, HGB_E_INVALID, "subtract_siblings: null pointer");
    // per pair: parent slot (int32) and built side, staged together
    std::vector<int32_t> plan(2 * (size_t)n_pairs);
    for (int i = 0; i < n_pairs; ++i) {
        const int32_t ps = parent_slot ? parent_slot[i] : i;
        if (ps < 0) return fail(c, HGB_E_INVALID, "subtract_siblings: negative parent slot");
        plan[2 * i] = ps;
        plan[2 * i + 1] = built_is_right[i] ? 1 : 0;
    }
    HGB_HIP(c, hipSetDevice(c->device));
    Stage* s = nullptr;
    hgb_status st = stage_upload(c, plan.data(), plan.size() * sizeof(int32_t), &s);
    if (st != HGB_OK) return st;
    const int64_t pair_vec = (int64_t)c->F * c->S;   // longlong2 per slot
    dim3 grid(grid_for(pair_vec, 256, 2048), (unsigned)n_pairs);
    {
        ProfScope ps(c, HGB_KERNEL_SUBTRACT);
        k_subtract<<<grid, 256, 0, c->stream>>>((const longlong2*)parent, (longlong2*)child,
                                                (const int32_t*)s->dev, pair_vec);
    }
    HGB_LAUNCHED(c, "k_subtract");
    return stage_release(c, s);
}

hgb_status hgb_find_splits(hgb_ctx* c, const int64_t* hist, int32_t n_nodes, double lambda,
                           double gamma, hgb_split* out)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_tree) return fail(c, HGB_E_STATE, "find_splits before begin_tree");
    if (n_nodes < 0 || n_nodes > 65535)
        return fail(c, HGB_E_INVALID, "find_splits: n_nodes out of range");
    if (!(lambda >= 0.0) || !std::isfinite(lambda) || !std::isfinite(gamma))
        return fail(c, HGB_E_INVALID, "find_splits: lambda must be finite and >= 0, gamma finite");
    if (n_nodes == 0) return HGB_OK;
    if (!hist || !out) return fail(c, HGB_E_INVALID, "find_splits: null pointer");
    HGB_HIP(c, hipSetDevice(c->device));
    hgb_status st = grow(c, &c->best, &c->best_cap, (int64_t)n_nodes * c->F);
    if (st != HGB_OK) return st;
    st = grow(c, &c->totals, &c->totals_cap, (int64_t)2 * n_nodes);
    if (st != HGB_OK) return st;
    const int waves = 4;
    dim3 grid((c->F + waves - 1) / waves, (unsigned)n_nodes);
    ProfScope ps(c, HGB_KERNEL_SPLIT);
    k_split_feature<<<grid, waves * kWave, 0, c->stream>>>(
        (const long long*)hist, c->F, c->B, c->S, c->has_missing, std::ldexp(1.0, -c->k_g),
        std::ldexp(1.0, -c->k_h), lambda, gamma, c->best, c->totals);
    HGB_LAUNCHED(c, "k_split_feature");
    static_assert(sizeof(SplitOut) == sizeof(hgb_split), "split record layout");
    k_split_reduce<<<(unsigned)n_nodes, 256, 0, c->stream>>>(c->best, c->totals, c->F,
                                                             (SplitOut*)out);
    HGB_LAUNCHED(c, "k_split_reduce");
    return HGB_OK;
}

hgb_status hgb_profile_enable(hgb_ctx* c, int enable)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    HGB_HIP(c, hipSetDevice(c->device));
    HGB_HIP(c, hipStreamSynchronize(c->stream));
    for (int k = 0; k < HGB_KERNEL_COUNT; ++k) {
        for (auto& pr : c->ev_pending[k]) {
            c->ev_pool.push_back(pr.first);
            c->ev_pool.push_back(pr.second);
        }
        c->ev_pending[k].clear();
        c->prof_ms[k] = 0.0;
        c->prof_launches[k] = 0;
    }
    c->prof = enable != 0;
    return HGB_OK;
}

hgb_status hgb_profile_query(hgb_ctx* c, int kernel, double* total_ms, int64_t* launches)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (kernel < 0 || kernel >= HGB_KERNEL_COUNT || !total_ms || !launches)
        return fail(c, HGB_E_INVALID, "profile_query: bad kernel id or null output");
    HGB_HIP(c, hipSetDevice(c->device));
    HGB_HIP(c, hipStreamSynchronize(c->stream));
    for (int k = 0; k < HGB_KERNEL_COUNT; ++k) {
        for (auto& pr : c->ev_pending[k]) {
            float ms = 0.0f;
            HGB_HIP(c, hipEventElapsedTime(&ms, pr.first, pr.second));
            c->prof_ms[k] += ms;
            c->prof_launches[k] += 1;
            c->ev_pool.push_back(pr.first);
            c->ev_pool.push_back(pr.second);
        }
        c->ev_pending[k].clear();
    }
    *total_ms = c->prof_ms[kernel];
    *launches = c->prof_launches[kernel];
    return HGB_OK;
}

}  // extern "C"
