// hgb: C ABI of the level histogram build (see include/hgb.h for the contract).
//
// Host side of the library: the context, argument validation, per-call launch
// planning and the staging of small plans to the device.  The kernels live in
// hgb_kernels.h.
#include "hgb.h"
#include "hgb_kernels.h"
#include "hgb_plan.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

using namespace hgb;

namespace {

// (The fill planner's constants are in hgb_plan.h.)
// A feature's top slot is hot when it holds at least 1/kHotSlotShare of the rows.
constexpr int64_t kHotSlotShare = 16;
// Rows up to this many bytes get a row-major copy (16,384 one-byte features
// included): below the root, a level reads only its built rows' lines from it.
constexpr int64_t kRowMajorMaxRowBytes = 65536;
constexpr int64_t kRowMajorSlack = 32;   // >= the widest row-tile load
// A row of the row-major copy is padded to a multiple of 16 bytes, and by
// kRowMajorSkew more when that is a multiple of kRowMajorSkewPeriod: with a
// stride of a large power of two (16,384 one-byte features), one tile's
// chunks of every row share their low address bits, and the level fill that
// reads them ran 15% slower (131,072 x 16,384, one lane per row: 0.60
// against 0.51 ms).
constexpr int64_t kRowMajorSkew = 128;
constexpr int64_t kRowMajorSkewPeriod = 1024;
constexpr int64_t kTransposeMaxBlocks = 65536;   // k_transpose's blocks per feature group (they stride)
// begin_tree's max pass: at most this many blocks, each writing its pair of
// maxima for k_max_final.
constexpr int kMaxBlocks = 4096;
// Default fixed-point precision of begin_tree (bits below the largest value).
constexpr int kDefaultPrecision = 30;
constexpr int kStages = 16;
constexpr int kEpochEvents = 4;
constexpr int kEpochUses = 6;
// Pinned host words (host_words, 16 of them): [0..1] the maxima, [2] the
// error word, and the sequence numbers kernels post after their results.
constexpr int kHostTreeSeq = 8;
constexpr int kHostPartSeq = 9;

// Initial capacity of an upload stage: larger than any level's plan of the
// matrices measured here (the level-3 plan of 131,072 x 16,384 is about 70 KB).
constexpr size_t kStageMinBytes = 256 * 1024;

// Scratch of hgb_find_splits_noalloc: one array per device, held until the
// process ends.  In host code `scratch` is only a stand-in for the device
// array: hgb_create looks up its address on each device (hipGetSymbolAddress)
// and every host use goes through that address.
constexpr size_t kNoAllocScratchBytes = HGB_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_dev;   // per device: the address of `scratch` there

struct Stage {
    void* host = nullptr;   // pinned
    void* dev = nullptr;
    size_t cap = 0;
    uint64_t release_seq = 0;    // the context's release count when its consumers were enqueued
    bool pending = false;
    const void* use = nullptr;   // what the kernels read: dev, or the pinned host copy
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
    // hgb_set_async_begin: begin_tree returns without waiting for the maxima;
    // the host reads them (and checks them) at the next call that needs them
    bool async_begin = false;
    bool scales_pending = false;          // the current tree's maxima are not read yet
    int tree_precision = 30;              // the precision the current tree was started with
    hgb_status deferred = HGB_OK;         // a started tree's non-finite values, for hgb_sync
    std::string deferred_msg;

    // level scratch
    int2* gh = nullptr;
    int64_t gh_cap = 0;
    long long* partial = nullptr;   // partial histograms of nodes split over several blocks
    int64_t partial_cap = 0;
    int32_t* part = nullptr;        // partition: chunk counts, left bases, per-node records
    int64_t part_cap = 0;
    int32_t* part_host = nullptr;   // pinned copy of the per-node records
    int64_t part_host_cap = 0;
    uint8_t* part_flags = nullptr;  // partition: direction of each position (1 = left)
    int64_t part_flags_cap = 0;
    FeatureBest* best = nullptr;
    int64_t best_cap = 0;
    long long* totals = nullptr;
    int64_t totals_cap = 0;
    double* level_terms = nullptr;        // find_level_split: [n_nodes][candidates] gains
    int64_t level_terms_cap = 0;
    LevelBest* level_best = nullptr;      // find_level_split: per-block winners
    int64_t level_best_cap = 0;

    // this device's copy of the no-allocation scratch array (set up by hgb_create)
    unsigned char* noalloc_scratch = nullptr;

    // small device words: [0..1] max patterns, [2] error flags, [3] 1 when the
    // quantize pass must encode the rows again, [4..11] the quantize scales
    // 2^k (also the next tree's guess) and the split scales 2^-k (four doubles)
    uint32_t* dev_words = nullptr;
    uint32_t* host_words = nullptr;   // pinned
    uint32_t* max_part = nullptr;     // begin_tree: per-block maxima, 2 x kMaxBlocks
    int32_t* rot = nullptr;           // per feature: the skipped slot (stored bins are rotated by it)
    bool skip = false;                // the fills skip each feature's slot 0 (a hot slot exists)
    hipEvent_t host_ready = nullptr;  // hgb_sync: the stream has drained

    Stage stage[kStages];
    int stage_next = 0;
    // Stage releases record no event of their own (an event on the stream
    // costs the device about 3 us): every kEpochUses releases, one event of a
    // small ring marks the stream, and a stage is reused once an event
    // recorded after its release has passed.
    uint64_t stage_seq = 0;                     // releases so far
    hipEvent_t epoch_ev[kEpochEvents] = {};
    uint64_t epoch_seq[kEpochEvents] = {};      // releases covered by each event
    int epoch_next = 0;
    uint64_t last_epoch_seq = 0;
    // sequence numbers of the results kernels post to pinned host memory:
    // the maxima of each tree (host_words[8]) and the node records of each
    // partition (host_words[9])
    uint32_t tree_seq = 0;
    uint32_t part_seq = 0;

    // HGB_DEBUG_PLAN=1 in the environment prints each fill plan to stderr
    bool debug_plan = false;
    // kernels read the launch plans from pinned host memory (HGB_PLAN_HOST=0:
    // from a device copy)
    bool plan_host = true;
    // HGB_FILL_TUNE="key=value,..." overrides the fill planner (developer
    // tuning): root_lc, root_tile, root_ipc, level_lc, level_tile, level_ipc
    // (ipc = items per CU), align (rows an item boundary is a multiple of),
    // piece (fixed cost of a level item, in rows), il (row-major level fill,
    // wide sums) and root_il (root fill, wide or packed sums): 1 slot-major
    // interleaved tile, 0 feature-major; pair (row-major interleaved level
    // fills with 32-byte chunks: 1 two lanes per row, 0 one); -1 keeps the
    // planner's choice.
    int tune[kTuneKeys] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};

    // optional per-kernel timing
    bool prof = false;
    std::vector<hipEvent_t> ev_pool;
    // kernels whose dynamic-LDS limit has been raised, and to what
    std::vector<std::pair<const void*, size_t>> lds_set;
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

// Wait for `ev`: poll it for up to kPollMicros, then block.  A level loop
// waits for small results (maxima, node records) several times per tree, most
// of them ready within tens of microseconds, where a blocking wait would add
// the host's wake-up latency; a longer wait (a large level still running)
// blocks instead of holding a host core.
constexpr int64_t kPollMicros = 200;

hgb_status poll_event(hgb_ctx* c, hipEvent_t ev)
{
    const auto t0 = std::chrono::steady_clock::now();
    for (;;) {
        const hipError_t e = hipEventQuery(ev);
        if (e == hipSuccess) return HGB_OK;
        if (e != hipErrorNotReady) return fail(c, HGB_E_DEVICE, "HIP error: %s", hipGetErrorString(e));
        const auto waited = std::chrono::steady_clock::now() - t0;
        if (std::chrono::duration_cast<std::chrono::microseconds>(waited).count() >= kPollMicros) break;
    }
    HGB_HIP(c, hipEventSynchronize(ev));
    return HGB_OK;
}

// Wait until a kernel has stored `want` into the pinned word w (its last
// store, after the results it hands the host): poll for up to kPollMicros,
// then keep polling but yield the core between checks (a sleep would wake
// tens of microseconds late, and the device waits for the host's next
// launches).  Every 64th check also asks the stream: one that has drained
// without the store (a launch that failed) is an error, not a hang.
hgb_status wait_word(hgb_ctx* c, const uint32_t* w, uint32_t want)
{
    const volatile uint32_t* vw = w;
    const auto t0 = std::chrono::steady_clock::now();
    bool spin = true;
    for (uint64_t i = 0;; ++i) {
        if (*vw == want) {
            std::atomic_thread_fence(std::memory_order_acquire);
            return HGB_OK;
        }
        if (spin) {
            const auto waited = std::chrono::steady_clock::now() - t0;
            spin = std::chrono::duration_cast<std::chrono::microseconds>(waited).count() < kPollMicros;
            continue;
        }
        if ((i & 63) == 0) {
            const hipError_t e = hipStreamQuery(c->stream);
            if (*vw == want) continue;   // (taken at the top)
            if (e == hipSuccess) return fail(c, HGB_E_DEVICE, "the stream drained without a kernel's result");
            if (e != hipErrorNotReady) return fail(c, HGB_E_DEVICE, "HIP error: %s", hipGetErrorString(e));
        }
        std::this_thread::yield();
    }
}

// Mark the stream with the next event of the epoch ring: it covers every
// stage released so far.
hgb_status record_epoch(hgb_ctx* c)
{
    const int k = c->epoch_next;
    if (!c->epoch_ev[k]) HGB_HIP(c, hipEventCreateWithFlags(&c->epoch_ev[k], hipEventDisableTiming));
    HGB_HIP(c, hipEventRecord(c->epoch_ev[k], c->stream));
    c->epoch_seq[k] = c->stage_seq;
    c->last_epoch_seq = c->stage_seq;
    c->epoch_next = (k + 1) % kEpochEvents;
    return HGB_OK;
}

// Stage `bytes` of host data (a launch plan: items, slot lists) for the
// kernels.  By default the kernels read it in place from the stage's pinned
// host buffer: a plan is read once per block, and a copy kernel on the stream
// would sit between a level's kernels (in place measured 1% faster for the
// 10M x 28 tree, 6% for the grown one, whose next level is planned while the
// device waits).  HGB_PLAN_HOST=0 copies it to the stage's device buffer on
// the stream instead.  The stage is released by stage_release after its
// consumers have been enqueued; it is reused only once an epoch event
// recorded after that release has passed (one is recorded then if none
// was).  (Copies on a second stream ordered by events measured slower than
// either.)
hgb_status stage_upload(hgb_ctx* c, const void* src, size_t bytes, Stage** out)
{
    Stage& s = c->stage[c->stage_next];
    c->stage_next = (c->stage_next + 1) % kStages;
    if (s.pending) {
        // the earliest epoch event that covers the release
        int best = -1;
        for (int k = 0; k < kEpochEvents; ++k)
            if (c->epoch_ev[k] && c->epoch_seq[k] >= s.release_seq &&
                (best < 0 || c->epoch_seq[k] < c->epoch_seq[best]))
                best = k;
        if (best < 0) {
            best = c->epoch_next;
            hgb_status st = record_epoch(c);
            if (st != HGB_OK) return st;
        }
        hgb_status st = poll_event(c, c->epoch_ev[best]);
        if (st != HGB_OK) return st;
        s.pending = false;
    }
    if (bytes > s.cap) {
        // Reallocating pinned memory is slow (and a free synchronizes the
        // device), so a stage starts large and at least doubles.
        if (s.host) HGB_HIP(c, hipHostFree(s.host));
        if (s.dev) HGB_HIP(c, hipFree(s.dev));
        s.host = s.dev = nullptr;
        const size_t want = std::max<size_t>(std::max<size_t>(bytes, 2 * s.cap), kStageMinBytes);
        s.cap = 0;
        // Coherent (fine-grained) pinned memory: the kernels read plans in
        // place, and the host rewrites a stage for later kernels; in default
        // (non-coherent) pinned memory the GPU's L2 may cache its lines.
        HGB_HIP(c, hipHostMalloc(&s.host, want, hipHostMallocCoherent));
        HGB_HIP(c, hipMalloc(&s.dev, want));
        s.cap = want;
    }
    if (bytes) {
        std::memcpy(s.host, src, bytes);
        if (!c->plan_host) HGB_HIP(c, hipMemcpyAsync(s.dev, s.host, bytes, hipMemcpyHostToDevice, c->stream));
    }
    s.use = c->plan_host ? s.host : s.dev;
    *out = &s;
    return HGB_OK;
}

hgb_status stage_release(hgb_ctx* c, Stage* s)
{
    s->release_seq = ++c->stage_seq;
    s->pending = true;
    if (c->stage_seq - c->last_epoch_seq >= (uint64_t)kEpochUses) return record_epoch(c);
    return HGB_OK;
}

// A stage held from its upload until its consumers are enqueued.  release()
// marks it released; on an early (error) return the destructor does, so a
// plan that an already launched kernel reads is never handed out again
// before that kernel is done.
struct StageLease {
    hgb_ctx* c;
    Stage* s = nullptr;
    explicit StageLease(hgb_ctx* ctx) : c(ctx) {}
    StageLease(const StageLease&) = delete;
    StageLease& operator=(const StageLease&) = delete;
    hgb_status release()
    {
        Stage* t = s;
        s = nullptr;
        return t ? stage_release(c, t) : HGB_OK;
    }
    ~StageLease()
    {
        if (s) (void)stage_release(c, s);
    }
};

// Record `*ev` (created on first use) on the stream and poll it.
hgb_status wait_here(hgb_ctx* c, hipEvent_t* ev)
{
    if (!*ev) HGB_HIP(c, hipEventCreateWithFlags(ev, hipEventDisableTiming));
    HGB_HIP(c, hipEventRecord(*ev, c->stream));
    return poll_event(c, *ev);
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

// The current tree's inverse scales 2^-k_g, 2^-k_h on the device, written by
// k_max_final: the split kernels read them there, so no host round trip
// stands between begin_tree and a level's launches.
const double* inv_scales(const hgb_ctx* c) { return (const double*)(c->dev_words + 4) + 2; }

// What the planner (hgb_plan.h) reads of a context.
PlanCtx plan_ctx(const hgb_ctx* c)
{
    PlanCtx pc;
    pc.n = c->n;
    pc.F = c->F;
    pc.S = c->S;
    pc.bin_bytes = c->bin_bytes;
    pc.precision = c->precision;
    pc.skip = c->skip;
    pc.rm_stride = c->bins_rm ? c->rm_stride : 0;
    pc.n_cu = c->n_cu;
    for (int k = 0; k < kTuneKeys; ++k) pc.tune[k] = c->tune[k];
    return pc;
}

template <typename K>
hgb_status set_lds(hgb_ctx* c, K kernel, size_t bytes)
{
    // once per kernel and size: the attribute persists for the process
    const void* fn = (const void*)kernel;
    for (auto& e : c->lds_set)
        if (e.first == fn) {
            if (e.second >= bytes) return HGB_OK;
            HGB_HIP(c, hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes));
            e.second = bytes;
            return HGB_OK;
        }
    HGB_HIP(c, hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes));
    c->lds_set.emplace_back(fn, bytes);
    return HGB_OK;
}

struct FillArgs {
    const int2* gh;
    const int32_t* row_index;
    const FillItem* items;
    int n_items;               // root: one block per item
    const int32_t* block_first;   // levels: items of block b are [block_first[b], block_first[b + 1])
    int n_blocks;
    int vec_ok;
    int drain;
    int64_t* hist;
    int64_t* partial;
    ZeroList zero;   // level fills: node slots the fill clears first
};

template <typename BinT, int ACC, bool SKIP>
hgb_status launch_fill_acc(hgb_ctx* c, const FillPlan& p, const FillArgs& a)
{
    const int n_grid = p.kind == kFillRoot ? a.n_items : a.n_blocks;
    const unsigned grid = (unsigned)(8 * ((n_grid + 7) / 8));
    unsigned long long* partial = (unsigned long long*)a.partial;
    unsigned long long* hist = (unsigned long long*)a.hist;
    const BinT* bins = (const BinT*)c->bins;
    hgb_status st = HGB_OK;
#define HGB_LAUNCH(kern, ...)                                                            \
    do {                                                                                 \
        st = set_lds(c, kern, p.lds_bytes);                                              \
        if (st != HGB_OK) return st;                                                     \
        kern<<<grid, p.threads, p.lds_bytes, c->stream>>>(__VA_ARGS__);                  \
    } while (0)
    if (p.kind == kFillRoot && p.il) {
#define HGB_ROOT_IL_LC(TF, LC0) HGB_LAUNCH((k_fill_root_il<BinT, TF, SKIP, ACC, LC0>), bins, c->n, c->F, c->S, p.lc, a.gh, a.items, a.n_items, a.vec_ok, a.drain, hist, partial, c->rot)
#define HGB_ROOT_IL(TF) do { if (p.lc == 0) HGB_ROOT_IL_LC(TF, true); else HGB_ROOT_IL_LC(TF, false); } while (0)
        if constexpr (ACC == kPacked) {
            // (the plan keeps 16 positions, one-byte bins and no skipped slot)
            if constexpr (!SKIP && sizeof(BinT) == 1) {
                if (p.tile == 16 && p.drain > 0 && (int64_t)c->S * 16 <= (int64_t)kRootIlPackedCells * p.threads) {
                    HGB_ROOT_IL(16);
                } else {
                    return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
                }
            } else {
                return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
            }
        } else {
            // (the plan keeps TF * sizeof(BinT) <= 32, and <= 16 with SKIP)
            constexpr int kMaxBytes = SKIP ? 16 : 32;
            switch (p.tile) {
            case 32:
                if constexpr (32 * sizeof(BinT) <= kMaxBytes) {
                    HGB_ROOT_IL(32);
                    break;
                }
                return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
            case 16:
                if constexpr (16 * sizeof(BinT) <= kMaxBytes) {
                    HGB_ROOT_IL(16);
                    break;
                }
                return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
            case 8: HGB_ROOT_IL(8); break;
            default: return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
            }
        }
#undef HGB_ROOT_IL
#undef HGB_ROOT_IL_LC
    } else if (p.kind == kFillRoot) {
#define HGB_ROOT(NF) HGB_LAUNCH((k_fill_root<BinT, NF, ACC, SKIP>), bins, c->n, c->F, c->S, p.lc, a.gh, a.items, a.n_items, a.vec_ok, a.drain, hist, c->rot)
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
        case 1: HGB_LAUNCH((k_fill_cols<BinT, 1, ACC, SKIP>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.block_first, a.n_blocks, a.drain, hist, partial, c->rot, a.zero); break;
        case 2: HGB_LAUNCH((k_fill_cols<BinT, 2, ACC, SKIP>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.block_first, a.n_blocks, a.drain, hist, partial, c->rot, a.zero); break;
        case 4: HGB_LAUNCH((k_fill_cols<BinT, 4, ACC, SKIP>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.block_first, a.n_blocks, a.drain, hist, partial, c->rot, a.zero); break;
        default: HGB_LAUNCH((k_fill_cols<BinT, 8, ACC, SKIP>), bins, c->n, c->F, c->S, p.lc, a.gh, a.row_index, a.items, a.block_first, a.n_blocks, a.drain, hist, partial, c->rot, a.zero); break;
        }
    } else {
        // row-major: packed sums in registers (ra cells per thread), wide sums in LDS
        const uint8_t* rm = (const uint8_t*)c->bins_rm;
#define HGB_ROWS(LT, RA, E, IL) HGB_ROWS_LC(LT, RA, E, IL, false)
#define HGB_ROWS_LC(LT, RA, E, IL, LC0) HGB_LAUNCH((k_fill_rows<BinT, LT, ACC, RA, E, SKIP, IL, LC0>), rm, c->rm_stride, c->n, c->F, c->S, p.lc, c->q, a.row_index, a.items, a.block_first, a.n_blocks, a.drain, hist, partial, c->dev_words + 2, c->rot, a.zero)
        if constexpr (ACC == kPacked) {
            if (p.ra != kRegAccCells) return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
            switch (p.lt) {
            case 32: HGB_ROWS(32, kRegAccCells, kRegAccEntries, 0); break;
            case 16: HGB_ROWS(16, kRegAccCells, kRegAccEntries, 0); break;
            case 8: HGB_ROWS(8, kRegAccCells, kRegAccEntries, 0); break;
            case 4: HGB_ROWS(4, kRegAccCells, kRegAccEntries, 0); break;
            default: HGB_ROWS(2, kRegAccCells, kRegAccEntries, 0); break;
            }
        } else {
            if (p.ra != 0) return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
            if (p.il == 2) {   // lane pairs: 32-byte chunks only
                if (p.lt != 2 * kPairHalfBytes) return fail(c, HGB_E_DEVICE, "fill: internal error in the plan");
                if (p.lc == 0) HGB_ROWS_LC(32, 0, kWideRowEntries, 2, true);
                else HGB_ROWS(32, 0, kWideRowEntries, 2);
            } else if (p.il) {
                switch (p.lt) {
                case 32: HGB_ROWS(32, 0, kWideRowEntries, 1); break;
                case 16: HGB_ROWS(16, 0, kWideRowEntries, 1); break;
                case 8: HGB_ROWS(8, 0, kWideRowEntries, 1); break;
                case 4: HGB_ROWS(4, 0, kWideRowEntries, 1); break;
                default: HGB_ROWS(2, 0, kWideRowEntries, 1); break;
                }
            } else {
                switch (p.lt) {
                case 32: HGB_ROWS(32, 0, kWideRowEntries, 0); break;
                case 16: HGB_ROWS(16, 0, kWideRowEntries, 0); break;
                case 8: HGB_ROWS(8, 0, kWideRowEntries, 0); break;
                case 4: HGB_ROWS(4, 0, kWideRowEntries, 0); break;
                default: HGB_ROWS(2, 0, kWideRowEntries, 0); break;
                }
            }
        }
#undef HGB_ROWS
#undef HGB_ROWS_LC
    }
#undef HGB_LAUNCH
    HGB_LAUNCHED(c, "fill");
    return HGB_OK;
}

hgb_status launch_fill(hgb_ctx* c, const FillPlan& p, const FillArgs& a)
{
    if (c->skip) {
        if (c->bin_bytes == 1)
            return p.acc == kPacked ? launch_fill_acc<uint8_t, kPacked, true>(c, p, a)
                                    : launch_fill_acc<uint8_t, kWide, true>(c, p, a);
        return p.acc == kPacked ? launch_fill_acc<uint16_t, kPacked, true>(c, p, a)
                                : launch_fill_acc<uint16_t, kWide, true>(c, p, a);
    }
    if (c->bin_bytes == 1)
        return p.acc == kPacked ? launch_fill_acc<uint8_t, kPacked, false>(c, p, a)
                                : launch_fill_acc<uint8_t, kWide, false>(c, p, a);
    return p.acc == kPacked ? launch_fill_acc<uint16_t, kPacked, false>(c, p, a)
                            : launch_fill_acc<uint16_t, kWide, false>(c, p, a);
}

// Sum partial histograms into their nodes' slots: the merge list inline in
// the arguments when it is short, else read from its staged plan.
hgb_status launch_merge(hgb_ctx* c, const std::vector<MergeEntry>& merges, const MergeEntry* staged,
                        dim3 grid, int64_t* hist)
{
    const int64_t node_vec = (int64_t)c->F * c->S;
    MergeInline inl{};
    const MergeEntry* plan = staged;
    if (merges.size() <= (size_t)kMergeInline) {
        std::memcpy(inl.e, merges.data(), merges.size() * sizeof(MergeEntry));
        plan = nullptr;
    }
    k_merge<<<grid, 256, 0, c->stream>>>((const longlong2*)c->partial, (longlong2*)hist, plan, inl, node_vec);
    HGB_LAUNCHED(c, "k_merge");
    return HGB_OK;
}

// Zero whole node slots of the level buffer; the slot list is staged.
hgb_status launch_zero(hgb_ctx* c, int64_t* hist, const int32_t* slots_dev, size_t n_slots)
{
    if (n_slots == 0) return HGB_OK;
    const int64_t node_elems = (int64_t)c->F * c->S * 2;
    dim3 grid(grid_for(node_elems, 256, 1024), (unsigned)n_slots);
    {
        ProfScope ps(c, HGB_KERNEL_ZERO);
        k_zero_slices<<<grid, 256, 0, c->stream>>>(hist, slots_dev, node_elems);
    }
    HGB_LAUNCHED(c, "k_zero_slices");
    return HGB_OK;
}

// Fill of a level below the root: the cut (hgb_plan.h cut_level), then one
// fill launch (which also clears the slots that merges add into, and empty
// nodes' slots) and one merge launch for the nodes split over several blocks.
hgb_status fill_level(hgb_ctx* c, const FillPlan& plan, const std::vector<std::pair<int, int>>& tiles,
                      const int32_t* row_index, const std::vector<int64_t>& begin,
                      const std::vector<int64_t>& count, const std::vector<int32_t>& slots,
                      int64_t total, int64_t* hist)
{
    const int64_t node_elems = (int64_t)c->F * c->S * 2;
    const PlanCtx pc = plan_ctx(c);
    LevelCut cut;
    if (const char* msg = cut_level(&pc, plan, tiles, begin, count, slots, &cut))
        return fail(c, HGB_E_UNSUPPORTED, "%s", msg);
    const std::vector<FillItem>& items = cut.items;
    const std::vector<int32_t>& block_first = cut.block_first;
    const std::vector<MergeEntry>& merges = cut.merges;
    const std::vector<int32_t>& zero_slots = cut.zero_slots;
    const int n_blocks = (int)(block_first.size() - 1);
    if (c->debug_plan)
        std::fprintf(stderr,
                     "[hgb] fill kind %d acc %d copies %d tile %d lt %d ra %d il %d drain %d chunk %lld items %zu "
                     "lds %zu blocks %d partials %lld merges %zu\n",
                     (int)plan.kind, plan.acc, 1 << plan.lc, plan.tile, plan.lt, plan.ra, plan.il, plan.drain,
                     (long long)cut.budget, items.size(), plan.lds_bytes, n_blocks, (long long)cut.n_partial,
                     merges.size());

    hgb_status st = HGB_OK;
    if (cut.n_partial > 0) {
        st = grow(c, &c->partial, &c->partial_cap, cut.n_partial * node_elems);
        if (st != HGB_OK) return st;
    }
    // the row-major fill reads each row's (g, h) itself; the others read
    // them gathered into level order
    if (total > 0 && plan.kind != kFillRowsKind) {
        st = grow(c, &c->gh, &c->gh_cap, total);
        if (st != HGB_OK) return st;
        ProfScope ps(c, HGB_KERNEL_GATHER);
        k_gather<<<grid_for(total, 256, 8192), 256, 0, c->stream>>>(c->q, row_index, total, c->n, c->gh,
                                                                    c->dev_words + 2);
        HGB_LAUNCHED(c, "k_gather");
    }
    if (items.empty() && zero_slots.empty()) return HGB_OK;

    // one upload: items, block list, merges, slots to zero (each part
    // 256-byte aligned)
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t off_blocks = up(items.size() * sizeof(FillItem));
    const size_t off_merges = off_blocks + up(block_first.size() * sizeof(int32_t));
    const size_t off_zero = off_merges + up(merges.size() * sizeof(MergeEntry));
    const size_t bytes = off_zero + zero_slots.size() * sizeof(int32_t);
    std::vector<uint8_t> blob(bytes, 0);
    if (!items.empty()) std::memcpy(blob.data(), items.data(), items.size() * sizeof(FillItem));
    std::memcpy(blob.data() + off_blocks, block_first.data(), block_first.size() * sizeof(int32_t));
    if (!merges.empty())
        std::memcpy(blob.data() + off_merges, merges.data(), merges.size() * sizeof(MergeEntry));
    if (!zero_slots.empty())
        std::memcpy(blob.data() + off_zero, zero_slots.data(), zero_slots.size() * sizeof(int32_t));
    StageLease sg(c);
    st = stage_upload(c, blob.data(), bytes, &sg.s);
    if (st != HGB_OK) return st;
    const uint8_t* dev = (const uint8_t*)sg.s->use;
    if (items.empty()) {   // nothing to fill: the slots to clear get their own launch
        st = launch_zero(c, hist, (const int32_t*)(dev + off_zero), zero_slots.size());
        if (st != HGB_OK) return st;
        return sg.release();
    }
    {
        FillArgs a{};
        // the fill clears the listed slots before k_merge adds into them
        a.zero.slots = (const int32_t*)(dev + off_zero);
        a.zero.n = (int)zero_slots.size();
        a.zero.node_vec = (int64_t)c->F * c->S;
        a.gh = c->gh;
        a.row_index = row_index;
        a.items = (const FillItem*)dev;
        a.block_first = (const int32_t*)(dev + off_blocks);
        a.n_blocks = n_blocks;
        a.drain = std::max(plan.drain, 1);
        a.hist = hist;
        a.partial = (int64_t*)c->partial;
        {
            ProfScope pl(c, HGB_KERNEL_FILL_LEVEL);
            st = launch_fill(c, plan, a);
        }
        if (st != HGB_OK) return st;
        if (!merges.empty()) {
            ProfScope pm(c, HGB_KERNEL_MERGE);
            const int64_t node_vec = (int64_t)c->F * c->S;
            dim3 grid(grid_for(node_vec, 256, 1024), (unsigned)merges.size());
            st = launch_merge(c, merges, (const MergeEntry*)(dev + off_merges), grid, hist);
            if (st != HGB_OK) return st;
        }
    }
    return sg.release();
}

}  // namespace

// The current tree's exponents from the maxima k_max_final wrote into pinned
// host memory (the tree's number has arrived after them).  Returns nullptr, or what
// was not finite.
static const char* read_scales(hgb_ctx* c)
{
    const uint32_t pg = c->host_words[0], ph = c->host_words[1];
    if (pg >= 0x7f800000u) return "begin_tree: NaN or Inf gradient";
    if (ph >= 0x7f800000u) return "begin_tree: NaN, Inf or negative hessian";
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
            k[i] = c->tree_precision - e;
        }
    }
    c->k_g = k[0];
    c->k_h = k[1];
    return nullptr;
}

// A tree started by an asynchronous begin_tree: wait for its maxima, keep
// its exponents, and hold a non-finite value for the next hgb_sync.
static hgb_status resolve_scales(hgb_ctx* c)
{
    if (!c->scales_pending) return HGB_OK;
    const hgb_status st = wait_word(c, c->host_words + kHostTreeSeq, c->tree_seq);
    if (st != HGB_OK) return st;
    c->scales_pending = false;
    if (const char* bad = read_scales(c)) {
        c->deferred = HGB_E_NONFINITE;
        c->deferred_msg = bad;
    }
    return HGB_OK;
}

// Start a tree from any row source: exact maxima of |g| and of h, the scales
// from their exponents (on the device, for the quantize pass and the split
// kernels), then the quantize pass, which re-derives each row's (g, h) from
// the source.  The host reads the maxima back to check them and keep the
// exponents: right away (one wait), or, with async_begin, when a later call
// needs them.
template <class Src>
static hgb_status begin_tree_from(hgb_ctx* c, const Src& src, int vec)
{
    HGB_HIP(c, hipSetDevice(c->device));
    // the previous tree's maxima, before this tree's overwrite them
    hgb_status rst = resolve_scales(c);
    if (rst != HGB_OK) return rst;
    c->have_tree = false;
    hgb_status st = grow(c, &c->q, &c->q_cap, c->n);
    if (st != HGB_OK) return st;
    const int max_blocks = grid_for((c->n + 3) / 4, 256, kMaxBlocks);
    {
        ProfScope ps(c, HGB_KERNEL_QUANTIZE);
        k_grad_hess_max<Src><<<max_blocks, 256, 0, c->stream>>>(src, c->n, vec, c->max_part,
                                                                 (const double*)(c->dev_words + 4), c->q);
        HGB_LAUNCHED(c, "k_grad_hess_max");
        k_max_final<<<1, 256, 0, c->stream>>>(c->max_part, max_blocks, c->dev_words, c->precision,
                                              (double*)(c->dev_words + 4), c->host_words, c->dev_words + 3,
                                              Src::kGuess ? 1 : 0, c->host_words + kHostTreeSeq, ++c->tree_seq);
        HGB_LAUNCHED(c, "k_max_final");
    }
    // k_max_final wrote the maxima into pinned host memory too (the host
    // checks them and keeps the exponents for the split pass), then the
    // tree's number; the quantize pass, which takes its scales from the
    // device, already runs while the host waits for that number.
    {
        ProfScope ps(c, HGB_KERNEL_QUANTIZE);
        k_quantize<Src><<<grid_for((c->n + 3) / 4, 256, 8192), 256, 0, c->stream>>>(
            src, c->n, vec, (const double*)(c->dev_words + 4), c->dev_words + 3, c->q);
        HGB_LAUNCHED(c, "k_quantize");
    }
    c->tree_precision = c->precision;
    if (c->async_begin) {
        c->scales_pending = true;
        c->have_tree = true;
        return HGB_OK;
    }
    hgb_status wst = wait_word(c, c->host_words + kHostTreeSeq, c->tree_seq);
    if (wst != HGB_OK) return wst;
    if (const char* bad = read_scales(c)) return fail(c, HGB_E_NONFINITE, "%s", bad);
    c->have_tree = true;
    return HGB_OK;
}

static bool aligned16(const void* p) { return p == nullptr || (uintptr_t)p % 16 == 0; }

static_assert(HGB_OBJ_SQUARED == kObjSquared && HGB_OBJ_LOGISTIC == kObjLogistic &&
                  HGB_OBJ_POISSON == kObjPoisson,
              "objective codes");

template <int OBJ>
static hgb_status begin_tree_objective_as(hgb_ctx* c, const float* m, const float* y, const float* w, int vec)
{
    if (w) return begin_tree_from(c, ObjectiveSource<OBJ, true>{m, y, w}, vec);
    return begin_tree_from(c, ObjectiveSource<OBJ, false>{m, y, nullptr}, vec);
}

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
    if (const char* e = std::getenv("HGB_PLAN_HOST")) c->plan_host = e[0] != '0';
    if (const char* e = std::getenv("HGB_FILL_TUNE")) {
        static const char* keys[kTuneKeys] = {"root_lc", "root_tile", "root_ipc", "level_lc", "level_tile",
                                              "level_ipc", "align", "piece", "il", "root_il", "pair"};
        std::string spec(e);
        size_t pos = 0;
        while (pos < spec.size()) {
            size_t end = spec.find(',', pos);
            if (end == std::string::npos) end = spec.size();
            const std::string kv = spec.substr(pos, end - pos);
            const size_t eq = kv.find('=');
            if (eq != std::string::npos)
                for (int k = 0; k < kTuneKeys; ++k)
                    if (kv.compare(0, eq, keys[k]) == 0) c->tune[k] = std::atoi(kv.c_str() + eq + 1);
            pos = end + 1;
        }
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) == hipSuccess && prop.multiProcessorCount > 0)
        c->n_cu = prop.multiProcessorCount;
    c->stream = (hipStream_t)hip_stream;
    {
        // the no-allocation scratch: its address on this device, looked up
        // once per device with the device current
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (g_scratch_dev.size() < (size_t)n) g_scratch_dev.resize((size_t)n, nullptr);
        if (!g_scratch_dev[device]) {
            void* ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
                delete c;
                return HGB_E_DEVICE;
            }
            g_scratch_dev[device] = ptr;
        }
        c->noalloc_scratch = (unsigned char*)g_scratch_dev[device];
    }
    // The words kernels post for the host (maxima, error word, sequence
    // numbers) are in coherent pinned memory, as are the partition's node
    // records: a kernel's stores there reach the host in the order its fences
    // give them.  In default (non-coherent) pinned memory they pass through
    // the GPU's write-back L2, and a sequence number could reach the host
    // before the results it vouches for.
    if (hipMalloc((void**)&c->dev_words, 64) != hipSuccess ||
        hipMalloc((void**)&c->max_part, sizeof(uint32_t) * 2 * kMaxBlocks) != hipSuccess ||
        hipHostMalloc((void**)&c->host_words, 64, hipHostMallocCoherent) != hipSuccess ||
        hipMemset(c->dev_words, 0, 64) != hipSuccess) {
        hgb_destroy(c);
        return HGB_E_DEVICE;
    }
    std::memset(c->host_words, 0, 64);   // no sequence number posted yet
    // The launch-plan stages at their initial size, now: a pinned allocation
    // takes a few hundred microseconds, and made on first use it stalled the
    // first trees of a fit (131,072 x 16,384 uses four stages a tree, so its
    // fifth tree still allocated some).
    for (Stage& st : c->stage) {
        if (hipHostMalloc(&st.host, kStageMinBytes, hipHostMallocCoherent) != hipSuccess ||
            hipMalloc(&st.dev, kStageMinBytes) != hipSuccess) {
            hgb_destroy(c);
            return HGB_E_DEVICE;
        }
        st.cap = kStageMinBytes;
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
        if (s.host) (void)hipHostFree(s.host);
        if (s.dev) (void)hipFree(s.dev);
    }
    for (hipEvent_t e : c->epoch_ev)
        if (e) (void)hipEventDestroy(e);
    for (auto& v : c->ev_pending)
        for (auto& pr : v) {
            (void)hipEventDestroy(pr.first);
            (void)hipEventDestroy(pr.second);
        }
    for (hipEvent_t e : c->ev_pool) (void)hipEventDestroy(e);
    if (c->host_ready) (void)hipEventDestroy(c->host_ready);
    (void)hipFree(c->bins);
    (void)hipFree(c->bins_rm);
    (void)hipFree(c->q);
    (void)hipFree(c->gh);
    (void)hipFree(c->partial);
    (void)hipFree(c->part);
    (void)hipFree(c->part_flags);
    if (c->part_host) (void)hipHostFree(c->part_host);
    (void)hipFree(c->best);
    (void)hipFree(c->totals);
    (void)hipFree(c->level_terms);
    (void)hipFree(c->level_best);
    (void)hipFree(c->dev_words);
    (void)hipFree(c->max_part);
    (void)hipFree(c->rot);
    (void)hipHostFree(c->host_words);
    delete c;
}

const char* hgb_last_error(const hgb_ctx* c)
{
    return c ? c->err.c_str() : "null context";
}

// After a stream sync that followed a copy of the device error word into
// host_words[2]: report (and clear) what the kernels flagged.
static hgb_status take_flags(hgb_ctx* c)
{
    const uint32_t flags = c->host_words[2];
    if (flags) {
        k_clear_u32<<<1, 64, 0, c->stream>>>(c->dev_words + 2, 1);
        HGB_LAUNCHED(c, "k_clear_u32");
        HGB_HIP(c, hipStreamSynchronize(c->stream));
        if (flags & kErrRowIndex)
            return fail(c, HGB_E_INVALID, "a row index outside [0, n_rows) was skipped");
    }
    return HGB_OK;
}

hgb_status hgb_sync(hgb_ctx* c)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    HGB_HIP(c, hipSetDevice(c->device));
    k_post_u32<<<1, 64, 0, c->stream>>>(c->dev_words + 2, c->host_words + 2);
    HGB_LAUNCHED(c, "k_post_u32");
    hgb_status st = wait_here(c, &c->host_ready);
    if (st != HGB_OK) return st;
    st = resolve_scales(c);
    if (st != HGB_OK) return st;
    st = take_flags(c);
    if (c->deferred != HGB_OK) {   // reported once, before a skipped row index
        const hgb_status d = c->deferred;
        c->deferred = HGB_OK;
        return fail(c, d, "%s", c->deferred_msg.c_str());
    }
    return st;
}

hgb_status hgb_set_async_begin(hgb_ctx* c, int enable)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    c->async_begin = enable != 0;
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
    {   // the current tree's maxima first: this call reuses their host words
        const hgb_status rst = resolve_scales(c);
        if (rst != HGB_OK) return rst;
    }
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
    // Each feature's most frequent slot.  When some feature's holds at least
    // 1/kHotSlotShare of the rows (a skewed feature, or a sparse column's
    // missing slot), the copy is rotated per feature so that it reads as 0 and
    // the fills skip it (recovering its cell by subtraction); otherwise the
    // copy stays as given and the fills add every slot.
    {
        if (c->rot) HGB_HIP(c, hipFree(c->rot));
        c->rot = nullptr;
        c->skip = false;
        HGB_HIP(c, hipMalloc((void**)&c->rot, sizeof(int32_t) * (size_t)n_features));
        uint32_t* counts = nullptr;
        const size_t n_counts = (size_t)n_features * S + n_features;   // counts, then each top count
        HGB_HIP(c, hipMalloc((void**)&counts, sizeof(uint32_t) * n_counts));
        HGB_HIP(c, hipMemsetAsync(counts, 0, sizeof(uint32_t) * n_counts, c->stream));
        const dim3 cgrid((unsigned)((n_rows + kCountChunk - 1) / kCountChunk), (unsigned)n_features);
        const size_t clds = sizeof(uint32_t) * (size_t)S * kCountCopies;
        hgb_status st = bin_bytes == 1 ? set_lds(c, k_slot_counts<uint8_t>, clds)
                                       : set_lds(c, k_slot_counts<uint16_t>, clds);
        if (st != HGB_OK) {
            (void)hipFree(counts);
            return st;
        }
        if (bin_bytes == 1)
            k_slot_counts<uint8_t><<<cgrid, 1024, clds, c->stream>>>((const uint8_t*)c->bins, n_rows, S, counts);
        else
            k_slot_counts<uint16_t><<<cgrid, 1024, clds, c->stream>>>((const uint16_t*)c->bins, n_rows, S, counts);
        HGB_LAUNCHED(c, "k_slot_counts");
        uint32_t* top = counts + (size_t)n_features * S;
        k_hot_slot<<<(unsigned)n_features, 256, 0, c->stream>>>(counts, S, c->rot, top);
        HGB_LAUNCHED(c, "k_hot_slot");
        std::vector<uint32_t> top_host(n_features);
        HGB_HIP(c, hipMemcpyAsync(top_host.data(), top, sizeof(uint32_t) * n_features, hipMemcpyDeviceToHost,
                                  c->stream));
        HGB_HIP(c, hipStreamSynchronize(c->stream));
        HGB_HIP(c, hipFree(counts));
        const uint32_t top_max = *std::max_element(top_host.begin(), top_host.end());
        c->skip = (int64_t)top_max * kHotSlotShare >= (int64_t)n_rows;
        if (c->skip) {
            const dim3 rgrid((unsigned)grid_for(n_rows, 256, 64), (unsigned)n_features);
            if (bin_bytes == 1)
                k_rotate<uint8_t><<<rgrid, 256, 0, c->stream>>>((uint8_t*)c->bins, n_rows, S, c->rot);
            else
                k_rotate<uint16_t><<<rgrid, 256, 0, c->stream>>>((uint16_t*)c->bins, n_rows, S, c->rot);
            HGB_LAUNCHED(c, "k_rotate");
        } else {
            HGB_HIP(c, hipMemsetAsync(c->rot, 0, sizeof(int32_t) * (size_t)n_features, c->stream));
        }
    }
    if ((int64_t)n_features * bin_bytes <= kRowMajorMaxRowBytes) {
        int64_t stride = ((int64_t)n_features * bin_bytes + 15) / 16 * 16;
        if (stride % kRowMajorSkewPeriod == 0) stride += kRowMajorSkew;
        // kRowMajorSlack bytes after the last row: a tile's load may run past
        // the end of a row, into the next row or this slack
        HGB_HIP(c, hipMalloc(&c->bins_rm, (size_t)(stride * n_rows + kRowMajorSlack)));
        HGB_HIP(c, hipMemsetAsync(c->bins_rm, 0, (size_t)(stride * n_rows + kRowMajorSlack), c->stream));
        c->rm_stride = stride;
        dim3 tgrid((unsigned)std::min<int64_t>(((int64_t)n_rows + 63) / 64, kTransposeMaxBlocks),
                   (unsigned)((n_features + 63) / 64));
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
    const int vec = aligned16(grad) && aligned16(hess);
    return begin_tree_from(c, GradSource{grad, hess}, vec);
}

hgb_status hgb_begin_tree_objective(hgb_ctx* c, int32_t objective, const float* margin,
                                    const float* label, const float* weight)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_data) return fail(c, HGB_E_STATE, "begin_tree_objective before upload_bins");
    if (!margin || !label) return fail(c, HGB_E_INVALID, "begin_tree_objective: null score or label pointer");
    const int vec = aligned16(margin) && aligned16(label) && aligned16(weight);
    switch (objective) {
    case HGB_OBJ_SQUARED: return begin_tree_objective_as<kObjSquared>(c, margin, label, weight, vec);
    case HGB_OBJ_LOGISTIC: return begin_tree_objective_as<kObjLogistic>(c, margin, label, weight, vec);
    case HGB_OBJ_POISSON: return begin_tree_objective_as<kObjPoisson>(c, margin, label, weight, vec);
    default: return fail(c, HGB_E_INVALID, "begin_tree_objective: unknown objective");
    }
}

hgb_status hgb_copy_quantized(hgb_ctx* c, int32_t* q_dev)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!q_dev) return fail(c, HGB_E_INVALID, "copy_quantized: null output");
    if (!c->have_tree) return fail(c, HGB_E_STATE, "copy_quantized before begin_tree");
    HGB_HIP(c, hipSetDevice(c->device));
    HGB_HIP(c, hipMemcpyAsync(q_dev, c->q, (size_t)c->n * sizeof(int2), hipMemcpyDeviceToDevice, c->stream));
    return HGB_OK;
}

hgb_status hgb_set_precision(hgb_ctx* c, int32_t bits)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (bits < 1 || bits > 30)
        return fail(c, HGB_E_INVALID, "set_precision: bits must be in [1, 30]");
    const hgb_status rst = resolve_scales(c);
    if (rst != HGB_OK) return rst;
    c->precision = bits;
    c->have_tree = false;
    return HGB_OK;
}

hgb_status hgb_get_scales(const hgb_ctx* cc, int32_t* k_g, int32_t* k_h)
{
    if (!cc || !k_g || !k_h) return HGB_E_INVALID;
    // reading the scales of an asynchronously started tree waits for them
    // (the context is logically unchanged)
    hgb_ctx* c = const_cast<hgb_ctx*>(cc);
    if (!c->have_tree) return HGB_E_STATE;
    const hgb_status st = resolve_scales(c);
    if (st != HGB_OK) return st;
    if (c->deferred != HGB_OK) return c->deferred;   // still reported by the next hgb_sync
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
        if (slots[i] < -1) return fail(c, HGB_E_INVALID, "build_level: output slot below -1");
        if (slots[i] == -1 && root) return fail(c, HGB_E_INVALID, "build_level: the root cannot be skipped");
        if (slots[i] == -1) count[i] = 0;   // skipped: none of its rows are read
    }
    {
        std::vector<int32_t> sorted;
        for (int32_t v : slots)
            if (v >= 0) sorted.push_back(v);
        std::sort(sorted.begin(), sorted.end());
        if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
            return fail(c, HGB_E_INVALID, "build_level: two nodes share an output slot");
    }
    HGB_HIP(c, hipSetDevice(c->device));
    const int64_t total = root ? c->n : (int64_t)node_offsets[n_nodes];
    // The root reads rows in order; other levels read through the row index,
    // from the row-major copy when there is one.
    const bool rm = !root && c->bins_rm != nullptr;
    const PlanCtx pc = plan_ctx(c);
    FillPlan plan = plan_fill(&pc, root, rm);
    const std::vector<std::pair<int, int>> tiles = feature_tiles(&pc, plan, root);
    for (const auto& t : tiles)
        if (t.second < 1 || (root && t.second > (plan.il ? plan.tile : 8)) || t.first + t.second > c->F)
            return fail(c, HGB_E_DEVICE, "build_level: internal error in the tile plan");

    if (!root) return fill_level(c, plan, tiles, row_index, begin, count, slots, total, hist);

    RootCut rc;
    cut_root(&pc, plan, tiles, total, slots[0], &rc);
    std::vector<FillItem>* groups = rc.groups;
    const std::vector<MergeEntry>& merges = rc.merges;
    const bool zero_root = rc.zero_root;
    if (rc.use_partial) {
        hgb_status gst = grow(c, &c->partial, &c->partial_cap, rc.n_chunks * (int64_t)c->F * c->S * 2);
        if (gst != HGB_OK) return gst;
    }
    if (c->debug_plan)
        std::fprintf(stderr,
                     "[hgb] fill kind %d acc %d copies %d tile %d lt %d ra %d il %d drain %d chunk %lld items %zu "
                     "lds %zu\n",
                     (int)plan.kind, plan.acc, 1 << plan.lc, plan.tile, plan.lt, plan.ra, plan.il, plan.drain,
                     (long long)rc.chunk, rc.n_items, plan.lds_bytes);
    // one upload: the root's slot (to zero before atomic merges), each
    // width's items, then the merges (each part 256-byte aligned)
    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    size_t offs[9] = {};
    size_t bytes = 256;
    for (int wdt = 8; wdt >= 0; --wdt) {
        offs[wdt] = bytes;
        bytes += up(groups[wdt].size() * sizeof(FillItem));
    }
    const size_t off_merges = bytes;
    bytes += merges.size() * sizeof(MergeEntry);
    std::vector<uint8_t> blob(bytes, 0);
    std::memcpy(blob.data(), &slots[0], sizeof(int32_t));
    for (int wdt = 8; wdt >= 0; --wdt)
        if (!groups[wdt].empty())
            std::memcpy(blob.data() + offs[wdt], groups[wdt].data(), groups[wdt].size() * sizeof(FillItem));
    if (!merges.empty())
        std::memcpy(blob.data() + off_merges, merges.data(), merges.size() * sizeof(MergeEntry));
    StageLease sg(c);
    hgb_status st = stage_upload(c, blob.data(), bytes, &sg.s);
    if (st != HGB_OK) return st;
    const uint8_t* dev = (const uint8_t*)sg.s->use;
    if (zero_root) {
        st = launch_zero(c, hist, (const int32_t*)dev, 1);
        if (st != HGB_OK) return st;
    }
    for (int wdt = 8; wdt >= 0; --wdt) {
        std::vector<FillItem>& items = groups[wdt];
        if (items.empty()) continue;
        FillPlan gp = plan;
        if (wdt > 0) {
            gp.tile = wdt;
            gp.lds_bytes = (size_t)(wdt * feature_lds(plan.acc, c->S, plan.lc) + 8 * kFixWords);
        }
        FillArgs a{};
        a.gh = c->q;
        a.items = (const FillItem*)(dev + offs[wdt]);
        a.n_items = (int)items.size();
        // whole-group vector loads need every column aligned to a group of
        // kRootRows rows (chunk starts are multiples of 128)
        a.vec_ok = (c->n % kRootRows == 0) ? 1 : 0;
        a.drain = std::max(plan.drain, 1);
        a.hist = hist;
        a.partial = (int64_t*)c->partial;
        ProfScope pr(c, HGB_KERNEL_FILL_ROOT);
        st = launch_fill(c, gp, a);
        if (st != HGB_OK) return st;
    }
    if (!merges.empty()) {
        ProfScope pm(c, HGB_KERNEL_MERGE);
        const int64_t node_vec = (int64_t)c->F * c->S;
        dim3 grid(grid_for(node_vec, 256, 1024), (unsigned)merges.size());
        st = launch_merge(c, merges, (const MergeEntry*)(dev + off_merges), grid, hist);
        if (st != HGB_OK) return st;
    }
    return sg.release();
}

hgb_status hgb_subtract_siblings(hgb_ctx* c, const int64_t* parent, int64_t* child,
                                 const uint8_t* built_is_right, int32_t n_pairs)
{
    return hgb_subtract_siblings_slots(c, parent, child, built_is_right, nullptr, n_pairs);
}

hgb_status hgb_subtract_siblings_slots(hgb_ctx* c, const int64_t* parent, int64_t* child,
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
    const int64_t pair_vec = (int64_t)c->F * c->S;   // longlong2 per slot
    dim3 grid(grid_for(pair_vec, 256, 2048), (unsigned)n_pairs);
    SubtractInline inl{};
    StageLease s(c);
    const int32_t* plan_dev = nullptr;
    if (n_pairs <= kSubtractInlinePairs) {
        std::memcpy(inl.v, plan.data(), plan.size() * sizeof(int32_t));
    } else {
        hgb_status st = stage_upload(c, plan.data(), plan.size() * sizeof(int32_t), &s.s);
        if (st != HGB_OK) return st;
        plan_dev = (const int32_t*)s.s->use;
    }
    {
        ProfScope ps(c, HGB_KERNEL_SUBTRACT);
        k_subtract<<<grid, 256, 0, c->stream>>>((const longlong2*)parent, (longlong2*)child, plan_dev,
                                                inl, pair_vec);
    }
    HGB_LAUNCHED(c, "k_subtract");
    return s.release();
}

// Checks of find_splits' arguments (both entry points).
static hgb_status check_find_splits(hgb_ctx* c, const int64_t* hist, int32_t n_nodes, double lambda,
                                    double gamma, const hgb_split* out, const char* who)
{
    if (!c->have_tree) return fail(c, HGB_E_STATE, "%s before begin_tree", who);
    if (n_nodes < 0 || n_nodes > 65535) return fail(c, HGB_E_INVALID, "%s: n_nodes out of range", who);
    if (!(lambda >= 0.0) || !std::isfinite(lambda) || !std::isfinite(gamma))
        return fail(c, HGB_E_INVALID, "%s: lambda must be finite and >= 0, gamma finite", who);
    if (n_nodes > 0 && (!hist || !out)) return fail(c, HGB_E_INVALID, "%s: null pointer", who);
    return HGB_OK;
}

// The split scan's shape: per node, n_entries per-block winners (one per block
// of 4 features, or per feature for wide bins), and how the lanes hold bins.
struct SplitShape {
    int per;        // bins per lane
    bool aligned;   // the histogram is 16-byte aligned
    bool sliced;    // wide bins: one block of kSliceWaves waves per feature
    int n_entries;
};

static SplitShape split_shape(const hgb_ctx* c, const int64_t* hist)
{
    SplitShape sh;
    // a lane's bins in registers when there are at most 4 of them (one wave
    // per feature) or at most 4 x 4 per wave of a sliced block (wide bins),
    // the buffer 16-byte aligned; otherwise read twice from memory
    sh.per = (c->B + kWave - 1) / kWave;
    sh.aligned = ((uintptr_t)hist & 15) == 0;
    sh.sliced = sh.aligned && sh.per > 4 && sh.per <= 4 * kSliceWaves;
    sh.n_entries = sh.sliced ? c->F : (c->F + 3) / 4;
    return sh;
}

// The per-feature scan into best/totals (device scratch of the shape's size),
// then the per-node reduction into out.
static hgb_status launch_find_splits(hgb_ctx* c, const SplitShape& sh, const int64_t* hist, int32_t n_nodes,
                                     double lambda, double gamma, hgb_split* out, FeatureBest* best,
                                     long long* totals)
{
    static_assert(sizeof(SplitOut) == sizeof(hgb_split), "split record layout");
    const int waves = 4;   // features per block; one best per block
    dim3 grid((unsigned)sh.n_entries, (unsigned)n_nodes);
#define HGB_SPLIT(PER)                                                                              \
    k_split_feature<PER><<<grid, waves * kWave, 0, c->stream>>>(                                    \
        (const long long*)hist, c->F, c->B, c->S, c->has_missing, inv_scales(c), lambda, gamma, best, \
        totals)
#define HGB_SPLIT_SLICED(PER)                                                                       \
    k_split_feature_sliced<PER><<<grid, kSliceWaves * kWave, 0, c->stream>>>(                       \
        (const long long*)hist, c->F, c->B, c->S, c->has_missing, inv_scales(c), lambda, gamma, best, \
        totals)
    const int per = sh.per;
    if (sh.sliced) {
        if (per <= 2 * kSliceWaves) HGB_SPLIT_SLICED(2);
        else HGB_SPLIT_SLICED(4);
    } else if (!sh.aligned || per > 16) HGB_SPLIT(0);
    else if (per <= 1) HGB_SPLIT(1);
    else if (per <= 2) HGB_SPLIT(2);
    else if (per <= 4) HGB_SPLIT(4);
    else if (per <= 8) HGB_SPLIT(8);
    else HGB_SPLIT(16);
#undef HGB_SPLIT
#undef HGB_SPLIT_SLICED
    HGB_LAUNCHED(c, "k_split_feature");
    k_split_reduce<<<(unsigned)n_nodes, split_reduce_threads(sh.n_entries), 0, c->stream>>>(
        best, totals, sh.n_entries, (SplitOut*)out);
    HGB_LAUNCHED(c, "k_split_reduce");
    return HGB_OK;
}

hgb_status hgb_find_splits(hgb_ctx* c, const int64_t* hist, int32_t n_nodes, double lambda,
                           double gamma, hgb_split* out)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    hgb_status st = check_find_splits(c, hist, n_nodes, lambda, gamma, out, "find_splits");
    if (st != HGB_OK || n_nodes == 0) return st;
    HGB_HIP(c, hipSetDevice(c->device));
    const SplitShape sh = split_shape(c, hist);
    st = grow(c, &c->best, &c->best_cap, (int64_t)n_nodes * sh.n_entries);
    if (st != HGB_OK) return st;
    st = grow(c, &c->totals, &c->totals_cap, (int64_t)2 * n_nodes);
    if (st != HGB_OK) return st;
    ProfScope ps(c, HGB_KERNEL_SPLIT);
    return launch_find_splits(c, sh, hist, n_nodes, lambda, gamma, out, c->best, c->totals);
}

// Bytes of the no-allocation scratch a find_splits of n_nodes would use: the
// per-block winners (256-byte aligned), then the node totals.
static size_t noalloc_split_bytes(const SplitShape& sh, int32_t n_nodes, size_t* totals_off)
{
    const size_t best = (size_t)n_nodes * (size_t)sh.n_entries * sizeof(FeatureBest);
    *totals_off = (best + 255) / 256 * 256;
    return *totals_off + (size_t)2 * n_nodes * sizeof(long long);
}

hgb_status hgb_find_splits_noalloc(hgb_ctx* c, const int64_t* hist, int32_t n_nodes, double lambda,
                                   double gamma, hgb_split* out)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    hgb_status st = check_find_splits(c, hist, n_nodes, lambda, gamma, out, "find_splits_noalloc");
    if (st != HGB_OK || n_nodes == 0) return st;
    if (!c->noalloc_scratch) return fail(c, HGB_E_DEVICE, "find_splits_noalloc: no scratch on this device");
    const SplitShape sh = split_shape(c, hist);
    size_t totals_off = 0;
    const size_t need = noalloc_split_bytes(sh, n_nodes, &totals_off);
    if (need > kNoAllocScratchBytes)
        return fail(c, HGB_E_UNSUPPORTED,
                    "find_splits_noalloc: %d nodes x %d features need %zu bytes of scratch, more than its %zu",
                    n_nodes, c->F, need, kNoAllocScratchBytes);
    HGB_HIP(c, hipSetDevice(c->device));
    // Every entry the reduction reads is written by the scan first, so the
    // scratch needs no clearing (it keeps the last call's contents).
    return launch_find_splits(c, sh, hist, n_nodes, lambda, gamma, out, (FeatureBest*)c->noalloc_scratch,
                              (long long*)(c->noalloc_scratch + totals_off));
}

hgb_status hgb_find_level_split(hgb_ctx* c, const int64_t* hist, int32_t n_nodes, double lambda,
                                double gamma, hgb_split* out)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_tree) return fail(c, HGB_E_STATE, "find_level_split before begin_tree");
    if (n_nodes < 0 || n_nodes > 65535)
        return fail(c, HGB_E_INVALID, "find_level_split: n_nodes out of range");
    if (!(lambda >= 0.0) || !std::isfinite(lambda) || !std::isfinite(gamma))
        return fail(c, HGB_E_INVALID, "find_level_split: lambda must be finite and >= 0, gamma finite");
    if (!out || (n_nodes > 0 && !hist)) return fail(c, HGB_E_INVALID, "find_level_split: null pointer");
    HGB_HIP(c, hipSetDevice(c->device));
    const int n_dirs = c->has_missing ? 2 : 1;
    const int64_t n_cand = (int64_t)c->F * c->B * n_dirs;
    const int64_t n_blocks = n_nodes > 0 ? (n_cand + 255) / 256 : 0;
    hgb_status st = grow(c, &c->level_terms, &c->level_terms_cap, std::max<int64_t>(1, n_cand * n_nodes));
    if (st != HGB_OK) return st;
    st = grow(c, &c->level_best, &c->level_best_cap, std::max<int64_t>(1, n_blocks));
    if (st != HGB_OK) return st;
    ProfScope ps(c, HGB_KERNEL_SPLIT);
    if (n_nodes > 0) {
        const int waves = 4;
        dim3 grid((c->F + waves - 1) / waves, (unsigned)n_nodes);
        const int per = (c->B + kWave - 1) / kWave;
        const bool aligned = ((uintptr_t)hist & 15) == 0;
#define HGB_LEVEL(PER)                                                                              \
    k_level_gain<PER><<<grid, waves * kWave, 0, c->stream>>>(                                       \
        (const long long*)hist, c->F, c->B, c->S, c->has_missing, inv_scales(c), lambda, gamma,      \
        c->level_terms)
        if (!aligned || per > 16) HGB_LEVEL(0);
        else if (per <= 1) HGB_LEVEL(1);
        else if (per <= 2) HGB_LEVEL(2);
        else if (per <= 4) HGB_LEVEL(4);
        else if (per <= 8) HGB_LEVEL(8);
        else HGB_LEVEL(16);
#undef HGB_LEVEL
        HGB_LAUNCHED(c, "k_level_gain");
        k_level_sum<<<(unsigned)n_blocks, 256, 0, c->stream>>>(c->level_terms, n_nodes, n_cand, c->level_best);
        HGB_LAUNCHED(c, "k_level_sum");
    }
    k_level_pick<<<1, 256, 0, c->stream>>>(c->level_best, (int)n_blocks, c->B, n_dirs, (SplitOut*)out + n_nodes);
    HGB_LAUNCHED(c, "k_level_pick");
    if (n_nodes > 0) {
        const unsigned rblocks = (unsigned)std::min<int64_t>((n_nodes + 3) / 4, 64);
        k_level_records<<<rblocks, 256, 0, c->stream>>>((const long long*)hist, c->level_terms, n_nodes, c->F,
                                                        c->B, c->S, c->has_missing, (SplitOut*)out);
        HGB_LAUNCHED(c, "k_level_records");
    }
    return HGB_OK;
}

hgb_status hgb_subtract_find_splits(hgb_ctx* c, const int64_t* parent, int64_t* child,
                                    const uint8_t* built_is_right, const int32_t* parent_slot,
                                    int32_t n_pairs, double lambda, double gamma, hgb_split* out)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_tree) return fail(c, HGB_E_STATE, "subtract_find_splits before begin_tree");
    if (n_pairs < 0 || n_pairs > 32767)
        return fail(c, HGB_E_INVALID, "subtract_find_splits: n_pairs out of range");
    if (!(lambda >= 0.0) || !std::isfinite(lambda) || !std::isfinite(gamma))
        return fail(c, HGB_E_INVALID, "subtract_find_splits: lambda must be finite and >= 0, gamma finite");
    if (n_pairs == 0) return HGB_OK;
    if (!parent || !child || !built_is_right || !out)
        return fail(c, HGB_E_INVALID, "subtract_find_splits: null pointer");
    const int per = (c->B + kWave - 1) / kWave;
    const bool aligned = ((uintptr_t)parent & 15) == 0 && ((uintptr_t)child & 15) == 0;
    if (!aligned || per > 16) {   // the two passes
        hgb_status st = hgb_subtract_siblings_slots(c, parent, child, built_is_right, parent_slot, n_pairs);
        if (st != HGB_OK) return st;
        return hgb_find_splits(c, child, 2 * n_pairs, lambda, gamma, out);
    }
    std::vector<int32_t> plan(2 * (size_t)n_pairs);
    for (int i = 0; i < n_pairs; ++i) {
        const int32_t ps = parent_slot ? parent_slot[i] : i;
        if (ps < 0) return fail(c, HGB_E_INVALID, "subtract_find_splits: negative parent slot");
        plan[2 * i] = ps;
        plan[2 * i + 1] = built_is_right[i] ? 1 : 0;
    }
    HGB_HIP(c, hipSetDevice(c->device));
    const int n_nodes = 2 * n_pairs;
    // one best per block of 4 features, or per feature for wide bins (a
    // sliced block of kSliceWaves waves per feature)
    const bool sliced = per > 4 && per <= 4 * kSliceWaves;
    const int n_entries = sliced ? c->F : (c->F + 3) / 4;
    hgb_status st = grow(c, &c->best, &c->best_cap, (int64_t)n_nodes * n_entries);
    if (st != HGB_OK) return st;
    st = grow(c, &c->totals, &c->totals_cap, (int64_t)2 * n_nodes);
    if (st != HGB_OK) return st;
    SubtractInline inl{};
    StageLease s(c);
    const int32_t* plan_dev = nullptr;
    if (n_pairs <= kSubtractInlinePairs) {
        std::memcpy(inl.v, plan.data(), plan.size() * sizeof(int32_t));
    } else {
        st = stage_upload(c, plan.data(), plan.size() * sizeof(int32_t), &s.s);
        if (st != HGB_OK) return st;
        plan_dev = (const int32_t*)s.s->use;
    }
    const int waves = 4;
    dim3 grid((unsigned)n_entries, (unsigned)n_pairs);
    const double* sc = inv_scales(c);
    {
        ProfScope ps(c, HGB_KERNEL_SPLIT);
#define HGB_SUBSPLIT(PER)                                                                          \
    k_subtract_split<PER><<<grid, waves * kWave, 0, c->stream>>>(                                  \
        (const long long*)parent, (long long*)child, plan_dev, inl, c->F, c->B, c->S, c->has_missing, \
        sc, lambda, gamma, c->best, c->totals)
#define HGB_SUBSPLIT_SLICED(PER)                                                                   \
    k_subtract_split_sliced<PER><<<grid, kSliceWaves * kWave, 0, c->stream>>>(                     \
        (const long long*)parent, (long long*)child, plan_dev, inl, c->F, c->B, c->S, c->has_missing, \
        sc, lambda, gamma, c->best, c->totals)
        if (sliced) {
            if (per <= 2 * kSliceWaves) HGB_SUBSPLIT_SLICED(2);
            else HGB_SUBSPLIT_SLICED(4);
        } else if (per <= 1) HGB_SUBSPLIT(1);
        else if (per <= 2) HGB_SUBSPLIT(2);
        else if (per <= 4) HGB_SUBSPLIT(4);
        else if (per <= 8) HGB_SUBSPLIT(8);
        else HGB_SUBSPLIT(16);
#undef HGB_SUBSPLIT
#undef HGB_SUBSPLIT_SLICED
        HGB_LAUNCHED(c, "k_subtract_split");
        k_split_reduce<<<(unsigned)n_nodes, split_reduce_threads(n_entries), 0, c->stream>>>(c->best, c->totals, n_entries, (SplitOut*)out);
        HGB_LAUNCHED(c, "k_split_reduce");
    }
    return s.release();
}

// The partition; nt: read the split features' bins with non-temporal loads
// (depthwise levels, whose nodes split on many features).
static hgb_status partition_impl(hgb_ctx* c, const int32_t* row_index, const int32_t* node_offsets,
                                 int32_t n_nodes, const hgb_split* splits, int32_t* out_rows,
                                 int32_t* child_offsets, int32_t* n_children, int32_t* parent_node, bool nt)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!c->have_data) return fail(c, HGB_E_STATE, "partition_level before upload_bins");
    if (!splits || !child_offsets || !n_children)
        return fail(c, HGB_E_INVALID, "partition_level: null pointer");
    if (n_nodes < 1 || n_nodes > 65535)
        return fail(c, HGB_E_INVALID, "partition_level: n_nodes must be in [1, 65535]");
    const bool root = !row_index && !node_offsets;
    if (row_index && !node_offsets)
        return fail(c, HGB_E_INVALID, "partition_level: node_offsets required with row_index");
    if (root && n_nodes != 1)
        return fail(c, HGB_E_INVALID, "partition_level: the root (no row index) is one node");
    std::vector<int32_t> offs(n_nodes + 1);
    if (root) {
        offs[0] = 0;
        offs[1] = (int32_t)c->n;
    } else {
        if (node_offsets[0] != 0) return fail(c, HGB_E_INVALID, "partition_level: offsets must start at 0");
        for (int i = 0; i <= n_nodes; ++i) {
            offs[i] = node_offsets[i];
            if (i > 0 && offs[i] < offs[i - 1])
                return fail(c, HGB_E_INVALID, "partition_level: offsets decrease at node %d", i - 1);
        }
        if (!row_index && offs[n_nodes] != 0)
            return fail(c, HGB_E_INVALID, "partition_level: row_index is NULL but the nodes hold rows");
    }
    if (offs[n_nodes] > 0 && !out_rows) return fail(c, HGB_E_INVALID, "partition_level: null output");
    HGB_HIP(c, hipSetDevice(c->device));

    // chunks of each node's rows, in node order
    std::vector<PartItem> items;
    std::vector<int32_t> first;
    part_chunks(offs, n_nodes, &items, &first);
    const int64_t n_items = (int64_t)items.size();

    auto up = [](size_t b) { return (b + 255) / 256 * 256; };
    const size_t off_first = up(items.size() * sizeof(PartItem));
    const size_t off_offs = off_first + up(first.size() * sizeof(int32_t));
    const size_t bytes = off_offs + offs.size() * sizeof(int32_t);
    std::vector<uint8_t> blob(bytes, 0);
    if (!items.empty()) std::memcpy(blob.data(), items.data(), items.size() * sizeof(PartItem));
    std::memcpy(blob.data() + off_first, first.data(), first.size() * sizeof(int32_t));
    std::memcpy(blob.data() + off_offs, offs.data(), offs.size() * sizeof(int32_t));

    hgb_status st = grow(c, &c->part, &c->part_cap, 2 * n_items + 3 * (int64_t)n_nodes + 1);
    if (st != HGB_OK) return st;
    if (c->part_host_cap < 3 * (int64_t)n_nodes) {
        if (c->part_host) HGB_HIP(c, hipHostFree(c->part_host));
        c->part_host = nullptr;
        c->part_host_cap = 0;
        HGB_HIP(c, hipHostMalloc((void**)&c->part_host, sizeof(int32_t) * 3 * (size_t)n_nodes,
                                 hipHostMallocCoherent));   // (see host_words)
        c->part_host_cap = 3 * (int64_t)n_nodes;
    }
    st = grow(c, &c->part_flags, &c->part_flags_cap, std::max<int64_t>(offs[n_nodes], 1));
    if (st != HGB_OK) return st;
    int32_t* cnt = c->part;
    int32_t* left_base = c->part + n_items;
    int32_t* node_out = c->part + 2 * n_items;

    StageLease sg(c);
    st = stage_upload(c, blob.data(), bytes, &sg.s);
    if (st != HGB_OK) return st;
    const uint8_t* dev = (const uint8_t*)sg.s->use;
    const PartItem* items_dev = (const PartItem*)dev;
    const SplitOut* sp = (const SplitOut*)splits;
    {
        ProfScope ps(c, HGB_KERNEL_PARTITION);
        if (n_items > 0) {
#define HGB_PART_COUNT(BinT, NT)                                                                      \
    k_part_count<BinT, NT><<<(unsigned)n_items, kPartThreads, 0, c->stream>>>(                        \
        (const BinT*)c->bins, c->n, c->B, c->S, c->rot, row_index, items_dev, sp, cnt, c->part_flags, \
        c->dev_words + 2)
            if (c->bin_bytes == 1) {
                if (nt) HGB_PART_COUNT(uint8_t, true);
                else HGB_PART_COUNT(uint8_t, false);
            } else {
                if (nt) HGB_PART_COUNT(uint16_t, true);
                else HGB_PART_COUNT(uint16_t, false);
            }
#undef HGB_PART_COUNT
            HGB_LAUNCHED(c, "k_part_count");
        }
        const uint32_t seq = ++c->part_seq;
        if (n_items <= kPartScanLdsItems && n_nodes <= kPartScanLdsNodes)
            k_part_scan_lds<kPartScanLdsItems, kPartScanLdsNodes><<<1, 1024, 0, c->stream>>>(
                cnt, (int)n_items, (const int32_t*)(dev + off_first), (const int32_t*)(dev + off_offs), sp, n_nodes,
                left_base, node_out, c->part_host, c->dev_words + 2, c->host_words + 2,
                c->host_words + kHostPartSeq, seq);
        else
            k_part_scan<<<1, 1024, 0, c->stream>>>(cnt, items_dev, (int)n_items, (const int32_t*)(dev + off_first),
                                                   (const int32_t*)(dev + off_offs), sp, n_nodes, left_base,
                                                   node_out, c->part_host, c->dev_words + 2, c->host_words + 2,
                                                   c->host_words + kHostPartSeq, seq);
        // node records, error word, then the level's number, into pinned host memory
        HGB_LAUNCHED(c, "k_part_scan");
        if (n_items > 0) {
            k_part_scatter<<<(unsigned)n_items, kPartThreads, 0, c->stream>>>(row_index, items_dev, sp, c->part_flags,
                                                                      left_base, node_out, out_rows);
            HGB_LAUNCHED(c, "k_part_scatter");
        }
    }
    st = sg.release();
    if (st != HGB_OK) return st;
    // Wait for the node records only: the scatter keeps running while the
    // caller plans the next level (the stream orders whatever reads its rows).
    st = wait_word(c, c->host_words + kHostPartSeq, c->part_seq);
    if (st != HGB_OK) return st;
    st = take_flags(c);   // a row index outside [0, n)
    if (st != HGB_OK) return st;
    int32_t nc = 0;
    child_offsets[0] = 0;
    for (int i = 0; i < n_nodes; ++i) {
        if (!c->part_host[3 * i + 2]) continue;
        const int32_t left = c->part_host[3 * i + 1];
        child_offsets[nc + 1] = child_offsets[nc] + left;
        child_offsets[nc + 2] = child_offsets[nc] + (offs[i + 1] - offs[i]);
        if (parent_node) parent_node[nc / 2] = i;
        nc += 2;
    }
    *n_children = nc;
    return HGB_OK;
}

hgb_status hgb_partition_level(hgb_ctx* c, const int32_t* row_index, const int32_t* node_offsets,
                               int32_t n_nodes, const hgb_split* splits, int32_t* out_rows,
                               int32_t* child_offsets, int32_t* n_children, int32_t* parent_node)
{
    return partition_impl(c, row_index, node_offsets, n_nodes, splits, out_rows, child_offsets, n_children,
                          parent_node, false);
}

hgb_status hgb_grow_level(hgb_ctx* c, const int64_t* parent_hist, const hgb_split* parent_splits,
                          const int32_t* parent_rows, const int32_t* parent_offsets, int32_t n_parents,
                          int32_t* child_rows, int64_t* child_hist, hgb_split* child_splits,
                          int32_t* child_offsets, int32_t* n_children, uint8_t* built_is_right,
                          int32_t* parent_node, int64_t* built_rows, double lambda, double gamma,
                          int32_t oblivious)
{
    if (!c) return HGB_E_INVALID;
    c->err.clear();
    if (!parent_hist || !child_hist || !child_splits || !child_offsets || !n_children || !built_is_right)
        return fail(c, HGB_E_INVALID, "grow_level: null pointer");
    if (n_parents < 1 || n_parents > 32767)
        return fail(c, HGB_E_INVALID, "grow_level: n_parents must be in [1, 32767]");
    std::vector<int32_t> parents((size_t)n_parents);
    hgb_status st = partition_impl(c, parent_rows, parent_offsets, n_parents, parent_splits, child_rows,
                                   child_offsets, n_children, parents.data(), !oblivious);
    if (st != HGB_OK) return st;
    const int32_t nc = *n_children;
    if (built_rows) *built_rows = 0;
    if (nc == 0) return HGB_OK;
    const int32_t n_pairs = nc / 2;
    // the smaller child of each pair is built (the left one on a tie); the
    // other's slot is -1, so its rows are not read
    std::vector<int32_t> slots((size_t)nc, -1);
    int64_t rows = 0;
    for (int32_t j = 0; j < n_pairs; ++j) {
        const int32_t nl = child_offsets[2 * j + 1] - child_offsets[2 * j];
        const int32_t nr = child_offsets[2 * j + 2] - child_offsets[2 * j + 1];
        const uint8_t right = nr < nl ? 1 : 0;
        built_is_right[j] = right;
        slots[2 * j + right] = 2 * j + right;
        rows += right ? nr : nl;
        if (parent_node) parent_node[j] = parents[j];
    }
    if (built_rows) *built_rows = rows;
    st = hgb_build_level(c, child_rows, child_offsets, nc, child_hist, slots.data());
    if (st != HGB_OK) return st;
    if (oblivious) {
        st = hgb_subtract_siblings_slots(c, parent_hist, child_hist, built_is_right, parents.data(), n_pairs);
        if (st != HGB_OK) return st;
        return hgb_find_level_split(c, child_hist, nc, lambda, gamma, child_splits);
    }
    return hgb_subtract_find_splits(c, parent_hist, child_hist, built_is_right, parents.data(), n_pairs, lambda,
                                    gamma, child_splits);
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
    if (kernel == HGB_KERNEL_FILL) {   // the sum of its three parts, each timed on its own
        *total_ms = c->prof_ms[HGB_KERNEL_FILL_ROOT] + c->prof_ms[HGB_KERNEL_FILL_LEVEL] +
                    c->prof_ms[HGB_KERNEL_MERGE];
        *launches = c->prof_launches[HGB_KERNEL_FILL_ROOT] + c->prof_launches[HGB_KERNEL_FILL_LEVEL] +
                    c->prof_launches[HGB_KERNEL_MERGE];
        return HGB_OK;
    }
    *total_ms = c->prof_ms[kernel];
    *launches = c->prof_launches[kernel];
    return HGB_OK;
}

}  // extern "C"
