// Host-side launch planning of the hgb library: fill plans (tile layout,
// copies, accumulation mode) from a cost model, the cut of a level's rows into
// per-block shares, the root's row chunks, and the partition's chunks.  Plain
// C++ over hgb_layout.h: it includes no HIP header, so it is compiled and
// tested on the host alone (tests/host/plan_test.cpp, also under the address
// and undefined-behaviour sanitizers).
#pragma once

#include <algorithm>
#include <cstdint>
#include <string>
#include <utility>
#include <vector>

#include "hgb_layout.h"

namespace hgb {

// gfx950: 160 KiB of LDS per CU; every fill runs one 1024-thread block per CU.
constexpr int64_t kFillLdsBudget = 160 * 1024;
// What a tile may take of it: the rest holds the item's totals and the
// features' recovered cells (kFixWords).
constexpr int64_t kTileLdsBudget = kFillLdsBudget - 8 * kFixWords;
constexpr int kRootThreads = 1024;
constexpr int kLevelThreads = 1024;
// Fill items per CU: the root gets one equal share per CU (equal items finish
// together, and fewer items mean fewer merges of partial histograms).
constexpr int64_t kRootItemsPerCu = 1;
// Level fills: blocks per CU, each taking an equal share of the level's rows.
constexpr int64_t kLevelBlocksPerCu = 1;
// Fixed cost of one fill item, in rows per cell of its tile: zeroing the tile,
// the pipeline's ramp and writing the tile out weigh about as much as this
// many rows.
constexpr double kPieceRowsPerCell = 0.25;
// A node split over more blocks than this is merged in several groups, added
// into its zeroed slot with atomics.
constexpr int kMergeGroup = 32;
// Most nodes a level may hold.
constexpr int kMaxLevelNodes = 65535;

// What the planner reads of a context: the resident matrix's shape, the
// precision, whether the skipped slot is on, the chip's CU count and the
// developer overrides (HGB_FILL_TUNE: root_lc, root_tile, root_ipc,
// level_lc, level_tile, level_ipc, align, piece, il, root_il, pair; -1 = the
// planner's choice).
constexpr int kTuneKeys = 11;
struct PlanCtx {
    int64_t n = 0;
    int F = 0, S = 0, bin_bytes = 1, precision = 30;
    bool skip = false;
    int64_t rm_stride = 0;   // bytes per row of the row-major copy (0: none)
    int n_cu = 256;
    int tune[kTuneKeys] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
};

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
    int ra;             // rows, packed: register-accumulator cells per thread (0: LDS)
    int il;             // slot-major interleaved tile (lane-rotated features)
    size_t lds_bytes;
};

// Row-major level fills with a register accumulator: cells per thread and
// entries per thread and step.
constexpr int kRegAccCells = 8;
constexpr int kRegAccEntries = 1;
// Entries per thread and step of the wide row-major fill.
constexpr int kWideRowEntries = 1;

// LDS bytes per feature of a tile: the copies, plus the packed accumulator.
inline int64_t feature_lds(int acc, int S, int lc)
{
    return (int64_t)tile_words(acc, 1, S, lc) * 8;
}

// Packed sums stay exact while every copy-slot sees at most
// kPackedRowsPerCopy rows between drains.  Copy c is used by threads / C
// threads, each taking `per_thread` rows per step; the root kernel may add up
// to kRootRows - 1 tail rows on one copy after its last step.  Returns the
// steps between drains (0: not even one step fits).
inline int packed_drain_steps(int threads, int lc, int per_thread)
{
    const int64_t per_copy_step = (int64_t)(threads >> lc) * per_thread;
    return (int)((kPackedRowsPerCopy - (kRootRows - 1)) / per_copy_step);
}

// Cost model of the root and feature-major fills per cell (seconds), fitted
// to measurements on the MI355X: random-bin ds_add_u64 runs at kLdsOps[lc]
// lanes per clock per CU with 2^lc lane-interleaved copies, bins stream from
// HBM at ~6 TB/s, and every feature tile of a row chunk re-reads and unpacks
// the (g, h) pair (~30 TB/s equivalent).  In these kernels the terms add up
// rather than overlap.
inline double fill_cost(int acc, int lc, int tile, int w)
{
    static const double kLdsOps[5] = {4.3, 4.75, 5.4, 6.9, 8.4};
    const double lds = (acc == kWide ? 2.0 : 1.0) / (kLdsOps[lc] * 2.4e9 * 256);
    return lds + w / 6.0e12 + (8.0 / tile) / 30.0e12;
}

// The same for the root's interleaved tile of tf positions (wide sums), over
// F features: the adds spread over tf * 2^lc bank pairs (32: conflict-free)
// but every position is added, used or not; one (g, h) read serves tf
// features; and the register rotation and per-lane feature offsets cost about
// two vector instructions per add more than the feature-major tile (64 lanes
// per clock per CU).
inline double fill_cost_il(int lc, int tf, int F, int w)
{
    const double clk = 2.4e9 * 256;
    const int spread = tf << lc;
    const double ops = spread >= 32 ? 9.0 : spread >= 16 ? 6.5 : spread >= 8 ? 5.0 : 4.3;
    const double waste = (double)((F + tf - 1) / tf * tf) / F;
    const double lds = 2.0 * waste / (ops * clk);
    const double valu = 2.0 * waste / (64.0 * clk);
    return lds + w / 6.0e12 + (8.0 / tf) / 30.0e12 + valu;
}

// The root's interleaved tile with packed sums: one add per position, plus
// the drains -- every `drain` steps of 4 rows per thread, each of the tile's
// S * tf * 2^lc words is exchanged with zero once (a conflict-free LDS
// atomic) and two barriers stall the block.
inline double fill_cost_il_packed(int lc, int tf, int F, int w, int S, int drain)
{
    const double clk = 2.4e9 * 256;
    const double waste = (double)((F + tf - 1) / tf * tf) / F;
    const double ops = 9.0;
    const double drain_per_cell = (double)S * (1 << lc) / ((double)drain * kRootThreads * kRootRows);
    const double lds = (waste + drain_per_cell) / (ops * clk);
    const double valu = 1.5 * waste / (64.0 * clk);
    return lds + w / 6.0e12 + (8.0 / tf) / 30.0e12 + valu;
}

// Lane pairs (il = 2): an interleaved tile over 32-byte chunks takes each row
// on two lanes, one 16-byte half each.  A lane alone loads its chunk in two
// instructions, and when rows lie far apart (a wide matrix) each of them is a
// request of its own to L2, which is what throttled that fill; a pair's halves
// leave one load instruction as one request.
//
// Row-major level fills read scattered rows.  Cost per row (seconds) of a plan
// with n_tiles feature tiles: the LDS adds at the same rates as above (plus
// the packed drains: lane-contiguous LDS reads and writes); each row's lines
// from HBM once at ~5 TB/s (the tiles of a share run side by side on one XCD
// and share them through L2); and per tile a 64-byte L2 transfer of the row's
// segment plus its index and (g, h), at ~10 TB/s (fitted to 10M x 28 and 131K x 16K level
// timings).
inline double rows_cost(int acc, int lc, int F, int n_tiles, int64_t row_bytes, double drain_ops_per_row,
                 int il = 0, int tile = 0)
{
    static const double kLdsOps[5] = {4.3, 4.75, 5.4, 6.9, 8.4};
    const double clk = 2.4e9 * 256;
    // The interleaved tile spreads a wave's adds over tile * 2^lc bank pairs
    // (32 is conflict-free, ~9.9 lanes per clock; measured with lds_rate) but
    // adds every one of the tile's positions, the unused ones included.
    const int spread = tile << lc;
    const double il_ops = spread >= 32 ? 9.0 : spread >= 16 ? 6.5 : spread >= 8 ? 5.0 : 4.3;
    const double adds = il ? (double)n_tiles * tile : (double)F;
    const double lds = adds * (acc == kWide ? 2.0 : 1.0) / ((il ? il_ops : kLdsOps[lc]) * clk) +
                       drain_ops_per_row / (16.0 * clk);
    // Vector ALU work per add, 64 lanes per clock per CU: about 3 instructions
    // (unpack, address), 6 with the interleaved tile's rotation and per-lane
    // feature offset, 5 when a lane pair shares the row (each lane rotates
    // half the chunk).  It decides narrow matrices, where the gather dominates
    // and the interleaved tile's faster adds buy little (a 28-feature matrix).
    const double valu = adds * (il == 2 ? 5.0 : il ? 6.0 : 3.0) / (64.0 * clk);
    const double lines = (double)std::max<int64_t>((row_bytes + 127) / 128, 1) * 128.0;
    const double mem = lines / 5.0e12 + n_tiles * (64.0 + 12.0) / 10.0e12;
    return std::max(lds, mem) + 0.25 * std::min(lds, mem) + valu;
}

// Threads of a k_split_reduce block: a node with many feature entries (a wide
// matrix) takes 1,024, so each thread walks a few of them; a node with at most
// 64 entries (a narrow matrix) takes one wave, whose reduction steps need no
// wait on other waves.
inline unsigned split_reduce_threads(int n_entries)
{
    return n_entries >= 4096 ? (unsigned)kSplitReduceMaxThreads : n_entries <= 64 ? 64u : 256u;
}

inline FillPlan plan_rows(const PlanCtx* c)
{
    FillPlan p{};
    p.kind = kFillRowsKind;
    p.threads = kLevelThreads;
    const int S = c->S, w = c->bin_bytes, F = c->F;
    // The cheapest plan of one accumulation mode (false: none fits).
    auto search = [&](int acc, FillPlan& q) {
        double best = 1e300;
        bool found = false;
        for (int lt = 32; lt >= 2; lt >>= 1) {
            if (lt < w) continue;
            const int tile = lt / w;
            const int force_tile = c->tune[4];
            if (force_tile > 0 && tile != force_tile) continue;
            const int nf = std::min(tile, F);
            const int n_tiles = (F + nf - 1) / nf;
            for (int lc = 4; lc >= 0; --lc) {
                const int force_lc = c->tune[3];
                if (force_lc >= 0 && lc != force_lc) continue;
                for (int il = 0; il <= (acc == kWide ? 1 : 0); ++il) {
                    if (c->tune[8] >= 0 && il != c->tune[8]) continue;
                    // packed sums live in registers, wide sums in LDS
                    const int ra = acc == kPacked ? kRegAccCells : 0;
                    if (ra > 0 && nf * S > ra * kLevelThreads) continue;
                    const int e = ra > 0 ? kRegAccEntries : kWideRowEntries;
                    const int64_t words = il ? (int64_t)2 * S * (tile << lc)
                                             : (int64_t)nf * (acc == kWide ? 2 : 1) * (S << lc);
                    if (words * 8 > kTileLdsBudget) continue;
                    int drain = 0;
                    double drain_ops = 0.0;
                    if (acc == kPacked) {
                        drain = packed_drain_steps(kLevelThreads, lc, e);
                        if (drain == 0) continue;
                        drain_ops = 2.0 * nf * S * (1 << lc) / ((double)kLevelThreads * e * drain) * n_tiles;
                    }
                    // an interleaved tile over 32-byte chunks takes each row on
                    // two lanes (il = 2) unless switched off
                    const int il_mode = il && lt == 2 * kPairHalfBytes && c->tune[10] != 0 ? 2 : il;
                    const double cost = rows_cost(acc, lc, F, n_tiles, c->rm_stride, drain_ops, il_mode, tile);
                    if (cost < best) {
                        best = cost;
                        found = true;
                        q.acc = acc;
                        q.lc = lc;
                        q.tile = tile;
                        q.lt = lt;
                        q.ra = ra;
                        q.il = il_mode;
                        q.drain = drain;
                        q.step_rows = (int64_t)kLevelThreads / (il_mode == 2 ? 2 : 1) * e;
                        q.lds_bytes = (size_t)(words + kFixWords) * 8;
                    }
                }
            }
        }
        return found;
    };
    // At P <= 19 packed sums halve the adds, but a wide plan with lane pairs
    // measured faster wherever one fits (level fills, 10M x 28: 0.435 against
    // 0.454 ms per step; 131,072 x 16,384: 0.486 against 0.561 ms): the packed
    // row fill keeps one lane per row and a feature-major tile.  Otherwise
    // packed sums where they fit, else wide ones.
    FillPlan wide = p, packed = p;
    const bool have_wide = search(kWide, wide);
    const bool have_packed = c->precision <= kPackedMaxBits && search(kPacked, packed);
    bool found = true;
    if (have_packed && !(have_wide && wide.il == 2)) p = packed;
    else if (have_wide) p = wide;
    else found = false;
    if (!found) {   // one wide feature of one copy always fits (S <= HGB_MAX_SLOTS)
        p.acc = kWide;
        p.lc = 0;
        p.tile = 1;
        p.lt = w;
        p.ra = 0;
        p.il = 0;
        p.drain = 0;
        p.step_rows = (int64_t)kLevelThreads * kWideRowEntries;
        p.lds_bytes = (size_t)(2 * S + kFixWords) * 8;
    }
    return p;
}

inline FillPlan plan_fill(const PlanCtx* c, bool root, bool rm)
{
    if (!root && rm) return plan_rows(c);
    FillPlan p{};
    const int S = c->S;
    const int w = c->bin_bytes;
    p.kind = root ? kFillRoot : (rm ? kFillRowsKind : kFillCols);
    p.threads = root ? kRootThreads : kLevelThreads;
    auto per_thread_of = [&](int tile) {
        return p.kind == kFillRoot ? kRootRows : (p.kind == kFillCols ? cols_entries(tile) : kLevelEntries);
    };
    const int64_t budget = kTileLdsBudget;
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
                    p.il = 0;
                }
            }
        }
        // The root's interleaved tile with packed sums: 16 positions, 2^lc >= 2
        // copies (so that the 64 lanes of an add meet 32 bank pairs and a
        // step's 4 rows per thread put at most 2,048 rows on a copy), and
        // each thread's share of the S * 16 cells in registers between drains.
        // One-byte bins without the skipped slot: the register cells fit
        // beside 16 positions of loads only there.
        for (int lc = 1; root && acc == kPacked && lc <= 2; ++lc) {
            const int tf = 16;
            if (w != 1 || c->skip) break;
            if (c->tune[9] == 0) break;
            if (c->tune[1] > 0 && tf != c->tune[1]) break;
            if (c->tune[0] >= 0 && lc != c->tune[0]) continue;
            if ((int64_t)S * tf > (int64_t)kRootIlPackedCells * kRootThreads) break;
            if ((int64_t)root_il_words(kPacked, tf, S, lc) * 8 > budget) continue;
            const int drain = packed_drain_steps(kRootThreads, lc, kRootRows);
            if (drain == 0) continue;
            const int64_t il_tiles = (c->F + tf - 1) / tf;
            const int64_t il_chunks = std::max<int64_t>(1, kRootItemsPerCu * c->n_cu / il_tiles);
            const double merge_s = il_chunks > 1 ? 4e-6 + 2.0 * il_chunks * c->F * S * 16.0 / 5.0e12 : 0.0;
            const double cells = std::max(1.0, (double)c->n * c->F);
            const double cost = fill_cost_il_packed(lc, tf, c->F, w, S, drain) + merge_s / cells;
            if (cost < best || (c->tune[9] == 1 && !(found && p.il))) {
                best = cost;
                found = true;
                p.acc = kPacked;
                p.lc = lc;
                p.tile = tf;
                p.lt = 0;
                p.il = 1;
                p.drain = drain;
            }
        }
        // The root's interleaved tile (wide sums): tf positions of 2^lc copies.
        // A position's bins take w registers per thread; 32 registers of them
        // fit beside the skipped slot's bookkeeping only up to 16 bytes.
        for (int tf = 32; root && acc == kWide && tf >= 8; tf >>= 1) {
            if (tf * w > (c->skip ? 16 : 32)) continue;
            if (c->tune[9] == 0) break;
            if (c->tune[1] > 0 && tf != c->tune[1]) continue;
            // Few tiles mean many row chunks per tile, whose partial histograms
            // a k_merge launch sums: its launch and traffic, spread per cell.
            const int64_t il_tiles = (c->F + tf - 1) / tf;
            const int64_t il_chunks = std::max<int64_t>(1, kRootItemsPerCu * c->n_cu / il_tiles);
            const double merge_s = il_chunks > 1 ? 4e-6 + 2.0 * il_chunks * c->F * S * 16.0 / 5.0e12 : 0.0;
            const double cells = std::max(1.0, (double)c->n * c->F);
            for (int lc = 0; lc <= 4; ++lc) {
                if (c->tune[0] >= 0 && lc != c->tune[0]) continue;
                if ((int64_t)2 * S * (tf << lc) * 8 > budget) continue;
                const double cost = fill_cost_il(lc, tf, c->F, w) + merge_s / cells;
                if (cost < best || (c->tune[9] == 1 && !(found && p.il))) {
                    best = cost;
                    found = true;
                    p.acc = kWide;
                    p.lc = lc;
                    p.tile = tf;
                    p.lt = 0;
                    p.il = 1;
                    p.drain = 0;
                }
            }
        }
    }
    if (!found) {   // one wide feature of one copy always fits (S <= HGB_MAX_SLOTS)
        p.acc = kWide;
        p.lc = 0;
        p.tile = 1;
        p.lt = p.kind == kFillRowsKind ? w : 0;
        p.il = 0;
    }
    if (p.il) {
        // the last tile may be partial; the tile itself never narrower than 8
        p.lds_bytes = (size_t)(root_il_words(p.acc, p.tile, S, p.lc) + kFixWords) * 8;
        p.step_rows = (int64_t)p.threads * kRootRows;
        if (p.acc == kWide) p.drain = 0;
        return p;
    }
    if (p.kind != kFillRowsKind) {
        // rows loads cover exactly `tile` features; the others take min(NF, F)
        while (p.tile > 1 && (p.tile >> 1) >= c->F) p.tile >>= 1;
    }
    p.lds_bytes = (size_t)(p.tile * feature_lds(p.acc, S, p.lc) + 8 * kFixWords);
    p.step_rows = (int64_t)p.threads * per_thread_of(p.tile);
    p.drain = p.acc == kPacked ? packed_drain_steps(p.threads, p.lc, per_thread_of(p.tile)) : 0;
    return p;
}


// Feature tiles (f0, width) of a build.  Root tiles of the feature-major
// kernels have exactly the kernel's width: equal tiles when a divisor of F
// close to the planned width exists (plan.tile is narrowed to it), else full
// tiles, then the remainder split into powers of two, each width its own
// launch.  Interleaved and level tiles are plan.tile wide, the last one
// possibly narrower (those kernels take the width at run time).
inline std::vector<std::pair<int, int>> feature_tiles(const PlanCtx* c, FillPlan& plan, bool root)
{
    std::vector<std::pair<int, int>> tiles;
    if (root && !plan.il) {
        for (int d = plan.tile; d >= 1 && 2 * d > plan.tile; --d)
            if (c->F % d == 0) {
                plan.tile = d;
                break;
            }
    }
    int f0 = 0;
    for (; f0 + plan.tile <= c->F; f0 += plan.tile) tiles.emplace_back(f0, plan.tile);
    if (f0 < c->F) {
        if (root && !plan.il) {
            for (int wdt = plan.tile >> 1; wdt >= 1; wdt >>= 1)
                if (f0 + wdt <= c->F) {
                    tiles.emplace_back(f0, wdt);
                    f0 += wdt;
                }
        } else {
            tiles.emplace_back(f0, c->F - f0);
        }
    }
    return tiles;
}

// The cut of a level below the root.  The level order is cut into equal-cost
// shares, one per block (kLevelBlocksPerCu per CU, divided among the feature
// tiles), so every CU gets the same work whatever the node sizes.  A piece
// costs its rows plus a fixed piece_rows (zeroing the tile, the pipeline's
// ramp, writing the tile out), so a share that touches many small nodes takes
// fewer rows.  A share crosses node boundaries: its block takes one item per
// node it touches, in order.  A node inside one share is stored straight into
// its slot; a node split over several shares leaves one partial histogram per
// share, summed by merges in groups of kMergeGroup (added atomically into the
// zeroed slot when there are several groups).  Empty nodes' slots are cleared.
struct LevelCut {
    std::vector<FillItem> items;         // per block, in block order
    std::vector<int32_t> block_first;    // items of block b: [block_first[b], block_first[b + 1])
    std::vector<MergeEntry> merges;
    std::vector<int32_t> zero_slots;     // slots to clear before the merges add into them
    int64_t n_partial = 0;               // partial histograms written
    int64_t budget = 0;                  // cost of a share, in rows
    int64_t piece_rows = 0;              // fixed cost of a piece, in rows
    int64_t n_shares = 0;
    int64_t align = 128;                 // cuts inside a node fall on multiples of this
};

// x rounded down to a multiple of `align` (> 0); a mask when align is a power
// of two, as it is unless overridden (a 64-bit division costs tens of cycles
// and the level cut rounds once per piece).
inline int64_t round_down(int64_t x, int64_t align)
{
    return (align & (align - 1)) == 0 ? x & ~(align - 1) : x / align * align;
}

// The number of shares the level cut makes from nodes of count[] rows with a
// cost budget b per share (each piece costs piece_rows plus its rows; b is at
// least piece_rows + align), or a number above `limit` once it passes it.  The
// cut fills shares greedily in level order: a share is closed once less than
// piece_rows + align of its budget is left; a piece that does not end its node
// ends on a multiple of align rows.  A fresh share's piece that does not end
// its node therefore takes `full` = round_down(b - piece_rows) rows and closes
// the share (less than align is left), so a node's run of such pieces is
// counted with one division instead of piece by piece.
inline int64_t level_shares(const std::vector<int64_t>& count, int64_t b, int64_t piece_rows, int64_t align,
                            int64_t limit)
{
    const int64_t room = b - piece_rows;   // >= align
    const int64_t full = round_down(room, align);
    int64_t left = b, n = 0;
    bool open = false;
    for (const int64_t rows : count) {
        int64_t rem = rows;
        while (rem > 0) {
            if (open && left < piece_rows + align) {
                if (++n > limit) return n;
                left = b;
                open = false;
            }
            if (!open && rem > room) {
                // k fresh shares of `full` rows until at most `room` are left
                // (rem stays > 0: full <= room); all but the last are closed
                const int64_t k = (rem - room + full - 1) / full;
                n += k - 1;
                if (n > limit) return n;
                rem -= k * full;
                left = room - full;
                open = true;
                continue;
            }
            int64_t take = std::min(rem, left - piece_rows);
            if (take < rem) take = std::min(std::max<int64_t>(round_down(take, align), align), rem);
            left -= piece_rows + take;
            open = true;
            rem -= take;
        }
    }
    return n + (open ? 1 : 0);
}

// begin[i], count[i]: node i's rows in the level order (count 0: empty or
// skipped); slots[i]: its output slot (-1: skipped).  Returns nullptr, or a
// message when the level needs more partial histograms or items than the
// kernels index.
inline const char* cut_level(const PlanCtx* c, const FillPlan& plan, const std::vector<std::pair<int, int>>& tiles,
                             const std::vector<int64_t>& begin, const std::vector<int64_t>& count,
                             const std::vector<int32_t>& slots, LevelCut* out)
{
    const int n_nodes = (int)begin.size();
    const int n_tiles = (int)tiles.size();
    int64_t bpc = kLevelBlocksPerCu;
    if (c->tune[5] > 0) bpc = c->tune[5];
    const int64_t shares = std::max<int64_t>(1, bpc * c->n_cu / n_tiles);
    int64_t align = 128;
    if (c->tune[6] > 0) align = (c->tune[6] + 7) / 8 * 8;
    int64_t piece_rows = std::max<int64_t>((int64_t)(kPieceRowsPerCell * std::min(plan.tile, c->F) * c->S), 1);
    if (c->tune[7] >= 0) piece_rows = std::max(c->tune[7], 1);
    int64_t nonempty = 0, built = 0;   // skipped nodes count 0 rows
    for (int i = 0; i < n_nodes; ++i) {
        nonempty += count[i] > 0;
        built += count[i];
    }
    int64_t budget = 0;

    // pieces of each share, in level order: (node, begin, end, chunk of node)
    struct Piece {
        int node;
        int64_t rb, re;
        int chunk;
    };
    std::vector<Piece> pieces;
    std::vector<int64_t> share_first;
    std::vector<int> pieces_of;
    auto cut = [&]() {
        pieces.clear();
        share_first.assign(1, 0);
        pieces_of.assign(n_nodes, 0);
        int64_t left = budget;   // cost left in the current share
        bool open = false;       // the current share holds a piece
        for (int i = 0; i < n_nodes; ++i) {
            int64_t at = begin[i];
            const int64_t end = begin[i] + count[i];
            while (at < end) {
                if (open && left < piece_rows + align) {   // close the share
                    share_first.push_back((int64_t)pieces.size());
                    left = budget;
                    open = false;
                }
                int64_t take = std::min(end - at, left - piece_rows);
                // inside a node, cut on multiples of `align` rows
                if (at + take < end) take = std::max<int64_t>(round_down(take, align), align);
                take = std::min(take, end - at);
                pieces.push_back({i, at, at + take, pieces_of[i]++});
                left -= piece_rows + take;
                open = true;
                at += take;
            }
        }
        if (open) share_first.push_back((int64_t)pieces.size());
        return (int64_t)share_first.size() - 1;
    };
    // A budget close to the smallest whose cut fits one round of blocks (a
    // larger budget never needs more shares): gallop up from the lower bound,
    // then bisect until the bracket is within 1/256 of the budget.  The host
    // plans every level between device steps, so the search is kept short.
    {
        int64_t lo = std::max<int64_t>((built + piece_rows * nonempty + shares - 1) / shares,
                                       piece_rows + align);
        const int64_t cap = std::max<int64_t>(built + piece_rows * (nonempty + 1) + align, lo);
        auto fits = [&](int64_t b) { return level_shares(count, b, piece_rows, align, shares) <= shares; };
        int64_t hi = lo;
        while (hi < cap && !fits(hi)) {
            lo = hi + 1;
            hi = std::min<int64_t>(cap, 2 * hi);
        }
        while (hi - lo > std::max<int64_t>(align, hi / 256)) {
            const int64_t mid = lo + (hi - lo) / 2;
            if (fits(mid)) hi = mid;
            else lo = mid + 1;
        }
        budget = hi;
    }
    const int64_t n_shares = cut();

    // partial slots and merges of split nodes; slots to zero first
    std::vector<int32_t> partial_base(n_nodes, -1);
    out->merges.clear();
    out->zero_slots.clear();
    int64_t n_partial = 0;
    for (int i = 0; i < n_nodes; ++i) {
        if (count[i] == 0 && slots[i] >= 0) out->zero_slots.push_back(slots[i]);   // -1: skipped
        if (pieces_of[i] <= 1) continue;
        if (n_partial > INT32_MAX / 2) return "build_level: too many partial histograms";
        partial_base[i] = (int32_t)n_partial;
        const int groups = (pieces_of[i] + kMergeGroup - 1) / kMergeGroup;
        if (groups > 1) out->zero_slots.push_back(slots[i]);
        for (int g = 0; g < groups; ++g) {
            MergeEntry m{};
            m.out_slot = slots[i];
            m.first = (int32_t)(n_partial + (int64_t)g * kMergeGroup);
            m.count = std::min(kMergeGroup, pieces_of[i] - g * kMergeGroup);
            m.atomic = groups > 1 ? 1 : 0;
            out->merges.push_back(m);
        }
        n_partial += pieces_of[i];
    }
    if (n_partial > INT32_MAX / 2 || (int64_t)out->merges.size() > kMaxLevelNodes)
        return "build_level: too many partial histograms";

    // blocks (share, tile), tile fastest: the tiles of one share read the same
    // rows, and the kernel gives each XCD a contiguous run of blocks
    out->items.clear();
    out->block_first.clear();
    if (pieces.size() * (size_t)n_tiles > (size_t)INT32_MAX / 8 || n_shares * n_tiles > INT32_MAX / 8)
        return "build_level: too many fill items";
    out->items.reserve(pieces.size() * (size_t)n_tiles);
    out->block_first.reserve((size_t)n_shares * n_tiles + 1);
    for (int64_t r = 0; r < n_shares; ++r)
        for (int t = 0; t < n_tiles; ++t) {
            out->block_first.push_back((int32_t)out->items.size());
            for (int64_t k = share_first[r]; k < share_first[r + 1]; ++k) {
                const Piece& pc = pieces[k];
                FillItem it{};
                if (partial_base[pc.node] >= 0) {
                    it.out_slot = partial_base[pc.node] + pc.chunk;
                    it.dest = kDestPartial;
                } else {
                    it.out_slot = slots[pc.node];
                    it.dest = kDestStore;
                }
                it.row_begin = (int32_t)pc.rb;
                it.row_end = (int32_t)pc.re;
                it.f0_nf = tiles[t].first | (tiles[t].second << 16);
                out->items.push_back(it);
            }
        }
    out->block_first.push_back((int32_t)out->items.size());
    out->n_partial = n_partial;
    out->budget = budget;
    out->piece_rows = piece_rows;
    out->n_shares = n_shares;
    out->align = align;
    return nullptr;
}

// The root's items: about kRootItemsPerCu x (CUs) equal row chunks, a
// multiple of 128 rows (the bin and (g, h) loads stay cache-line aligned), in
// (chunk, tile) order: the tiles of one chunk read the same (g, h) rows, and
// the kernel gives each XCD a contiguous run of items.  groups[w] holds the
// items of tiles of width w (one launch each); with the interleaved tile every
// item (the last tile possibly partial) is in groups[0], one launch.  The
// interleaved tile covers many features, so a tile's chunks are many: each
// writes a partial histogram, summed by merges of kMergeGroup (atomically
// when there are several groups).  Feature-major tiles have few chunks each
// and add theirs atomically into the zeroed slot.
struct RootCut {
    std::vector<FillItem> groups[9];
    std::vector<MergeEntry> merges;
    int64_t chunk = 0, n_chunks = 0;
    bool use_partial = false;   // chunks write partial histograms (merged afterwards)
    bool zero_root = false;     // the root's slot is cleared first (atomic adds)
    size_t n_items = 0;
};

inline void cut_root(const PlanCtx* c, const FillPlan& plan, const std::vector<std::pair<int, int>>& tiles,
                     int64_t total, int32_t slot, RootCut* out)
{
    int64_t ipc = kRootItemsPerCu;
    if (c->tune[2] > 0) ipc = c->tune[2];
    const int64_t target = ipc * c->n_cu;
    int64_t align = 128;
    if (c->tune[6] > 0) align = (c->tune[6] + 7) / 8 * 8;
    const int n_tiles = (int)tiles.size();
    // Equal items, at most `target` of them: one item more than a multiple of
    // the resident blocks would cost a whole extra round.
    const int64_t chunks = std::max<int64_t>(1, target / n_tiles);
    int64_t ch = (total + chunks - 1) / chunks;
    ch = std::max<int64_t>((ch + align - 1) / align * align, align);
    const int64_t nchunks = (total + ch - 1) / ch;
    out->chunk = ch;
    out->n_chunks = nchunks;
    out->use_partial = plan.il && nchunks > 1;
    out->merges.clear();
    if (out->use_partial) {
        const int64_t n_groups = (nchunks + kMergeGroup - 1) / kMergeGroup;
        for (int64_t g = 0; g < n_groups; ++g) {
            MergeEntry m{};
            m.out_slot = slot;
            m.first = (int32_t)(g * kMergeGroup);
            m.count = (int32_t)std::min<int64_t>(kMergeGroup, nchunks - g * kMergeGroup);
            m.atomic = n_groups > 1 ? 1 : 0;
            out->merges.push_back(m);
        }
    }
    out->zero_root = nchunks > 1 && (!out->use_partial || out->merges.size() > 1);
    out->n_items = 0;
    for (auto& g : out->groups) g.clear();
    for (int64_t j = 0; j < nchunks; ++j)
        for (int t = 0; t < n_tiles; ++t) {
            FillItem it{};
            it.out_slot = out->use_partial ? (int32_t)j : slot;
            it.row_begin = (int32_t)(j * ch);
            it.row_end = (int32_t)std::min<int64_t>((j + 1) * ch, total);
            it.f0_nf = tiles[t].first | (tiles[t].second << 16);
            it.dest = out->use_partial ? kDestPartial : (nchunks > 1 ? kDestAtomic : kDestStore);
            out->groups[plan.il ? 0 : tiles[t].second].push_back(it);
            ++out->n_items;
        }
}

// The partition's chunks: each node's positions [offs[i], offs[i + 1]) in
// pieces of kPartChunk, node by node; first[i] is node i's first chunk
// (first[n_nodes] = the chunk count).  Positions are stepped in 64 bits: the
// last chunk of a node may end within kPartChunk of 2^31.
inline void part_chunks(const std::vector<int32_t>& offs, int n_nodes, std::vector<PartItem>* items,
                        std::vector<int32_t>* first)
{
    items->clear();
    first->assign((size_t)n_nodes + 1, 0);
    for (int i = 0; i < n_nodes; ++i) {
        (*first)[i] = (int32_t)items->size();
        for (int64_t b = offs[i]; b < offs[i + 1]; b += kPartChunk)
            items->push_back({i, (int32_t)b, (int32_t)std::min<int64_t>(b + kPartChunk, offs[i + 1]), offs[i]});
    }
    (*first)[n_nodes] = (int32_t)items->size();
}

}  // namespace hgb
