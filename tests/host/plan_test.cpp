// Host-only tests of the launch planner (hgb_plan.h): fill plans, feature
// tiles, the level cut, the root cut and the partition's chunks, on the five
// workloads' shapes and on adversarial node lists (65,535 nodes, empty and
// skipped nodes, one giant node, level orders ending near 2^31).  Built with
// the address and undefined-behaviour sanitizers by tests/test_sanitizers.py.
#include "hgb_plan.h"

#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <tuple>

using namespace hgb;

static int g_checks = 0;
#define CHECK(cond, ...)                                                        \
    do {                                                                        \
        ++g_checks;                                                             \
        if (!(cond)) {                                                          \
            std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            std::fprintf(stderr, __VA_ARGS__);                                  \
            std::fprintf(stderr, "\n");                                         \
            std::exit(1);                                                       \
        }                                                                       \
    } while (0)

static PlanCtx ctx_of(int64_t n, int F, int S, int w, int precision, bool skip, bool rm)
{
    PlanCtx c;
    c.n = n;
    c.F = F;
    c.S = S;
    c.bin_bytes = w;
    c.precision = precision;
    c.skip = skip;
    c.rm_stride = rm ? ((int64_t)F * w + 15) / 16 * 16 : 0;
    c.n_cu = 256;
    return c;
}

// Rows one copy-slot of a packed tile can see between drains: the period's
// steps times the rows each copy takes per step, plus the root's tail rows.
static void check_plan(const PlanCtx& c, const FillPlan& p, bool root, bool rm)
{
    CHECK(p.lds_bytes > 0 && (int64_t)p.lds_bytes <= kFillLdsBudget, "lds %zu", p.lds_bytes);
    CHECK(p.tile >= 1, "tile %d", p.tile);
    CHECK(p.threads == 1024, "threads %d", p.threads);
    CHECK(p.acc == kWide || p.acc == kPacked, "acc %d", p.acc);
    if (p.acc == kPacked) {
        CHECK(c.precision <= kPackedMaxBits, "packed at P = %d", c.precision);
        CHECK(p.drain >= 1, "drain %d", p.drain);
        int per_thread = root ? kRootRows : (p.kind == kFillRowsKind ? 1 : cols_entries(p.tile));
        if (p.kind == kFillRowsKind && p.ra > 0) per_thread = 1;
        const int64_t per_copy_step = (int64_t)(p.threads >> p.lc) * per_thread;
        CHECK(p.drain * per_copy_step + (kRootRows - 1) <= kPackedRowsPerCopy,
              "drain %d x %lld rows per copy and step", p.drain, (long long)per_copy_step);
    }
    if (root && p.il) {
        CHECK(p.tile == 8 || p.tile == 16 || p.tile == 32, "il tile %d", p.tile);
        CHECK(p.tile * c.bin_bytes <= (c.skip ? 16 : 32), "il tile bytes");
        CHECK((int64_t)(root_il_words(p.acc, p.tile, c.S, p.lc) + kFixWords) * 8 == (int64_t)p.lds_bytes, "il lds");
    }
    if (!root && rm) {
        CHECK(p.kind == kFillRowsKind, "rows kind");
        CHECK(p.lt >= c.bin_bytes && p.lt % c.bin_bytes == 0 && p.tile == p.lt / c.bin_bytes, "lt %d", p.lt);
        if (p.acc == kPacked) CHECK(p.ra > 0 && (int64_t)std::min(p.tile, c.F) * c.S <= (int64_t)p.ra * 1024, "ra");
        CHECK(p.il >= 0 && p.il <= 2, "il %d", p.il);
        // lane pairs: interleaved wide sums over 32-byte chunks, unless switched off
        if (p.il == 2) CHECK(p.lt == 2 * kPairHalfBytes && p.acc == kWide && c.tune[10] != 0, "pair plan");
        if (p.il == 1) CHECK(p.lt != 2 * kPairHalfBytes || c.tune[10] == 0, "a 32-byte interleaved plan without pairs");
    }
}

static void check_tiles(const PlanCtx& c, const FillPlan& p, const std::vector<std::pair<int, int>>& tiles, bool root)
{
    int at = 0;
    for (const auto& t : tiles) {
        CHECK(t.first == at, "tiles not contiguous at %d", at);
        CHECK(t.second >= 1 && t.first + t.second <= c.F, "tile (%d, %d)", t.first, t.second);
        if (root && !p.il) CHECK(t.second <= 8 && (t.second == p.tile || (t.second & (t.second - 1)) == 0), "root tile width %d", t.second);
        else CHECK(t.second <= p.tile, "tile width %d > %d", t.second, p.tile);
        at += t.second;
    }
    CHECK(at == c.F, "tiles cover %d of %d features", at, c.F);
}

// The level cut's invariants for node lists begin/count/slots.
static void check_level(const PlanCtx& c, const FillPlan& p, const std::vector<std::pair<int, int>>& tiles,
                        const std::vector<int64_t>& begin, const std::vector<int64_t>& count,
                        const std::vector<int32_t>& slots, const char* what)
{
    LevelCut cut;
    const char* err = cut_level(&c, p, tiles, begin, count, slots, &cut);
    CHECK(err == nullptr, "%s: %s", what, err);
    const int n_nodes = (int)begin.size();
    const int n_tiles = (int)tiles.size();
    const int64_t n_blocks = (int64_t)cut.block_first.size() - 1;
    CHECK(n_blocks == cut.n_shares * n_tiles, "%s: blocks", what);
    const int64_t shares_cap = std::max<int64_t>(1, kLevelBlocksPerCu * c.n_cu / n_tiles);
    CHECK(cut.n_shares <= shares_cap, "%s: %lld shares > one round of %lld", what, (long long)cut.n_shares,
          (long long)shares_cap);
    CHECK(cut.block_first.front() == 0 && cut.block_first.back() == (int32_t)cut.items.size(), "%s: block list", what);
    CHECK(level_shares(count, cut.budget, cut.piece_rows, cut.align, INT64_MAX) == cut.n_shares,
          "%s: counted shares differ from the cut's %lld", what, (long long)cut.n_shares);
    // node of each item: by its row range (the nodes' ranges are disjoint and ordered)
    std::vector<std::pair<int64_t, int>> starts;
    for (int i = 0; i < n_nodes; ++i)
        if (count[i] > 0) starts.emplace_back(begin[i], i);
    auto node_of = [&](int64_t r) {
        auto it = std::upper_bound(starts.begin(), starts.end(), std::make_pair(r, INT32_MAX));
        CHECK(it != starts.begin(), "%s: row %lld before every node", what, (long long)r);
        return (--it)->second;
    };
    // per tile: the pieces, which must tile every node's [begin, begin + count) exactly
    std::vector<std::vector<std::pair<int64_t, int64_t>>> pieces(n_tiles);
    std::map<int, std::vector<int32_t>> partial_of;   // node -> its partial slots (first tile)
    std::vector<int> pieces_per_node(n_nodes, 0);
    for (int64_t b = 0; b < n_blocks; ++b) {
        int64_t cost = 0;
        CHECK(cut.block_first[b] <= cut.block_first[b + 1], "%s: block order", what);
        const int t = (int)(b % n_tiles);
        for (int32_t k = cut.block_first[b]; k < cut.block_first[b + 1]; ++k) {
            const FillItem& it = cut.items[k];
            const int f0 = it.f0_nf & 0xffff, nf = it.f0_nf >> 16;
            if (it.row_begin >= it.row_end || f0 != tiles[t].first || nf != tiles[t].second)
                CHECK(false, "%s: item %d (rows %d..%d, tile %d)", what, k, it.row_begin, it.row_end, t);
            pieces[t].emplace_back(it.row_begin, it.row_end);
            cost += cut.piece_rows + (it.row_end - it.row_begin);
            if (t != 0) continue;
            const int node = node_of(it.row_begin);
            CHECK(it.row_end <= begin[node] + count[node], "%s: item crosses node %d", what, node);
            CHECK(slots[node] >= 0, "%s: skipped node %d read", what, node);
            CHECK((it.row_begin - begin[node]) % cut.align == 0, "%s: cut inside node %d off the alignment", what, node);
            ++pieces_per_node[node];
            if (it.dest == kDestPartial) partial_of[node].push_back(it.out_slot);
            else CHECK(it.dest == kDestStore && it.out_slot == slots[node], "%s: store slot", what);
        }
        CHECK(cost <= cut.budget, "%s: block %lld costs %lld > budget %lld", what, (long long)b, (long long)cost,
              (long long)cut.budget);
    }
    for (int t = 0; t < n_tiles; ++t) {
        auto& v = pieces[t];
        std::sort(v.begin(), v.end());
        size_t k = 0;
        for (int i = 0; i < n_nodes; ++i) {
            if (count[i] == 0) continue;
            int64_t at = begin[i];
            while (k < v.size() && v[k].first < begin[i] + count[i]) {
                if (v[k].first != at) CHECK(false, "%s: node %d tile %d: gap or overlap at %lld", what, i, t, (long long)at);
                at = v[k].second;
                ++k;
            }
            if (at != begin[i] + count[i])
                CHECK(false, "%s: node %d tile %d covered to %lld of %lld", what, i, t, (long long)at,
                      (long long)(begin[i] + count[i]));
        }
        CHECK(k == v.size(), "%s: tile %d has pieces outside every node", what, t);
    }
    // partials and merges: each split node's partial slots are consecutive,
    // and the merges sum each exactly once into its slot
    std::vector<int> merged(cut.n_partial, 0);
    std::map<int32_t, int> groups_of_slot;
    for (const MergeEntry& m : cut.merges) {
        CHECK(m.count >= 1 && m.count <= kMergeGroup, "%s: merge count %d", what, m.count);
        CHECK(m.first >= 0 && m.first + m.count <= cut.n_partial, "%s: merge range", what);
        for (int j = 0; j < m.count; ++j) ++merged[m.first + j];
        ++groups_of_slot[m.out_slot];
    }
    for (int64_t j = 0; j < cut.n_partial; ++j)
        if (merged[j] != 1) CHECK(false, "%s: partial %lld merged %d times", what, (long long)j, merged[j]);
    for (const MergeEntry& m : cut.merges) CHECK((m.atomic != 0) == (groups_of_slot[m.out_slot] > 1), "%s: atomic flag", what);
    int64_t n_partial = 0;
    for (int i = 0; i < n_nodes; ++i) {
        if (pieces_per_node[i] <= 1) {
            CHECK(partial_of.count(i) == 0, "%s: whole node %d wrote a partial", what, i);
            continue;
        }
        auto v = partial_of[i];
        std::sort(v.begin(), v.end());
        CHECK((int)v.size() == pieces_per_node[i], "%s: node %d partials", what, i);
        for (size_t k = 1; k < v.size(); ++k) CHECK(v[k] == v[0] + (int32_t)k, "%s: node %d partial slots", what, i);
        CHECK(groups_of_slot.count(slots[i]) == 1, "%s: node %d has no merge", what, i);
        n_partial += (int64_t)v.size();
    }
    CHECK(n_partial == cut.n_partial, "%s: partial count", what);
    // slots the fill clears: every empty built node and every node merged atomically
    std::vector<int32_t> zs = cut.zero_slots;
    std::sort(zs.begin(), zs.end());
    CHECK(std::adjacent_find(zs.begin(), zs.end()) == zs.end(), "%s: a slot cleared twice", what);
    for (int i = 0; i < n_nodes; ++i) {
        const bool want = slots[i] >= 0 && (count[i] == 0 || groups_of_slot[slots[i]] > 1);
        const bool have = std::binary_search(zs.begin(), zs.end(), slots[i]);
        CHECK(want == have, "%s: node %d slot clear %d, want %d", what, i, (int)have, (int)want);
    }
}

static void check_root(const PlanCtx& c, FillPlan p, const char* what)
{
    const auto tiles = feature_tiles(&c, p, true);
    check_tiles(c, p, tiles, true);
    RootCut rc;
    cut_root(&c, p, tiles, c.n, 0, &rc);
    CHECK(rc.chunk % 128 == 0 && rc.chunk > 0, "%s: chunk %lld", what, (long long)rc.chunk);
    CHECK(rc.n_chunks * (int64_t)tiles.size() <= std::max<int64_t>(c.n_cu, (int64_t)tiles.size()), "%s: root items %lld", what,
          (long long)(rc.n_chunks * (int64_t)tiles.size()));
    std::map<int, std::vector<std::pair<int64_t, int64_t>>> by_f0;
    size_t items = 0;
    for (int wdt = 0; wdt <= 8; ++wdt)
        for (const FillItem& it : rc.groups[wdt]) {
            ++items;
            if (!p.il) CHECK((it.f0_nf >> 16) == wdt, "%s: group width", what);
            else CHECK(wdt == 0, "%s: interleaved items in one group", what);
            CHECK(it.row_begin < it.row_end && it.row_begin % rc.chunk == 0, "%s: chunk start", what);
            if (rc.use_partial) CHECK(it.dest == kDestPartial && it.out_slot == it.row_begin / rc.chunk, "%s: partial slot", what);
            else CHECK(it.dest == (rc.n_chunks > 1 ? kDestAtomic : kDestStore) && it.out_slot == 0, "%s: dest", what);
            by_f0[it.f0_nf & 0xffff].emplace_back(it.row_begin, it.row_end);
        }
    CHECK(items == rc.n_items && by_f0.size() == tiles.size(), "%s: items", what);
    for (auto& kv : by_f0) {
        std::sort(kv.second.begin(), kv.second.end());
        int64_t at = 0;
        for (auto& pr : kv.second) {
            CHECK(pr.first == at, "%s: root rows gap", what);
            at = pr.second;
        }
        CHECK(at == c.n, "%s: root rows covered to %lld", what, (long long)at);
    }
    if (rc.use_partial) {
        std::vector<int> seen(rc.n_chunks, 0);
        for (const MergeEntry& m : rc.merges)
            for (int j = 0; j < m.count; ++j) ++seen[m.first + j];
        for (int64_t j = 0; j < rc.n_chunks; ++j) CHECK(seen[j] == 1, "%s: chunk %lld merged %d times", what, (long long)j, seen[j]);
        CHECK(rc.zero_root == (rc.merges.size() > 1), "%s: zero_root", what);
    } else {
        CHECK(rc.merges.empty() && rc.zero_root == (rc.n_chunks > 1), "%s: atomic root", what);
    }
}

// level_shares against the greedy rule applied piece by piece: a share takes
// pieces while at least piece_rows + align of its budget is left, each piece
// as many rows as the rest of the budget allows after its piece_rows, cut to
// a multiple of align unless it ends the node.  Also the early exit: a
// count above `limit` is reported as such.
static void check_level_shares(std::mt19937_64& rng)
{
    for (int k = 0; k < 3000; ++k) {
        const int nn = 1 + (int)(rng() % 40);
        std::vector<int64_t> count(nn);
        for (auto& v : count) v = rng() % 4 == 0 ? 0 : (int64_t)(rng() % (rng() % 2 ? 300 : 30000));
        const int64_t align = rng() % 3 == 0 ? 8 * (1 + (int64_t)(rng() % 40)) : (int64_t)1 << (3 + rng() % 6);
        const int64_t piece_rows = 1 + (int64_t)(rng() % 2000);
        const int64_t b = piece_rows + align + (int64_t)(rng() % (rng() % 2 ? 500 : 20000));
        int64_t shares = 0, left = 0;
        for (const int64_t rows : count)
            for (int64_t done = 0; done < rows;) {
                if (shares == 0 || left < piece_rows + align) {
                    ++shares;
                    left = b;
                }
                int64_t take = left - piece_rows;
                if (take < rows - done) take = std::max<int64_t>(take - take % align, align);
                take = std::min(take, rows - done);
                left -= piece_rows + take;
                done += take;
            }
        CHECK(level_shares(count, b, piece_rows, align, INT64_MAX) == shares,
              "level_shares (b %lld, piece %lld, align %lld): %lld != %lld", (long long)b, (long long)piece_rows,
              (long long)align, (long long)level_shares(count, b, piece_rows, align, INT64_MAX), (long long)shares);
        if (shares > 0) {
            const int64_t limit = (int64_t)(rng() % (uint64_t)shares);
            CHECK(level_shares(count, b, piece_rows, align, limit) > limit, "early exit at %lld", (long long)limit);
        }
    }
}

static void check_part(const std::vector<int32_t>& offs, const char* what)
{
    const int n_nodes = (int)offs.size() - 1;
    std::vector<PartItem> items;
    std::vector<int32_t> first;
    part_chunks(offs, n_nodes, &items, &first);
    CHECK((int)first.size() == n_nodes + 1 && first[n_nodes] == (int32_t)items.size(), "%s: first", what);
    for (int i = 0; i < n_nodes; ++i) {
        int64_t at = offs[i];
        for (int32_t k = first[i]; k < first[i + 1]; ++k) {
            const PartItem& it = items[k];
            CHECK(it.node == i && it.node_begin == offs[i], "%s: chunk node", what);
            CHECK(it.begin == at && it.end > it.begin && (int64_t)it.end - it.begin <= kPartChunk, "%s: chunk %d", what, k);
            at = it.end;
        }
        CHECK(at == offs[i + 1], "%s: node %d chunks end at %lld of %d", what, i, (long long)at, offs[i + 1]);
    }
}

int main()
{
    // The five workloads' shapes and 2^31 - 1 rows: plans and tiles at P = 30, 19 and 12, with and
    // without the skipped slot.
    struct Shape { int64_t n; int F, S, w; } shapes[] = {
        {4096, 8, 256, 1}, {1000000, 100, 256, 1}, {10000000, 28, 256, 1}, {131072, 16384, 256, 1},
        {2000000, 50, 1025, 2}, {50000, 12, 257, 2}, {20000, 33000, 5, 2}, {1000, 3, 4096, 2},
        {INT32_MAX, 2, 256, 1}, {INT32_MAX, 1, 4096, 2}};
    for (const Shape& sh : shapes)
        for (int prec : {30, 19, 12})
            for (bool skip : {false, true})
                for (bool rm : {false, true}) {
                    if (rm && (int64_t)sh.F * sh.w > 65536) continue;
                    const PlanCtx c = ctx_of(sh.n, sh.F, sh.S, sh.w, prec, skip, rm);
                    FillPlan pr = plan_fill(&c, true, false);
                    check_plan(c, pr, true, false);
                    check_root(c, pr, "root");
                    FillPlan pl = plan_fill(&c, false, rm);
                    check_plan(c, pl, false, rm);
                    check_tiles(c, pl, feature_tiles(&c, pl, false), false);
                }
    // Random shapes.
    std::mt19937_64 rng(12345);
    for (int k = 0; k < 400; ++k) {
        const int w = 1 + (int)(rng() % 2);
        const int S = 2 + (int)(rng() % (w == 1 ? 255 : 4095));
        const int F = 1 + (int)(rng() % (rng() % 4 == 0 ? 40000 : 200));
        const int64_t n = 1 + (int64_t)(rng() % 3000000);
        const PlanCtx c = ctx_of(n, F, S, w, 1 + (int)(rng() % 30), rng() % 2, (int64_t)F * w <= 65536);
        FillPlan pr = plan_fill(&c, true, false);
        check_plan(c, pr, true, false);
        check_root(c, pr, "random root");
        FillPlan pl = plan_fill(&c, false, c.rm_stride > 0);
        check_plan(c, pl, false, c.rm_stride > 0);
        check_tiles(c, pl, feature_tiles(&c, pl, false), false);
    }

    // Level cuts on adversarial node lists, for a narrow and a wide matrix.
    for (int which = 0; which < 2; ++which) {
        const PlanCtx c = which == 0 ? ctx_of(10000000, 28, 256, 1, 30, false, true)
                                     : ctx_of(131072, 16384, 256, 1, 30, false, true);
        FillPlan p = plan_fill(&c, false, true);
        const auto tiles = feature_tiles(&c, p, false);
        auto run = [&](const std::vector<int64_t>& count, const std::vector<int32_t>& slots, const char* what) {
            std::vector<int64_t> begin(count.size());
            int64_t at = 0;
            std::vector<int64_t> cnt = count;
            for (size_t i = 0; i < count.size(); ++i) {
                begin[i] = at;
                at += count[i];
                if (slots[i] < 0) cnt[i] = 0;   // as build_level: a skipped node's rows are not read
            }
            check_level(c, p, tiles, begin, cnt, slots, what);
        };
        std::vector<int32_t> ident;
        auto slots_for = [&](size_t n) {
            ident.resize(n);
            for (size_t i = 0; i < n; ++i) ident[i] = (int32_t)i;
            return ident;
        };
        // 65,535 nodes: empty, one row, ragged (the narrow matrix: a wide
        // one's histograms of that many nodes would not fit the device)
        if (which == 0) {
            std::vector<int64_t> cnt(65535);
            for (size_t i = 0; i < cnt.size(); ++i) cnt[i] = i % 3 == 0 ? 0 : (int64_t)(rng() % 700);
            run(cnt, slots_for(cnt.size()), "65535 ragged nodes");
            for (auto& v : cnt) v = 1;
            run(cnt, slots_for(cnt.size()), "65535 one-row nodes");
            for (auto& v : cnt) v = 0;
            run(cnt, slots_for(cnt.size()), "65535 empty nodes");
        }
        // one giant node, alone and among small ones; level orders near 2^31
        run({INT32_MAX - 3}, slots_for(1), "one node of 2^31 - 4 rows");
        run({5, INT32_MAX - 200, 0, 190}, slots_for(4), "giant node among small ones, total 2^31 - 5");
        run({1, 2, 3}, slots_for(3), "tiny level");
        run({1 << 30, (1 << 30) - 1}, {-1, 1}, "skipped left child of 2^30 rows, built right one of 2^30 - 1");
        run({0}, slots_for(1), "one empty node");
        // skipped nodes (slot -1) and scattered output slots
        {
            std::vector<int64_t> cnt(600);
            std::vector<int32_t> sl(600);
            for (int i = 0; i < 600; ++i) {
                cnt[i] = (int64_t)(rng() % 50000);
                sl[i] = i % 2 ? -1 : (int32_t)(599 - i);
            }
            run(cnt, sl, "every other node skipped, slots reversed");
        }
        // Dirichlet-like sizes: a few huge, many tiny
        {
            std::vector<int64_t> cnt(128);
            for (int i = 0; i < 128; ++i) cnt[i] = i < 4 ? 2000000 : (int64_t)(rng() % 1000);
            run(cnt, slots_for(cnt.size()), "four huge nodes and 124 small ones");
        }
        for (int k = 0; k < 60; ++k) {
            const int nn = 1 + (int)(rng() % 300);
            std::vector<int64_t> cnt(nn);
            for (auto& v : cnt) v = (int64_t)(rng() % (rng() % 2 ? 100 : 400000));
            run(cnt, slots_for(cnt.size()), "random level");
        }
    }
    check_level_shares(rng);
    // Partition chunks, including nodes that end at 2^31 - 1.
    check_part({0, 1, 8192, 8193, 20000}, "small");
    check_part({0, INT32_MAX - 5000, INT32_MAX - 1, INT32_MAX}, "ending at 2^31 - 1");
    check_part({0, INT32_MAX}, "one node of 2^31 - 1");
    check_part({0, 0, 0}, "empty nodes");
    std::printf("plan_test: %d checks passed\n", g_checks);
    return 0;
}
