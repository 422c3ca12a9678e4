// Shapes and launch-plan records shared by the host planner (hgb_plan.h) and
// the device kernels (hgb_kernels.h).  Plain C++: no HIP types or attributes
// (the constexpr helpers are usable on both sides), so the planner can be
// compiled and tested on the host alone.
#pragma once

#include <stdint.h>

namespace hgb {

constexpr int kWave = 64;

// Accumulation modes of the fills.
//   kWide    two u64 LDS adds per cell, one per component (gradient and
//            hessian planes).  Exact for any fixed-point precision.
//   kPacked  one u64 LDS add per cell of qh * 2^32 + qg.  Each copy-slot sums
//            at most kPackedRowsPerCopy rows of |q| <= 2^19 between drains
//            into an int64 accumulator, so the low half never leaves the
//            int32 range and both sums decode exactly: G = sign-extended low
//            32 bits, H = (V - G) / 2^32.
enum { kWide = 0, kPacked = 1 };
constexpr int kPackedMaxBits = 19;
constexpr int kPackedRowsPerCopy = 4095;

// Row-major level fills with the interleaved tile and 32-byte row chunks may
// give each row to two lanes, each loading one half of the chunk (il = 2 in
// the plan; il = 1 is one lane per row).
constexpr int kPairHalfBytes = 16;

// LDS words after a fill's tile: the item's row totals, then (g, h) per
// feature of the tile (<= 32): the skipped slot's recovered cells.
constexpr int kFixWords = 2 + 2 * 32;

// LDS words of a feature-major tile of nf features and 2^lc copies: the
// copies, plus the packed accumulator.
constexpr int tile_words(int acc_mode, int nf, int S, int lc)
{
    return acc_mode == kWide ? nf * 2 * (S << lc) : nf * (S << lc) + nf * S * 2;
}

// LDS words of the interleaved root tile of tf positions before its fixed
// words: the copies, and for packed sums at least the one-copy wide layout
// the finish reads.
constexpr int root_il_words(int acc_mode, int tf, int S, int lc)
{
    return acc_mode == kWide ? 2 * S * (tf << lc) : (S * (tf << lc) > 2 * S * tf ? S * (tf << lc) : 2 * S * tf);
}

// Rows per thread and step of the root fills (consecutive rows, one load per
// feature), and register cells per thread of the packed interleaved root
// (1024 threads hold the 16 positions of up to 256 slots).
constexpr int kRootRows = 4;
constexpr int kRootIlPackedCells = 4;

// Entries per thread and step of the feature-major level fill with nf
// features (fewer for wide tiles, so the step's bins stay in registers).
constexpr int kLevelEntries = 8;
constexpr int cols_entries(int nf) { return nf >= 8 ? 4 : kLevelEntries; }

// One unit of fill work: rows [row_begin, row_end) of the level order, features
// [f0, f0 + nf), accumulated for one node.  `dest` says where the sums go:
// stored into slot out_slot of the level buffer (kDestStore), stored into
// slot out_slot of the partial buffer (kDestPartial: a node split over several
// items, merged afterwards), or added there with int64 atomics (kDestAtomic).
enum { kDestStore = 0, kDestPartial = 1, kDestAtomic = 2 };
struct FillItem {
    int32_t out_slot;
    int32_t row_begin;
    int32_t row_end;
    int32_t f0_nf;       // f0 | (nf << 16)
    int32_t dest;
    int32_t pad[3];
};

// Merge of a node split over several items: the sum of `count` partial slots
// from `first` on, stored into (or, for a node merged in several groups,
// added with atomics to) slot out_slot of the level buffer.
struct MergeEntry {
    int32_t out_slot;
    int32_t first;
    int32_t count;
    int32_t atomic;
};
// A merge list this short travels in the kernel's arguments.
constexpr int kMergeInline = 128;

// A subtraction plan of this many pairs travels in the kernel's arguments.
constexpr int kSubtractInlinePairs = 256;

// Split scan for features with more than 64 * 4 bins: waves per feature.
constexpr int kSliceWaves = 4;
// Largest block of the per-node split reduction.
constexpr int kSplitReduceMaxThreads = 1024;

// partition_level: fixed-size chunks of each node's rows, one block each.
// 512 threads of 8 positions: against 1,024 x 8, 1,024 x 16, 512 x 16,
// 512 x 12, 512 x 4, 384 x 8, 256 x 8, 256 x 16 and 256 x 32 the fastest
// count + scatter on a grown 10M x 28 tree (smaller chunks cost the scan more
// chunks than they save)
constexpr int kPartThreads = 512;   // threads of a count or scatter block
constexpr int kPartChunk = 4096;
// Largest level whose scan runs in LDS (k_part_scan_lds): chunks and nodes.
constexpr int kPartScanLdsItems = 8192;
constexpr int kPartScanLdsNodes = 4096;
struct PartItem {
    int32_t node;
    int32_t begin, end;   // positions [begin, end) of the node's rows
    int32_t node_begin;   // the node's first position
};

}  // namespace hgb
