/*
 * Serial CPU oracle for the level histogram build of histogram GBDT training.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke entry
 * point and the benchmark's CPU-baseline leg may load this library.  It shares
 * no code, header, table or constant with the HIP library; the two are meant
 * to be compared against each other.
 *
 * Everything here is a plain, slow, obviously correct restatement of what the
 * method computes, written in the order the pages describe it:
 *
 *   quantize      per-tree fixed-point encoding of (grad, hess) into integers
 *                 (the pages fix "int64 fixed point" cells but not the scale;
 *                 the scale rule below is this project's reading).
 *   build_hist    per node and feature, the (g, h) sums of the node's rows,
 *                 grouped by the slot each row's bin names.
 *   subtract      larger sibling = parent - smaller sibling, bin by bin.
 *   find_splits   scan each feature's bins with the XGBoost-style gain and pick
 *                 the best (feature, bin, default direction) per node.
 *   find_level_split  the oblivious variant: one (feature, bin, direction)
 *                 for all nodes of a level, by the gain summed over nodes.
 *   partition     route a node's rows to its two children by the chosen split
 *                 (used only to drive a multi-level tree in the tests).
 *   objective     per-row (grad, hess) of squared-error, logistic or Poisson
 *                 loss from scores and labels, with an exp written out in
 *                 full (Cody-Waite reduction, Taylor polynomial).
 *
 * Compiled with gcc -O2 -ffp-contract=off so that the fp64 gain expression is
 * evaluated exactly as written, one rounding per operation.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Quantization                                                              */
/* ------------------------------------------------------------------------ */

/*
 * Fixed-point encoding of one per-row component (gradient or hessian).
 *
 * Basis: bonsai "9. Parallelism & determinism", section "The idea": device
 * histogram cells are int64 fixed point, so a sum of cells is one integer in
 * any order.  The pages do not give the scale.  Reading used here:
 *
 *   M = max_i |c_i|.  If M == 0 then k = 0, else with 2^(e-1) <= M < 2^e
 *   (the frexp exponent e) k = P - e for a precision of P bits (1..30).
 *   q_i = rint(c_i * 2^k), rounding half to even.  c_i * 2^k is exact in
 *   double, and |q_i| <= 2^P <= 2^30, so q fits int32 and a sum over fewer
 *   than 2^32 rows fits int64.  P = 30 is the default; a smaller P is the
 *   narrower fixed point that the ybb.press article, section 7, packs two to
 *   a 64-bit word.
 *
 * Non-finite values are rejected; for the hessian (require_nonneg = 1) so are
 * negative values.  -0.0 counts as zero.
 */
int oracle_quantize(const float* c, int64_t n, int require_nonneg, int32_t bits,
                    int32_t* q_out, int32_t* k_out)
{
    if (bits < 1 || bits > 30) return ORACLE_E_INVALID;
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double x = (double)c[i];
        if (!isfinite(x)) return ORACLE_E_NONFINITE;
        if (require_nonneg && x < 0.0) return ORACLE_E_NONFINITE;
        double a = fabs(x);
        if (a > m) m = a;
    }
    int32_t k = 0;
    if (m != 0.0) {
        int e = 0;
        (void)frexp(m, &e);      /* m = f * 2^e with 0.5 <= f < 1 */
        k = bits - e;
    }
    for (int64_t i = 0; i < n; ++i) {
        double scaled = ldexp((double)c[i], k);   /* exact */
        q_out[i] = (int32_t)rint(scaled);         /* round half to even */
    }
    *k_out = k;
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Histogram fill                                                            */
/* ------------------------------------------------------------------------ */

static int64_t slot_of(const void* bins, int bin_bytes, int64_t idx)
{
    if (bin_bytes == 1) return (int64_t)((const uint8_t*)bins)[idx];
    return (int64_t)((const uint16_t*)bins)[idx];
}

/*
 * Check that every stored bin value is a valid slot: a value bin in
 * [0, n_bins), or, when the matrix has missing entries, the sentinel n_bins.
 */
int oracle_check_bins(const void* bins, int bin_bytes, int64_t n_rows,
                      int32_t n_features, int32_t n_bins, int32_t has_missing)
{
    int64_t limit = (int64_t)n_bins + (has_missing ? 1 : 0);
    int64_t total = n_rows * (int64_t)n_features;
    for (int64_t i = 0; i < total; ++i)
        if (slot_of(bins, bin_bytes, i) >= limit) return ORACLE_E_INVALID;
    return ORACLE_OK;
}

/*
 * Histogram of every node on a level.
 *
 * Basis: bonsai "E6. The wide-data wall", section "Two fills, one choice":
 * each row of a node contributes its (qg, qh) to the slot its bin names, in
 * each feature's histogram.  The cells are int64 (bonsai "9. Parallelism &
 * determinism", "The idea"), so the sum is exact and order-free.  This loop
 * walks node -> feature -> the node's rows, i.e. the feature-parallel fill of
 * the same page, run on one thread.
 *
 * bins:          feature-major [n_features][n_rows], u8 or u16 values.  A value
 *                b < n_bins goes to slot b; the sentinel n_bins (only with
 *                has_missing) goes to slot n_bins.
 * qg, qh:        quantized gradient / hessian per row.
 * row_index:     concatenated row lists of the nodes, node i owning entries
 *                [node_offsets[i], node_offsets[i+1]).  NULL means one node
 *                holding every row 0..n_rows-1 in order (the root).
 * hist:          [n_nodes][n_features][S][2] int64, S = n_bins + has_missing,
 *                component 0 = gradient, 1 = hessian.  Overwritten in full.
 */
void oracle_build_hist(const void* bins, int bin_bytes, int64_t n_rows,
                       int32_t n_features, int32_t n_bins, int32_t has_missing,
                       const int32_t* qg, const int32_t* qh,
                       const int32_t* row_index, const int64_t* node_offsets,
                       int32_t n_nodes, int64_t* hist)
{
    const int64_t S = (int64_t)n_bins + (has_missing ? 1 : 0);
    const int64_t node_elems = (int64_t)n_features * S * 2;
    memset(hist, 0, sizeof(int64_t) * (size_t)(node_elems * n_nodes));
    for (int32_t node = 0; node < n_nodes; ++node) {
        int64_t begin = row_index ? node_offsets[node] : 0;
        int64_t end = row_index ? node_offsets[node + 1] : n_rows;
        int64_t* h_node = hist + node * node_elems;
        for (int32_t f = 0; f < n_features; ++f) {
            const int64_t col = (int64_t)f * n_rows;
            int64_t* h_feat = h_node + (int64_t)f * S * 2;
            for (int64_t k = begin; k < end; ++k) {
                int64_t r = row_index ? (int64_t)row_index[k] : k;
                int64_t s = slot_of(bins, bin_bytes, col + r);
                h_feat[2 * s + 0] += (int64_t)qg[r];
                h_feat[2 * s + 1] += (int64_t)qh[r];
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Sibling subtraction                                                       */
/* ------------------------------------------------------------------------ */

/*
 * Basis: ybb.press GBDT engine article, section 三 (histogram subtraction):
 * hist(parent) = hist(left) + hist(right), so the sibling that was not built
 * is the parent minus the one that was, bin by bin.  Integer cells make this
 * exact, so the article's clamp of negative hessian sums is never needed.
 *
 * parent: [n_pairs][node_elems];  child: [2*n_pairs][node_elems].  For pair i
 * the built child sits at 2i + built_is_right[i]; the other child is written.
 */
void oracle_subtract(const int64_t* parent, int64_t* child,
                     const uint8_t* built_is_right, int32_t n_pairs,
                     int64_t node_elems)
{
    for (int32_t i = 0; i < n_pairs; ++i) {
        int r = built_is_right[i] ? 1 : 0;
        const int64_t* p = parent + (int64_t)i * node_elems;
        const int64_t* built = child + (int64_t)(2 * i + r) * node_elems;
        int64_t* other = child + (int64_t)(2 * i + 1 - r) * node_elems;
        for (int64_t e = 0; e < node_elems; ++e) other[e] = p[e] - built[e];
    }
}

/* ------------------------------------------------------------------------ */
/* Split scan                                                                */
/* ------------------------------------------------------------------------ */

/*
 * Gain of one candidate, the XGBoost-style score of the ybb.press article,
 * section 一, without the leading factor 1/2 (a positive constant factor does
 * not move the argmax):
 *
 *   gl^2/(hl+lambda) + gr^2/(hr+lambda) - g^2/(h+lambda) - gamma
 *
 * evaluated left to right in fp64 with no fused multiply-add.
 */
static double gain_of(double gl, double hl, double gr, double hr,
                      double g, double h, double lambda, double gamma)
{
    double left = gl * gl / (hl + lambda);
    double right = gr * gr / (hr + lambda);
    double parent = g * g / (h + lambda);
    return left + right - parent - gamma;
}

/*
 * Best split of every node.
 *
 * For each feature: totals (G, H) are the sum over all of the feature's slots.
 * Candidates are (b, d) for value bin b in [0, n_bins) and default direction
 * d: "right" only, or "right" then "left" when the matrix has missing values
 * (ybb.press article, section 四: try the missing rows on the left and on the
 * right and keep the better).  The left side holds the value bins <= b, plus
 * the missing slot when d is "left"; the right side is the rest.  A candidate
 * is valid when both sides have a positive integer hessian sum.
 *
 * Integer sums are turned into reals as (double)G * 2^-k (round-to-nearest
 * conversion, then an exact power-of-two scaling).
 *
 * Ties: candidates are visited in (feature, bin, direction right-then-left)
 * order and replaced only on a strictly larger gain, so among equal gains the
 * smallest feature, then bin, then "right" wins -- the serial order that
 * bonsai "9. Parallelism & determinism", section "In bonsai", keeps when it
 * merges per-feature winners in feature order.
 *
 * A node with no valid candidate reports feature = bin = -1 and gain -inf.
 * The reported totals are feature 0's slot sums (equal for every feature of a
 * consistent histogram).
 */
void oracle_find_splits(const int64_t* hist, int32_t n_nodes,
                        int32_t n_features, int32_t n_bins, int32_t has_missing,
                        int32_t k_g, int32_t k_h, double lambda, double gamma,
                        oracle_split* out)
{
    const int64_t S = (int64_t)n_bins + (has_missing ? 1 : 0);
    const int64_t node_elems = (int64_t)n_features * S * 2;
    for (int32_t node = 0; node < n_nodes; ++node) {
        const int64_t* h_node = hist + node * node_elems;
        oracle_split best;
        best.feature = -1;
        best.bin = -1;
        best.default_left = 0;
        best.pad = 0;
        best.gain = -INFINITY;
        best.g_left = 0;
        best.h_left = 0;
        best.g_total = 0;
        best.h_total = 0;
        for (int64_t s = 0; s < S; ++s) {
            best.g_total += h_node[2 * s + 0];
            best.h_total += h_node[2 * s + 1];
        }
        for (int32_t f = 0; f < n_features; ++f) {
            const int64_t* h_feat = h_node + (int64_t)f * S * 2;
            int64_t G = 0, H = 0;
            for (int64_t s = 0; s < S; ++s) {
                G += h_feat[2 * s + 0];
                H += h_feat[2 * s + 1];
            }
            int64_t G_miss = has_missing ? h_feat[2 * n_bins + 0] : 0;
            int64_t H_miss = has_missing ? h_feat[2 * n_bins + 1] : 0;
            double g = ldexp((double)G, -k_g);
            double h = ldexp((double)H, -k_h);
            int64_t G_prefix = 0, H_prefix = 0;
            for (int32_t b = 0; b < n_bins; ++b) {
                G_prefix += h_feat[2 * b + 0];
                H_prefix += h_feat[2 * b + 1];
                int n_dirs = has_missing ? 2 : 1;
                for (int d = 0; d < n_dirs; ++d) {   /* d = 0: right, 1: left */
                    int64_t GL = G_prefix + (d ? G_miss : 0);
                    int64_t HL = H_prefix + (d ? H_miss : 0);
                    int64_t GR = G - GL;
                    int64_t HR = H - HL;
                    if (!(HL > 0 && HR > 0)) continue;
                    double gain = gain_of(ldexp((double)GL, -k_g),
                                          ldexp((double)HL, -k_h),
                                          ldexp((double)GR, -k_g),
                                          ldexp((double)HR, -k_h),
                                          g, h, lambda, gamma);
                    if (gain > best.gain) {
                        best.feature = f;
                        best.bin = b;
                        best.default_left = d;
                        best.gain = gain;
                        best.g_left = GL;
                        best.h_left = HL;
                    }
                }
            }
        }
        out[node] = best;
    }
}

/* ------------------------------------------------------------------------ */
/* Row partition (drives multi-level trees in the tests)                     */
/* ------------------------------------------------------------------------ */

/*
 * Route every node's rows to its children by the node's split: a row goes
 * left when its bin for the split feature is a value bin <= split bin, or is
 * the missing sentinel and the default direction is left.  The order of rows
 * is kept within each child (a stable partition, as the device partition of
 * bonsai "10: CUDA histogram backend", section "The device context lifecycle",
 * keeps it).  Nodes without a valid split get no children.  The children of
 * the j-th split node (counting split nodes only) are 2j (left) and 2j+1
 * (right).
 *
 * out_row_index must hold node_offsets[n_nodes] entries; out_offsets must hold
 * 2 * n_nodes + 1 entries.  Returns the number of children written.
 */
int32_t oracle_partition(const void* bins, int bin_bytes, int64_t n_rows,
                         int32_t n_bins, const int32_t* row_index,
                         const int64_t* node_offsets, int32_t n_nodes,
                         const oracle_split* splits,
                         int32_t* out_row_index, int64_t* out_offsets)
{
    int32_t n_children = 0;
    int64_t pos = 0;
    out_offsets[0] = 0;
    for (int32_t node = 0; node < n_nodes; ++node) {
        if (splits[node].feature < 0) continue;
        int64_t begin = row_index ? node_offsets[node] : 0;
        int64_t end = row_index ? node_offsets[node + 1] : n_rows;
        const int64_t col = (int64_t)splits[node].feature * n_rows;
        for (int side = 0; side < 2; ++side) {        /* 0 = left, 1 = right */
            for (int64_t k = begin; k < end; ++k) {
                int64_t r = row_index ? (int64_t)row_index[k] : k;
                int64_t v = slot_of(bins, bin_bytes, col + r);
                int goes_left = (v == n_bins) ? (splits[node].default_left != 0)
                                              : (v <= splits[node].bin);
                if (goes_left == (side == 0)) out_row_index[pos++] = (int32_t)r;
            }
            out_offsets[++n_children] = pos;
        }
    }
    return n_children;
}

/*
 * One split for a whole level: the oblivious (symmetric) tree, in which every
 * node of a level uses the same feature and threshold.
 *
 * Basis: bonsai "10: CUDA histogram backend", section "The device context
 * lifecycle" (the oblivious grower scans the frontier's histograms with
 * find_level_split, the depthwise one with find_splits_many); ybb.press
 * article, section 五 (symmetric trees: one feature and one threshold per
 * level).  The pages give no formula; reading used here:
 *
 *   A candidate is (f, b, d) as in oracle_find_splits, the same for all nodes.
 *   In each node it splits the node's rows as a depthwise split would, with
 *   the node's own totals of feature f.  Its level score is the sum, over the
 *   nodes where it is valid (both sides with a positive hessian sum), of that
 *   node's gain (the oracle_find_splits gain, gamma included), added in node
 *   order starting from 0.0; a node where it is not valid adds nothing.  A
 *   candidate valid in no node is not a candidate.  The level split is the
 *   candidate with the largest score; ties go to the smallest f, then b, then
 *   right before left (the serial scan order, as for a node).
 *
 * out holds n_nodes + 1 records.  out[i] (i < n_nodes): the level's feature,
 * bin and direction; gain = node i's term of the score (0.0 where the split is
 * not valid in it); g_left, h_left = node i's left sums under the split;
 * g_total, h_total = node i's totals (feature 0's slot sums).  out[n_nodes]:
 * the level's feature, bin and direction, gain = the score, and the sums of
 * the four integer fields over the nodes.  With no candidate at all every
 * record has feature = bin = -1, default_left = 0, gain = -inf, g_left =
 * h_left = 0, and its totals.
 */
void oracle_find_level_split(const int64_t* hist, int32_t n_nodes,
                             int32_t n_features, int32_t n_bins, int32_t has_missing,
                             int32_t k_g, int32_t k_h, double lambda, double gamma,
                             oracle_split* out)
{
    const int64_t S = (int64_t)n_bins + (has_missing ? 1 : 0);
    const int64_t node_elems = (int64_t)n_features * S * 2;
    const int n_dirs = has_missing ? 2 : 1;
    /* per node, for the feature being scanned: inclusive prefix sums of the
     * value slots, the missing slot and the totals */
    int64_t* pre = (int64_t*)malloc(sizeof(int64_t) * 2 * (size_t)(n_nodes > 0 ? n_nodes : 1)
                                    * (size_t)(n_bins + 2));
    int found = 0;
    int32_t best_f = -1, best_b = -1, best_d = 0;
    double best_score = -INFINITY;
    for (int32_t f = 0; f < n_features && n_nodes > 0; ++f) {
        for (int32_t node = 0; node < n_nodes; ++node) {
            const int64_t* h_feat = hist + node * node_elems + (int64_t)f * S * 2;
            int64_t* p = pre + (int64_t)node * 2 * (n_bins + 2);
            int64_t G = 0, H = 0;
            for (int32_t b = 0; b < n_bins; ++b) {
                G += h_feat[2 * b + 0];
                H += h_feat[2 * b + 1];
                p[2 * b + 0] = G;
                p[2 * b + 1] = H;
            }
            p[2 * n_bins + 0] = has_missing ? h_feat[2 * n_bins + 0] : 0;   /* missing slot */
            p[2 * n_bins + 1] = has_missing ? h_feat[2 * n_bins + 1] : 0;
            p[2 * n_bins + 2] = G + p[2 * n_bins + 0];                       /* totals */
            p[2 * n_bins + 3] = H + p[2 * n_bins + 1];
        }
        for (int32_t b = 0; b < n_bins; ++b) {
            for (int d = 0; d < n_dirs; ++d) {   /* d = 0: right, 1: left */
                double score = 0.0;
                int valid_somewhere = 0;
                for (int32_t node = 0; node < n_nodes; ++node) {
                    const int64_t* p = pre + (int64_t)node * 2 * (n_bins + 2);
                    const int64_t G = p[2 * n_bins + 2], H = p[2 * n_bins + 3];
                    const int64_t GL = p[2 * b + 0] + (d ? p[2 * n_bins + 0] : 0);
                    const int64_t HL = p[2 * b + 1] + (d ? p[2 * n_bins + 1] : 0);
                    const int64_t GR = G - GL;
                    const int64_t HR = H - HL;
                    if (!(HL > 0 && HR > 0)) continue;
                    score += gain_of(ldexp((double)GL, -k_g), ldexp((double)HL, -k_h),
                                     ldexp((double)GR, -k_g), ldexp((double)HR, -k_h),
                                     ldexp((double)G, -k_g), ldexp((double)H, -k_h),
                                     lambda, gamma);
                    valid_somewhere = 1;
                }
                if (valid_somewhere && (!found || score > best_score)) {
                    found = 1;
                    best_f = f;
                    best_b = b;
                    best_d = d;
                    best_score = score;
                }
            }
        }
    }
    free(pre);

    oracle_split level;
    memset(&level, 0, sizeof level);
    level.feature = found ? best_f : -1;
    level.bin = found ? best_b : -1;
    level.default_left = found ? best_d : 0;
    level.gain = found ? best_score : -INFINITY;
    for (int32_t node = 0; node < n_nodes; ++node) {
        const int64_t* h_node = hist + node * node_elems;
        oracle_split r;
        memset(&r, 0, sizeof r);
        for (int64_t s = 0; s < S; ++s) {   /* totals: feature 0's slots */
            r.g_total += h_node[2 * s + 0];
            r.h_total += h_node[2 * s + 1];
        }
        r.feature = level.feature;
        r.bin = level.bin;
        r.default_left = level.default_left;
        r.gain = found ? 0.0 : -INFINITY;
        if (found) {
            const int64_t* h_feat = h_node + (int64_t)best_f * S * 2;
            int64_t G = 0, H = 0, GL = 0, HL = 0;
            for (int64_t s = 0; s < S; ++s) {
                G += h_feat[2 * s + 0];
                H += h_feat[2 * s + 1];
            }
            for (int32_t b = 0; b <= best_b; ++b) {
                GL += h_feat[2 * b + 0];
                HL += h_feat[2 * b + 1];
            }
            if (best_d) {
                GL += h_feat[2 * n_bins + 0];
                HL += h_feat[2 * n_bins + 1];
            }
            r.g_left = GL;
            r.h_left = HL;
            if (HL > 0 && H - HL > 0)
                r.gain = gain_of(ldexp((double)GL, -k_g), ldexp((double)HL, -k_h),
                                 ldexp((double)(G - GL), -k_g), ldexp((double)(H - HL), -k_h),
                                 ldexp((double)G, -k_g), ldexp((double)H, -k_h), lambda, gamma);
        }
        level.g_left += r.g_left;
        level.h_left += r.h_left;
        level.g_total += r.g_total;
        level.h_total += r.h_total;
        out[node] = r;
    }
    out[n_nodes] = level;
}

/* ------------------------------------------------------------------------ */
/* Objective gradients                                                       */
/* ------------------------------------------------------------------------ */

/*
 * exp(x) in double, written out so that any implementation that performs the
 * same IEEE operations in the same order gets the same bits (a libm's exp is
 * free to differ in the last place from one library to the next).
 *
 * Method: Cody and Waite's argument reduction ("Software Manual for the
 * Elementary Functions", 1980).  x = n ln2 + r with n = rint(x / ln2) and
 * |r| <= ln2 / 2, where ln 2 is split into a head with 36 significant bits
 * (so n * head is exact for |n| < 2^17) and the double nearest to the rest;
 * r = (x - n * head) - n * tail.  exp(r) is the Taylor polynomial of degree 13,
 * sum r^j / j!, in Horner form (the first dropped term is below 5e-18 for
 * |r| <= 0.347); the result is that polynomial scaled by 2^n (ldexp, exact
 * except where the result is subnormal, where it rounds once).
 * Beyond |x| > 1000 the result is +Inf or 0; NaN propagates.
 */
static double oracle_exp(double x)
{
    if (x != x) return x;
    if (x > 1000.0) return INFINITY;
    if (x < -1000.0) return 0.0;
    const double inv_ln2 = 1.4426950408889634;            /* 1 / ln 2, rounded */
    const double ln2_head = 0x1.62e42fefa0000p-1;          /* 36 leading bits of ln 2 */
    const double ln2_tail = 0x1.cf79abc9e3b3ap-40;         /* ln 2 - head, rounded */
    const double n = rint(x * inv_ln2);
    const double r = (x - n * ln2_head) - n * ln2_tail;
    /* 1/j! for j = 13 down to 0; each j! is exact in double */
    const double inv_fact[14] = {
        1.0 / 6227020800.0, 1.0 / 479001600.0, 1.0 / 39916800.0, 1.0 / 3628800.0,
        1.0 / 362880.0, 1.0 / 40320.0, 1.0 / 5040.0, 1.0 / 720.0, 1.0 / 120.0,
        1.0 / 24.0, 1.0 / 6.0, 1.0 / 2.0, 1.0, 1.0};
    double p = inv_fact[0];
    for (int j = 1; j < 14; ++j) p = p * r + inv_fact[j];
    return ldexp(p, (int)n);
}

void oracle_exp_array(const double* x, int64_t n, double* out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_exp(x[i]);
}

/*
 * Per-row gradient and hessian of a twice-differentiable loss at the current
 * raw score (margin) m of each row, for label y and optional weight w (NULL
 * means every weight is 1).
 *
 * Basis: bonsai "10: CUDA histogram backend", section "The device context
 * lifecycle": with a device-resident objective (squared error, logistic or
 * Poisson, weighted or not) begin_tree derives the (grad, hess) pairs on the device from the
 * resident scores and labels.  The pages name the losses but not their
 * derivatives; the ones below are the first and second derivatives in m of
 *
 *   squared error  (m - y)^2 / 2          g = m - y,         h = 1
 *   logistic       log(1 + e^m) - y m     g = p - y,         h = p (1 - p),
 *                                         with p = 1 / (1 + e^-m)
 *   Poisson        e^m - y m              g = e^m - y,       h = e^m
 *
 * each multiplied by the row's weight.  Every quantity is computed in double,
 * one rounding per operation in the order written (no fused multiply-add),
 * with oracle_exp above, and the pair is rounded once to fp32, the type that
 * begin_tree takes.  Nothing is validated here: a non-finite or negative
 * result is reported by quantization, as for gradients handed in directly.
 * Returns ORACLE_E_INVALID for an unknown objective.
 */
int oracle_objective(int32_t objective, const float* margin, const float* label,
                     const float* weight, int64_t n, float* grad, float* hess)
{
    if (objective < ORACLE_OBJ_SQUARED || objective > ORACLE_OBJ_POISSON) return ORACLE_E_INVALID;
    for (int64_t i = 0; i < n; ++i) {
        const double m = (double)margin[i];
        const double y = (double)label[i];
        const double w = weight ? (double)weight[i] : 1.0;
        double g, h;
        if (objective == ORACLE_OBJ_SQUARED) {
            g = m - y;
            h = 1.0;
        } else if (objective == ORACLE_OBJ_LOGISTIC) {
            const double p = 1.0 / (1.0 + oracle_exp(-m));
            g = p - y;
            h = p * (1.0 - p);
        } else {
            const double e = oracle_exp(m);
            g = e - y;
            h = e;
        }
        grad[i] = (float)(g * w);
        hess[i] = (float)(h * w);
    }
    return ORACLE_OK;
}
