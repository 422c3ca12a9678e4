/*
 * hgb -- level histogram build for histogram gradient-boosted trees, MI355X
 * (gfx950) native.  C ABI over hand-written HIP kernels.
 *
 * The operation, per tree level: each node built from rows gets, per feature,
 * the (gradient, hessian) sums of its rows grouped by the rows' bins; each
 * larger sibling is derived as parent minus the smaller one; scan
 * every feature's bins with the XGBoost-style gain and pick each node's split.
 *
 * Sources (the pages this library restates):
 *   [bonsai-10]  bonsai docs, "10: CUDA histogram backend"
 *   [bonsai-9]   bonsai guide, "9. Parallelism & determinism"
 *   [bonsai-E6]  bonsai engine notes, "E6. The wide-data wall"
 *   [ybb]        ybb.press article on GBDT engine engineering (sections 一 to 九,
 *                cited as 1 to 9)
 *
 * Conventions shared by every entry point:
 *   - n = rows, F = features, B = value bins per feature, S = B + has_missing
 *     histogram slots per feature.  A histogram slot is 16 bytes: int64 gradient
 *     sum then int64 hessian sum.  A node's histogram is [F][S][2] int64, and a
 *     level buffer is [node slots][F][S][2] int64, row-major.
 *   - Pointers named *_dev are device pointers on the context's device; *_host
 *     are host pointers that are read before the call returns.  The caller owns
 *     every argument buffer; the context owns its resident copies and scratch.
 *   - Work is enqueued asynchronously on the context's stream.  Arguments are
 *     validated synchronously; a rejected call enqueues nothing and returns a
 *     status, with a message from hgb_last_error().  A call that passed
 *     validation does not fail at launch time.  Conditions that can only be seen
 *     on the device (a row index out of range) are skipped by the kernels and
 *     reported by the next hgb_sync().
 *   - A context is not thread safe; use one per host thread.
 */
#ifndef HGB_H
#define HGB_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct hgb_ctx hgb_ctx;

typedef enum {
    HGB_OK = 0,
    HGB_E_INVALID = 1,      /* bad argument, size, offset or bin value */
    HGB_E_STATE = 2,        /* call out of order (e.g. build before begin_tree) */
    HGB_E_UNSUPPORTED = 3,  /* shape beyond the kernels' plan (too many bins) */
    HGB_E_NONFINITE = 4,    /* NaN/Inf gradient or hessian, or a negative hessian */
    HGB_E_DEVICE = 5        /* HIP runtime error, or no usable device */
} hgb_status;

/* One node's best split.  56 bytes, naturally aligned. */
typedef struct {
    int32_t feature;       /* -1 when no candidate is valid */
    int32_t bin;           /* value bins <= bin go left; -1 when none */
    int32_t default_left;  /* 1: rows in the missing slot go left */
    int32_t pad;           /* always 0 */
    double gain;           /* -inf when no candidate is valid */
    int64_t g_left;        /* fixed-point gradient sum of the left side */
    int64_t h_left;        /* fixed-point hessian sum of the left side */
    int64_t g_total;       /* node totals (feature 0's slot sums) */
    int64_t h_total;
} hgb_split;

/* Largest S = n_bins + has_missing the kernels accept. */
#define HGB_MAX_SLOTS 4096

/* 1 when a HIP device is present and usable, else 0 ([bonsai-10] "Always
 * registered, capability at runtime": the library always loads, and whether it
 * can run is a runtime question; its tests skip where there is no device).
 * Counts devices only; touches no device state. */
int hgb_available(void);

/* Create a context on `device`, enqueueing on `hip_stream` (a hipStream_t;
 * NULL selects the device's null stream).  *out receives the context
 * ([bonsai-10] "The device context lifecycle": one device context owns the
 * resident state of a fit, split by lifetime into the dataset, the per-tree
 * gradients and the per-level buffers).  The caller owns the stream.
 * Memory: a context allocates at creation 4 MiB of pinned host memory and 4
 * MiB of device memory for its launch plans (16 stages of 256 KiB, grown when a
 * plan needs more), and a few small coherent pinned buffers through which
 * kernels post results to the host.
 * Errors: HGB_E_INVALID for a null `out` or a device index out of range;
 *         HGB_E_DEVICE when no device is usable or an allocation fails. */
hgb_status hgb_create(int device, void* hip_stream, hgb_ctx** out);

/* Release the context and everything it owns ([bonsai-10] "The device
 * context lifecycle").  Synchronizes its stream first.  NULL is a no-op. */
void hgb_destroy(hgb_ctx* ctx);

/* Message describing the last failed call on this context ("" if none;
 * "null context" for NULL).  Valid until the next call on the context
 * ([bonsai-10] "The kernel": a shape the device path cannot take is declined
 * up front, with a reason, so the caller can fall back; a call that passed
 * its checks does not fail later). */
const char* hgb_last_error(const hgb_ctx* ctx);

/* Block until the context's stream has drained ([bonsai-10] "The device
 * context lifecycle": the host reads results once the level's work is done).
 * Returns HGB_E_NONFINITE if a tree started asynchronously since the previous
 * hgb_sync had a non-finite value (hgb_set_async_begin), else HGB_E_INVALID
 * if a kernel met a row index outside [0, n) since the previous hgb_sync
 * (those entries were skipped), HGB_E_DEVICE on a runtime error, else HGB_OK. */
hgb_status hgb_sync(hgb_ctx* ctx);

/*
 * Make the binned matrix resident ([bonsai-10] "The device context
 * lifecycle": the feature-major binned matrix is uploaded once per dataset;
 * u8 when every feature fits 256 bins, u16 otherwise).
 *
 * bins:        feature-major [n_features][n_rows], element size bin_bytes
 *              (1 = uint8, 2 = uint16); host memory if on_device == 0, device
 *              memory on the context's device otherwise.  Copied; the caller
 *              keeps ownership.
 * n_bins:      value bins per feature (B).  A stored value b < B is value bin b.
 * has_missing: when nonzero the value B is the missing sentinel, counted in
 *              histogram slot B (S = B + 1).  Otherwise S = B.
 * Errors: HGB_E_INVALID for non-positive sizes, bin_bytes not 1/2, B too large
 *         for the element type, or any stored value >= S (checked on the
 *         device, synchronously); HGB_E_UNSUPPORTED when S > HGB_MAX_SLOTS.
 * Device memory: the context keeps the feature-major copy and, when a row
 * takes at most 64 KiB, a row-major copy for the level fills (each row padded
 * to a multiple of 16 bytes, plus 128 bytes when that is a multiple of 1 KiB):
 * about twice the matrix in all, e.g. 2 GiB + 2 GiB + 16 MiB for 131,072 x
 * 16,384 one-byte bins, whose transpose takes about 3.4 ms once.
 * Invalidates the current tree (begin_tree must be called again).
 */
hgb_status hgb_upload_bins(hgb_ctx* ctx, const void* bins, int bin_bytes, int on_device,
                           int32_t n_rows, int32_t n_features, int32_t n_bins,
                           int32_t has_missing);

/*
 * Start a tree: fixed-point encode the per-row gradients and hessians
 * ([bonsai-9] "The idea": device histogram cells are int64 fixed point, so a
 * sum of cells is one integer whatever the order of the additions).
 *
 * For c in {grad, hess}: M = max |c_i|; k = 0 if M == 0, else k = P - e with
 * 2^(e-1) <= M < 2^e; q_i = round-half-even(c_i * 2^k).  |q_i| <= 2^P.  P is
 * the context's precision (hgb_set_precision, default 30).
 *
 * grad_dev, hess_dev: fp32 [n_rows] device arrays (n_rows of upload_bins).
 * Waits once for the two maxima, to check them (unless hgb_set_async_begin
 * is on).  The scales stay on the device for the later kernels.
 * Errors: HGB_E_STATE before upload_bins; HGB_E_NONFINITE for a NaN/Inf value
 *         or a hessian < 0 (-0.0 counts as 0) -- no tree is started then.
 *         With hgb_set_async_begin on, the non-finite check is deferred (see
 *         there).
 */
hgb_status hgb_begin_tree(hgb_ctx* ctx, const float* grad_dev, const float* hess_dev);

/*
 * Asynchronous begin_tree (enable nonzero) or the default, waiting one
 * (enable 0) ([bonsai-10] "Deferred": once the kernels are on the device, host
 * orchestration is what remains between the levels; here no host round trip
 * stands between a tree's start and its first level's launches).
 *
 * When on, hgb_begin_tree and hgb_begin_tree_objective enqueue their passes
 * and return HGB_OK without waiting for the maxima.  Everything the tree's
 * kernels need stays on the device.  The host reads the maxima back at the
 * next call that needs them: hgb_get_scales (which waits for them), the next
 * begin_tree, upload_bins, set_precision or hgb_sync.  A NaN/Inf value or a
 * negative hessian is then reported once, as HGB_E_NONFINITE, by the next
 * hgb_sync (hgb_get_scales also returns it); the histograms and splits of
 * that tree are meaningless.
 * Errors: HGB_E_INVALID for a null context.
 */
hgb_status hgb_set_async_begin(hgb_ctx* ctx, int enable);

/* Losses that hgb_begin_tree_objective differentiates. */
typedef enum {
    HGB_OBJ_SQUARED = 0,    /* (m - y)^2 / 2:        g = m - y, h = 1 */
    HGB_OBJ_LOGISTIC = 1,   /* log(1 + e^m) - y m:   g = p - y, h = p (1 - p), p = 1/(1 + e^-m) */
    HGB_OBJ_POISSON = 2     /* e^m - y m:            g = e^m - y, h = e^m */
} hgb_objective;

/*
 * begin_tree fed by a device-resident objective ([bonsai-10] "The device
 * context lifecycle": with the objective resident, the (grad, hess) pairs are
 * derived on the device from the resident scores and labels, so nothing
 * crosses the bus per tree).
 *
 * Per row i, in double, one rounding per operation in the order written and no
 * fused multiply-add: (g, h) from the table above at m = margin[i],
 * y = label[i], each times weight[i] (1 when weight_dev is NULL); exp is
 * computed by Cody-Waite argument reduction (ln 2 split into a 36-bit head
 * and its rounded remainder, n = rint(x / ln 2)) and the degree-13 Taylor
 * polynomial in Horner form, scaled by 2^n; it is +Inf above 1000 and 0 below
 * -1000.  Each of g and h is then rounded once to fp32, and the tree starts
 * exactly as hgb_begin_tree would with those fp32 arrays (same scales, same
 * codes, same errors).  The fp32 pairs are never stored.
 *
 * margin_dev, label_dev: fp32 [n_rows] device arrays; weight_dev: fp32
 * [n_rows] or NULL.  The caller owns all three.
 * Errors: as hgb_begin_tree; HGB_E_INVALID for an unknown objective or a NULL
 *         margin or label.
 */
hgb_status hgb_begin_tree_objective(hgb_ctx* ctx, int32_t objective, const float* margin_dev,
                                    const float* label_dev, const float* weight_dev);

/* Copy the current tree's fixed-point pairs (qg, qh) into q_dev, int32
 * [n_rows][2] on the device (stream-ordered; caller owns q_dev).
 * Errors: HGB_E_STATE before a tree is started. */
hgb_status hgb_copy_quantized(hgb_ctx* ctx, int32_t* q_dev);

/* Fixed-point precision P of the next begin_tree, in bits below the largest
 * |value| (1..30, default 30).  Any P gives exact int64 cells; at P <= 19 the
 * fill packs both components of a cell into one 64-bit LDS add (the packing of
 * [ybb] section 7), which halves its LDS traffic.  Ends the current tree.
 * Errors: HGB_E_INVALID for bits outside [1, 30]. */
hgb_status hgb_set_precision(hgb_ctx* ctx, int32_t bits);

/* The current tree's scales: a fixed-point sum X stands for X * 2^-k
 * ([bonsai-9] "The idea": the device cells are int64 fixed point; these are
 * the exponents that turn them back into gradient and hessian sums).
 * Waits for them after an asynchronous begin_tree.
 * Errors: HGB_E_INVALID for a null pointer; HGB_E_STATE before begin_tree;
 *         HGB_E_NONFINITE for a tree started asynchronously from non-finite
 *         values. */
hgb_status hgb_get_scales(const hgb_ctx* ctx, int32_t* k_g, int32_t* k_h);

/*
 * Build the histograms of a level's nodes from rows ([bonsai-E6] "Two fills,
 * one choice": each row of a node contributes its gradient and hessian to the
 * bin it falls in, in each feature's histogram; [bonsai-10] "Level batching":
 * all nodes of a level in one pass).  Cells are exact int64 sums of the
 * fixed-point values.
 *
 * row_index_dev:     int32, the nodes' row lists concatenated, node i owning
 *                    entries [node_offsets[i], node_offsets[i+1]).  Order within
 *                    a node does not change the result.  May be NULL when every
 *                    node is empty.
 * node_offsets_host: int32 [n_nodes + 1], starts at 0, non-decreasing.  When
 *                    both row_index_dev and node_offsets_host are NULL the call
 *                    builds the root: one node (n_nodes must be 1) holding rows
 *                    0..n-1 in order.
 * hist_dev:          level buffer; node i's histogram is written, in full, at
 *                    node slot out_slot_host[i] (i when out_slot_host is NULL).
 *                    A slot of -1 skips node i: its rows are not read and no
 *                    slot is written (so a level laid out by
 *                    hgb_partition_level builds only the smaller child of each
 *                    pair).  The caller sizes hist_dev to cover every slot
 *                    written.
 * Errors: HGB_E_STATE before begin_tree; HGB_E_INVALID for bad offsets, slots
 *         (below -1, or two nodes on one slot) or n_nodes < 1.
 */
hgb_status hgb_build_level(hgb_ctx* ctx, const int32_t* row_index_dev,
                           const int32_t* node_offsets_host, int32_t n_nodes,
                           int64_t* hist_dev, const int32_t* out_slot_host);

/*
 * Derive every pair's other child: other = parent - built, slot by slot, exact
 * ([ybb] section 3, histogram subtraction: the larger child's histogram is the
 * parent's minus the smaller one's; integer cells need no clamp).
 *
 * parent_dev:          [n_pairs][F][S][2] int64; pair i's parent is node slot i.
 * child_dev:           [2*n_pairs][F][S][2] int64; pair i's children are node
 *                      slots 2i (left) and 2i+1 (right).  The built child is at
 *                      2i + built_is_right_host[i]; the other one is written.
 * built_is_right_host: uint8 [n_pairs] (nonzero: the right child was built).
 * Errors: HGB_E_STATE before upload_bins; HGB_E_INVALID for n_pairs outside
 *         [0, 65535] or a null pointer with n_pairs > 0.
 */
hgb_status hgb_subtract_siblings(hgb_ctx* ctx, const int64_t* parent_dev, int64_t* child_dev,
                                 const uint8_t* built_is_right_host, int32_t n_pairs);

/*
 * hgb_subtract_siblings with the parents anywhere in a level buffer: pair i's
 * parent is node slot parent_slot_host[i] of parent_dev (i when
 * parent_slot_host is NULL), so the parents can stay where the previous level
 * left them ([bonsai-10] "The device context lifecycle": the previous
 * frontier's histograms stay resident and the children are derived from them
 * in place).  Otherwise as hgb_subtract_siblings.
 *
 * parent_slot_host:    int32 [n_pairs] or NULL.
 * Errors: as hgb_subtract_siblings; HGB_E_INVALID for a negative parent slot.
 */
hgb_status hgb_subtract_siblings_slots(hgb_ctx* ctx, const int64_t* parent_dev, int64_t* child_dev,
                                       const uint8_t* built_is_right_host,
                                       const int32_t* parent_slot_host, int32_t n_pairs);

/*
 * Best split of every node of a level ([ybb] section 1: the gain
 * G_L^2/(H_L+lambda) + G_R^2/(H_R+lambda) - G^2/(H+lambda) - gamma, here without
 * the constant factor 1/2; section 4: missing rows tried on each side;
 * [bonsai-9] "In bonsai": ties resolved as a serial scan in feature order).
 *
 * For each feature, candidates (b, d) for b in [0, B) and d in {right} (or
 * {right, left} when has_missing): the left side holds value bins <= b plus the
 * missing slot if d is left.  Valid iff both integer hessian sums are > 0.
 * Sums are converted as (double)X * 2^-k, the gain evaluated in fp64 left to
 * right without fused multiply-add.  The best is the largest gain; ties go to
 * the smallest feature, then bin, then right before left.
 *
 * hist_dev: [n_nodes][F][S][2] int64.  out_dev: hgb_split [n_nodes] (device).
 * Errors: HGB_E_STATE before begin_tree; HGB_E_INVALID for n_nodes < 0,
 *         lambda < 0 or non-finite lambda/gamma.
 */
hgb_status hgb_find_splits(hgb_ctx* ctx, const int64_t* hist_dev, int32_t n_nodes,
                           double lambda, double gamma, hgb_split* out_dev);

/*
 * hgb_find_splits for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, checks and results as hgb_find_splits, but its intermediate
 * per-feature winners and node totals live in one fixed array of
 * HGB_NOALLOC_SCRATCH_BYTES per device, allocated with the library and held
 * until the process ends, so the call itself allocates nothing (no hipMalloc,
 * no hipFree, no event, no staging buffer) and is not timed by
 * hgb_profile_enable.  The caller still passes the histograms and the output.
 *
 * The array is shared by every context and call on a device and keeps the
 * last call's contents (nothing in it needs clearing: each call writes every
 * entry it reads).  Calls that overlap on one device -- on different streams,
 * or from different host threads -- race on it; order them on one stream.
 *
 * Limit: n_nodes * ceil(F / 4) * 32 bytes (n_nodes * F * 32 with more than
 * 256 bins per feature), rounded up to 256, plus n_nodes * 16 must not exceed
 * HGB_NOALLOC_SCRATCH_BYTES.
 * Errors: as hgb_find_splits; HGB_E_UNSUPPORTED beyond the limit.
 */
#define HGB_NOALLOC_SCRATCH_BYTES (16u << 20)
hgb_status hgb_find_splits_noalloc(hgb_ctx* ctx, const int64_t* hist_dev, int32_t n_nodes,
                                   double lambda, double gamma, hgb_split* out_dev);

/*
 * The oblivious (symmetric) level split: one (feature, bin, direction) for all
 * n_nodes nodes of a level ([bonsai-10] "The device context lifecycle":
 * find_level_split is the oblivious grower's scan of the frontier; [ybb]
 * section 5: every node of a level of a symmetric tree uses the same feature
 * and threshold).
 *
 * Candidates, their validity in a node and a node's gain are those of
 * hgb_find_splits, each node using its own totals.  A candidate's level score
 * is the sum, in node order starting from 0.0, of its gain in each node where
 * it is valid (a node where it leaves a side without hessian adds nothing); a
 * candidate valid in no node is not a candidate.  The level split has the
 * largest score; ties go to the smallest feature, then bin, then right before
 * left.
 *
 * out_dev: hgb_split [n_nodes + 1] on the device.  Record i < n_nodes: the
 * level's feature, bin, default_left; gain = node i's term of the score (0.0
 * where the split is not valid in node i); g_left, h_left = node i's left
 * sums under the split; g_total, h_total = node i's totals (feature 0).
 * Record n_nodes: the level's feature, bin, default_left, gain = the score,
 * and the integer fields summed over the nodes.  With no candidate every
 * record has feature = bin = -1, default_left 0, gain -inf, g_left = h_left
 * = 0.  The node records can be handed to hgb_partition_level as they are:
 * every node then gets two children, one of them possibly empty.
 *
 * Scratch: n_nodes * n_features * n_bins * (1 or 2 directions) doubles.
 * Errors: as hgb_find_splits.
 */
hgb_status hgb_find_level_split(hgb_ctx* ctx, const int64_t* hist_dev, int32_t n_nodes,
                                double lambda, double gamma, hgb_split* out_dev);

/*
 * hgb_subtract_siblings_slots followed by hgb_find_splits over the 2 * n_pairs
 * children, in one pass over the histograms ([ybb] section 3 subtraction and
 * section 1 gain; [bonsai-10] "Level batching": the level's tail in a fixed
 * number of launches): the result (the other children written, one hgb_split
 * per child in out_dev) is exactly that of the two calls.  Arguments as for
 * those calls; out_dev holds 2 * n_pairs records.
 * Errors: as for those calls; HGB_E_INVALID for n_pairs above 32767.
 */
hgb_status hgb_subtract_find_splits(hgb_ctx* ctx, const int64_t* parent_dev, int64_t* child_dev,
                                    const uint8_t* built_is_right_host,
                                    const int32_t* parent_slot_host, int32_t n_pairs,
                                    double lambda, double gamma, hgb_split* out_dev);

/*
 * Route every split node's rows to its children on the device ([bonsai-10]
 * "The device context lifecycle": the level's rows are partitioned on the
 * device and only split records cross the bus).  A row goes left when its
 * stored value for the split feature is a value bin <= the split bin, or is
 * the missing sentinel and default_left is set.  The partition is stable: rows
 * keep their order within each child.  Nodes without a split (feature -1) get
 * no children and their rows are dropped.  The children of the j-th node with
 * a split (counting such nodes only, in node order) are 2j (left) and 2j + 1
 * (right).
 *
 * row_index_dev, node_offsets_host, n_nodes: the level's nodes as for
 *                       hgb_build_level (both NULL with n_nodes = 1: the root,
 *                       rows 0..n-1).
 * splits_dev:           hgb_split [n_nodes] (device), as find_splits writes them.
 * out_row_index_dev:    int32, room for every row of the split nodes (at most
 *                       node_offsets_host[n_nodes], or n for the root): the
 *                       children's rows, concatenated in child order.
 * child_offsets_host:   int32 [2 * n_nodes + 1]; on return [0, 2c] hold the
 *                       children's offsets into out_row_index_dev.
 * n_children_host:      on return, 2c for c nodes with a split.
 * parent_node_host:     int32 [n_nodes] or NULL; on return entry j holds the
 *                       node whose children are 2j and 2j + 1.
 * Waits until the child sizes are on the host (the host plans the next level
 * from them); the scatter of the rows may still be running then, ordered on
 * the stream before any later work.  A row index outside [0, n) is routed
 * right and reported as HGB_E_INVALID by this call.
 * Errors: HGB_E_STATE before upload_bins; HGB_E_INVALID for null pointers or
 *         bad offsets, n_nodes outside [1, 65535].
 */
hgb_status hgb_partition_level(hgb_ctx* ctx, const int32_t* row_index_dev,
                               const int32_t* node_offsets_host, int32_t n_nodes,
                               const hgb_split* splits_dev, int32_t* out_row_index_dev,
                               int32_t* child_offsets_host, int32_t* n_children_host,
                               int32_t* parent_node_host);

/*
 * One level of a depthwise tree grown on the device, in one call: the level
 * loop of [bonsai-10] "The device context lifecycle" (partition the previous
 * level's rows on the device, build the new level, find its splits; only the
 * child sizes cross the bus), with the histogram subtraction of [ybb] §3
 * (build the child with fewer rows, the left one on a tie, and derive its
 * sibling as parent minus built).  Exactly the calls
 *   hgb_partition_level(parent_rows, parent_offsets, n_parents, parent_splits)
 *   hgb_build_level(child_rows, child_offsets, n_children, child_hist, slots)
 *       with slots[i] = i for the built child of each pair, -1 for the other
 *   hgb_subtract_find_splits(parent_hist, child_hist, built_is_right,
 *       parent_node, n_children / 2, lambda, gamma, child_splits)
 * made back to back from the library, with no return to the caller in
 * between: the host plans the build while the partition's scatter runs.
 * With oblivious nonzero (the symmetric tree of [ybb] §5) the last call is
 *   hgb_subtract_siblings_slots(parent_hist, child_hist, built_is_right,
 *       parent_node, n_children / 2) then
 *   hgb_find_level_split(child_hist, n_children, lambda, gamma, child_splits)
 * and child_splits receives n_children + 1 records (the level's last).
 *
 * parent_hist_dev:      int64 [n_parents][F][S][2], the previous level's
 *                       histograms (device).
 * parent_splits_dev:    hgb_split [n_parents] (device).
 * parent_rows_dev, parent_offsets_host, n_parents: the previous level's nodes
 *                       as for hgb_partition_level (NULL, NULL, 1: the root).
 * child_rows_dev:       int32 (device), room for every row of the parents.
 * child_hist_dev:       int64 (device), room for 2 * n_parents node slots.
 * child_splits_dev:     hgb_split (device), room for 2 * n_parents records
 *                       (2 * n_parents + 1 when oblivious).
 * child_offsets_host:   int32 [2 * n_parents + 1]; on return [0, n_children]
 *                       hold the children's offsets into child_rows_dev.
 * n_children_host:      on return, 2c for c parents with a split; 0 means the
 *                       tree ends here (nothing is built).
 * built_is_right_host:  uint8 [n_parents]; on return entry j is 1 when child
 *                       2j + 1 (right) was built, 0 for child 2j.
 * parent_node_host:     int32 [n_parents] or NULL; on return entry j holds the
 *                       parent of children 2j and 2j + 1.
 * built_rows_host:      int64 or NULL; on return the rows of the built children.
 * lambda, gamma:        as for hgb_find_splits.
 * oblivious:            nonzero for the oblivious level split (above).
 * Errors: HGB_E_INVALID for null output pointers or n_parents outside
 *         [1, 32767]; otherwise as for the three calls (the first failing
 *         one's status; the calls after it are not made).
 */
hgb_status hgb_grow_level(hgb_ctx* ctx, const int64_t* parent_hist_dev, const hgb_split* parent_splits_dev,
                          const int32_t* parent_rows_dev, const int32_t* parent_offsets_host, int32_t n_parents,
                          int32_t* child_rows_dev, int64_t* child_hist_dev, hgb_split* child_splits_dev,
                          int32_t* child_offsets_host, int32_t* n_children_host, uint8_t* built_is_right_host,
                          int32_t* parent_node_host, int64_t* built_rows_host, double lambda, double gamma,
                          int32_t oblivious);

/*
 * Per-kernel device timing ([bonsai-10] "The kernel": the pages' backend
 * prints an upload / gpu / unpack breakdown when asked).  When enabled, every
 * launch is bracketed by HIP events on the context's stream.
 */
typedef enum {
    HGB_KERNEL_QUANTIZE = 0,   /* begin_tree: max-reduce + quantize */
    HGB_KERNEL_GATHER = 1,     /* build_level: level-order (g, h) gather */
    HGB_KERNEL_ZERO = 2,       /* build_level: zeroing of atomically merged slices */
    HGB_KERNEL_FILL = 3,       /* build_level: LDS histogram fill + merge (the sum of 7, 8, 9) */
    HGB_KERNEL_SUBTRACT = 4,   /* subtract_siblings */
    HGB_KERNEL_SPLIT = 5,      /* find_splits (both kernels) */
    HGB_KERNEL_PARTITION = 6,  /* partition_level (three kernels) */
    /* the parts of HGB_KERNEL_FILL, each launch bracketed on its own: */
    HGB_KERNEL_FILL_ROOT = 7,  /* the root's fill launches */
    HGB_KERNEL_FILL_LEVEL = 8, /* the fill launch of a level below the root */
    HGB_KERNEL_MERGE = 9,      /* merges of nodes' partial histograms */
    HGB_KERNEL_COUNT = 10
} hgb_kernel;

/* Turn timing on (nonzero) or off, and reset the counters. */
hgb_status hgb_profile_enable(hgb_ctx* ctx, int enable);

/* Total device milliseconds and launch count of one kernel class since the
 * last reset.  Synchronizes the stream.  HGB_E_INVALID for a bad id. */
hgb_status hgb_profile_query(hgb_ctx* ctx, int kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif
