/*
 * Serial CPU oracle -- TEST INFRASTRUCTURE ONLY (see oracle.c).
 * This header belongs to the oracle alone; the HIP library never includes it.
 */
#ifndef HGB_ORACLE_H
#define HGB_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ORACLE_OK = 0,
    ORACLE_E_INVALID = 1,
    ORACLE_E_NONFINITE = 4
};

enum {
    ORACLE_OBJ_SQUARED = 0,
    ORACLE_OBJ_LOGISTIC = 1,
    ORACLE_OBJ_POISSON = 2
};

typedef struct {
    int32_t feature;       /* -1 when the node has no valid split */
    int32_t bin;           /* value bins <= bin go left */
    int32_t default_left;  /* 1: missing rows go left */
    int32_t pad;
    double gain;
    int64_t g_left, h_left;
    int64_t g_total, h_total;
} oracle_split;

int oracle_quantize(const float* c, int64_t n, int require_nonneg, int32_t bits,
                    int32_t* q_out, int32_t* k_out);

int oracle_check_bins(const void* bins, int bin_bytes, int64_t n_rows,
                      int32_t n_features, int32_t n_bins, int32_t has_missing);

void oracle_build_hist(const void* bins, int bin_bytes, int64_t n_rows,
                       int32_t n_features, int32_t n_bins, int32_t has_missing,
                       const int32_t* qg, const int32_t* qh,
                       const int32_t* row_index, const int64_t* node_offsets,
                       int32_t n_nodes, int64_t* hist);

void oracle_subtract(const int64_t* parent, int64_t* child,
                     const uint8_t* built_is_right, int32_t n_pairs,
                     int64_t node_elems);

void oracle_find_splits(const int64_t* hist, int32_t n_nodes,
                        int32_t n_features, int32_t n_bins, int32_t has_missing,
                        int32_t k_g, int32_t k_h, double lambda, double gamma,
                        oracle_split* out);

void oracle_find_level_split(const int64_t* hist, int32_t n_nodes,
                             int32_t n_features, int32_t n_bins, int32_t has_missing,
                             int32_t k_g, int32_t k_h, double lambda, double gamma,
                             oracle_split* out);

int32_t oracle_partition(const void* bins, int bin_bytes, int64_t n_rows,
                         int32_t n_bins, const int32_t* row_index,
                         const int64_t* node_offsets, int32_t n_nodes,
                         const oracle_split* splits,
                         int32_t* out_row_index, int64_t* out_offsets);

void oracle_exp_array(const double* x, int64_t n, double* out);

int oracle_objective(int32_t objective, const float* margin, const float* label,
                     const float* weight, int64_t n, float* grad, float* hess);

#ifdef __cplusplus
}
#endif

#endif
