// Device kernels of the hgb library (gfx950).  Internal header: included by
// hgb.hip only.  All integer work is exact; the one floating-point kernel (the
// split scan) is compiled without fused multiply-add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hgb {

constexpr int kWave = 64;
constexpr uint32_t kErrRowIndex = 1u;

// ---------------------------------------------------------------------------
// begin_tree: exact maxima of |grad| and of hess as IEEE bit patterns.
// For non-negative floats the bit pattern orders like the value, so an
// unsigned max of the patterns is the pattern of the max.  The hessian's
// pattern is taken as stored (a negative value has its sign bit set and so
// lands above +Inf's pattern); -0.0 is mapped to +0.0.  Any max pattern
// >= 0x7f800000 therefore means NaN, Inf or a negative hessian.
// ---------------------------------------------------------------------------
__global__ void k_clear_u32(uint32_t* p, int n)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ __launch_bounds__(256) void k_grad_hess_max(const float* __restrict__ g,
                                                       const float* __restrict__ h, int64_t n,
                                                       uint32_t* __restrict__ out)
{
    uint32_t mg = 0, mh = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        uint32_t bg = __float_as_uint(g[i]) & 0x7fffffffu;
        uint32_t bh = __float_as_uint(h[i]);
        if (bh == 0x80000000u) bh = 0u;
        mg = bg > mg ? bg : mg;
        mh = bh > mh ? bh : mh;
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        uint32_t og = __shfl_xor(mg, off, kWave);
        uint32_t oh = __shfl_xor(mh, off, kWave);
        mg = og > mg ? og : mg;
        mh = oh > mh ? oh : mh;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) {
        atomicMax(&out[0], mg);
        atomicMax(&out[1], mh);
    }
}

// q = round-half-even(c * 2^k), both components packed per row as (qg, qh).
__global__ __launch_bounds__(256) void k_quantize(const float* __restrict__ g,
                                                  const float* __restrict__ h, int64_t n,
                                                  double scale_g, double scale_h,
                                                  int2* __restrict__ q)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        double a = (double)g[i] * scale_g;   // exact: power-of-two scaling of an fp32
        double b = (double)h[i] * scale_h;
        q[i] = make_int2((int)__builtin_rint(a), (int)__builtin_rint(b));
    }
}

// upload_bins: largest stored value, to validate every value is a slot.
template <typename BinT>
__global__ __launch_bounds__(256) void k_bins_max(const BinT* __restrict__ bins, int64_t total,
                                                  uint32_t* __restrict__ out)
{
    uint32_t m = 0;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        uint32_t v = bins[i];
        m = v > m ? v : m;
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        uint32_t o = __shfl_xor(m, off, kWave);
        m = o > m ? o : m;
    }
    if ((threadIdx.x & (kWave - 1)) == 0) atomicMax(out, m);
}

// ---------------------------------------------------------------------------
// build_level
// ---------------------------------------------------------------------------

// Level-order gather of the packed fixed-point pair: gh[k] = q[row_index[k]].
// An index outside [0, n) is flagged and contributes zero.
__global__ __launch_bounds__(256) void k_gather(const int2* __restrict__ q,
                                                const int32_t* __restrict__ row_index,
                                                int64_t total, int64_t n,
                                                int2* __restrict__ gh, uint32_t* __restrict__ err)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < total; k += stride) {
        int32_t r = row_index[k];
        int2 v = make_int2(0, 0);
        if ((uint32_t)r < (uint64_t)n) v = q[r];
        else atomicOr(err, kErrRowIndex);
        gh[k] = v;
    }
}

// One unit of fill work: rows [row_begin, row_end) of the level order, features
// [f0, f0 + nf), accumulated for the node whose histogram lands at out_slot.
struct FillItem {
    int32_t out_slot;
    int32_t row_begin;
    int32_t row_end;
    int32_t f0_nf;       // f0 | (nf << 16)
    int32_t atomic_merge;
    int32_t pad[3];
};

// Zero whole node slices of the level buffer (nodes merged with atomics, and
// empty nodes).  grid.y = slice, grid.x strides over the slice's elements.
__global__ __launch_bounds__(256) void k_zero_slices(int64_t* __restrict__ hist,
                                                     const int32_t* __restrict__ slots,
                                                     int64_t node_elems)
{
    int64_t* base = hist + (int64_t)slots[blockIdx.y] * node_elems;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < node_elems; e += stride)
        base[e] = 0;
}

// LDS-staged fill.  Each block owns one FillItem: it accumulates the item's
// rows into a block-private LDS histogram of its feature tile (separate int64
// planes for g and h, slot-major per feature), then merges the tile into the
// level buffer -- a plain store when the item covers the whole node, an int64
// atomic add otherwise.  Integer adds make the result independent of the order
// in which lanes, waves and blocks land.
template <typename BinT>
__global__ __launch_bounds__(256) void k_fill_lds(const BinT* __restrict__ bins, int64_t n,
                                                  int n_features, int S,
                                                  const int2* __restrict__ gh,
                                                  const int32_t* __restrict__ row_index,
                                                  const FillItem* __restrict__ items,
                                                  unsigned long long* __restrict__ hist)
{
    extern __shared__ unsigned long long lds[];
    const FillItem it = items[blockIdx.x];
    const int f0 = it.f0_nf & 0xffff;
    const int nf = it.f0_nf >> 16;
    const int cells = nf * S;
    unsigned long long* lg = lds;
    unsigned long long* lh = lds + cells;
    for (int i = threadIdx.x; i < 2 * cells; i += blockDim.x) lds[i] = 0ull;
    __syncthreads();

    const BinT* col0 = bins + (int64_t)f0 * n;
    for (int64_t k = it.row_begin + threadIdx.x; k < it.row_end; k += blockDim.x) {
        int64_t r = row_index ? (int64_t)row_index[k] : k;
        if ((uint64_t)r >= (uint64_t)n) continue;   // flagged by the gather
        const int2 v = gh[k];
        const unsigned long long vg = (unsigned long long)(long long)v.x;
        const unsigned long long vh = (unsigned long long)(long long)v.y;
        const BinT* p = col0 + r;
        for (int f = 0; f < nf; ++f) {
            const int b = (int)p[(int64_t)f * n];
            atomicAdd(&lg[f * S + b], vg);
            atomicAdd(&lh[f * S + b], vh);
        }
    }
    __syncthreads();

    unsigned long long* out = hist + ((int64_t)it.out_slot * n_features + f0) * (int64_t)S * 2;
    if (it.atomic_merge) {
        for (int i = threadIdx.x; i < cells; i += blockDim.x) {
            const unsigned long long a = lg[i], b = lh[i];
            if (a) atomicAdd(&out[2 * i], a);
            if (b) atomicAdd(&out[2 * i + 1], b);
        }
    } else {
        for (int i = threadIdx.x; i < cells; i += blockDim.x) {
            out[2 * i] = lg[i];
            out[2 * i + 1] = lh[i];
        }
    }
}

// ---------------------------------------------------------------------------
// subtract_siblings: other = parent - built, for every pair, elementwise.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_subtract(const longlong2* __restrict__ parent,
                                                  longlong2* __restrict__ child,
                                                  const int32_t* __restrict__ plan,
                                                  int64_t pair_vec)
{
    const int pair = blockIdx.y;
    const int32_t pslot = plan[2 * pair];
    const int r = plan[2 * pair + 1];
    const longlong2* p = parent + (int64_t)pslot * pair_vec;
    const longlong2* b = child + (int64_t)(2 * pair + r) * pair_vec;
    longlong2* o = child + (int64_t)(2 * pair + 1 - r) * pair_vec;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < pair_vec; e += stride) {
        longlong2 pv = p[e], bv = b[e];
        o[e] = make_longlong2(pv.x - bv.x, pv.y - bv.y);
    }
}

// ---------------------------------------------------------------------------
// find_splits
// ---------------------------------------------------------------------------

struct FeatureBest {
    double gain;
    int32_t code;    // 2 * bin + (default left ? 1 : 0); -1 when no valid candidate
    int32_t pad;
    long long g_left;
    long long h_left;
};

__device__ inline long long wave_shfl_up_i64(long long v, int d)
{
    int lo = __shfl_up((int)(v & 0xffffffffll), d, kWave);
    int hi = __shfl_up((int)(v >> 32), d, kWave);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__device__ inline long long wave_shfl_i64(long long v, int src)
{
    int lo = __shfl((int)(v & 0xffffffffll), src, kWave);
    int hi = __shfl((int)(v >> 32), src, kWave);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

__device__ inline long long wave_shfl_xor_i64(long long v, int mask)
{
    int lo = __shfl_xor((int)(v & 0xffffffffll), mask, kWave);
    int hi = __shfl_xor((int)(v >> 32), mask, kWave);
    return (long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo);
}

// (gain, code) order: larger gain first; on equal gains the smaller code.
// A code of -1 marks "no candidate" and loses to any candidate.
__device__ inline bool better(double ga, int ca, double gb, int cb)
{
    if (ca < 0) return false;
    if (cb < 0) return true;
    if (ga > gb) return true;
    if (ga < gb) return false;
    return ca < cb;
}

#pragma clang fp contract(off)
__device__ inline double split_gain(double gl, double hl, double gr, double hr, double parent,
                                    double lam, double gamma)
{
    double left = gl * gl / (hl + lam);
    double right = gr * gr / (hr + lam);
    double s = left + right;
    s = s - parent;
    return s - gamma;
}

// One wave per (node, feature): totals, a lane-contiguous prefix scan of the
// value bins, the gain of every (bin, direction) candidate, a wave argmax.
__global__ __launch_bounds__(256) void k_split_feature(const long long* __restrict__ hist,
                                                       int n_features, int n_bins, int S,
                                                       int has_missing, double scale_g,
                                                       double scale_h, double lam, double gamma,
                                                       FeatureBest* __restrict__ best,
                                                       long long* __restrict__ totals)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int f = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    const int node = blockIdx.y;
    if (f >= n_features) return;
    const long long* hf = hist + ((int64_t)node * n_features + f) * (int64_t)S * 2;
    const int per = (n_bins + kWave - 1) / kWave;
    const int b0 = lane * per;
    const int b1 = min(b0 + per, n_bins);

    long long sg = 0, sh = 0;
    for (int b = b0; b < b1; ++b) { sg += hf[2 * b]; sh += hf[2 * b + 1]; }
    // inclusive scan of lane sums
    long long ig = sg, ih = sh;
    for (int d = 1; d < kWave; d <<= 1) {
        long long tg = wave_shfl_up_i64(ig, d);
        long long th = wave_shfl_up_i64(ih, d);
        if (lane >= d) { ig += tg; ih += th; }
    }
    const long long miss_g = has_missing ? hf[2 * n_bins] : 0;
    const long long miss_h = has_missing ? hf[2 * n_bins + 1] : 0;
    const long long G = wave_shfl_i64(ig, kWave - 1) + miss_g;
    const long long H = wave_shfl_i64(ih, kWave - 1) + miss_h;
    const double g = (double)G * scale_g;
    const double h = (double)H * scale_h;
    const double parent = g * g / (h + lam);

    double bgain = 0.0;
    int bcode = -1;
    long long bgl = 0, bhl = 0;
    long long pg = ig - sg, ph = ih - sh;   // exclusive prefix
    const int n_dirs = has_missing ? 2 : 1;
    for (int b = b0; b < b1; ++b) {
        pg += hf[2 * b];
        ph += hf[2 * b + 1];
        for (int d = 0; d < n_dirs; ++d) {
            const long long GL = pg + (d ? miss_g : 0);
            const long long HL = ph + (d ? miss_h : 0);
            const long long GR = G - GL;
            const long long HR = H - HL;
            if (!(HL > 0 && HR > 0)) continue;
            const double gain = split_gain((double)GL * scale_g, (double)HL * scale_h,
                                           (double)GR * scale_g, (double)HR * scale_h, parent,
                                           lam, gamma);
            if (bcode < 0 || gain > bgain) {   // lane visits its codes in increasing order
                bgain = gain;
                bcode = 2 * b + d;
                bgl = GL;
                bhl = HL;
            }
        }
    }
    // wave argmax over (gain, code)
    int src = lane;
    double rg = bgain;
    int rc = bcode;
    for (int off = kWave / 2; off > 0; off >>= 1) {
        double og = __longlong_as_double(wave_shfl_xor_i64(__double_as_longlong(rg), off));
        int oc = __shfl_xor(rc, off, kWave);
        int os = __shfl_xor(src, off, kWave);
        if (better(og, oc, rg, rc)) { rg = og; rc = oc; src = os; }
    }
    const long long wgl = wave_shfl_i64(bgl, src);
    const long long whl = wave_shfl_i64(bhl, src);
    if (lane == 0) {
        FeatureBest out;
        out.gain = rc < 0 ? -__builtin_inf() : rg;
        out.code = rc;
        out.pad = 0;
        out.g_left = rc < 0 ? 0 : wgl;
        out.h_left = rc < 0 ? 0 : whl;
        best[(int64_t)node * n_features + f] = out;
        if (f == 0) { totals[2 * node] = G; totals[2 * node + 1] = H; }
    }
}

struct SplitOut {
    int32_t feature, bin, default_left, pad;
    double gain;
    long long g_left, h_left, g_total, h_total;
};

// One block per node: the best feature, scanning features in order per thread
// and then reducing across threads with the same (gain, feature) order.
__global__ __launch_bounds__(256) void k_split_reduce(const FeatureBest* __restrict__ best,
                                                      const long long* __restrict__ totals,
                                                      int n_features, SplitOut* __restrict__ out)
{
    __shared__ double s_gain[256];
    __shared__ int s_feat[256];
    const int node = blockIdx.x;
    const FeatureBest* nb = best + (int64_t)node * n_features;
    double bg = 0.0;
    int bf = -1;
    for (int f = threadIdx.x; f < n_features; f += blockDim.x) {
        const FeatureBest c = nb[f];
        if (c.code < 0) continue;
        if (bf < 0 || c.gain > bg) { bg = c.gain; bf = f; }
    }
    s_gain[threadIdx.x] = bg;
    s_feat[threadIdx.x] = bf;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            double og = s_gain[threadIdx.x + w];
            int of = s_feat[threadIdx.x + w];
            if (better(og, of, s_gain[threadIdx.x], s_feat[threadIdx.x])) {
                s_gain[threadIdx.x] = og;
                s_feat[threadIdx.x] = of;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        SplitOut o;
        const int f = s_feat[0];
        o.pad = 0;
        o.g_total = totals[2 * node];
        o.h_total = totals[2 * node + 1];
        if (f < 0) {
            o.feature = -1; o.bin = -1; o.default_left = 0;
            o.gain = -__builtin_inf();
            o.g_left = 0; o.h_left = 0;
        } else {
            const FeatureBest c = nb[f];
            o.feature = f;
            o.bin = c.code >> 1;
            o.default_left = c.code & 1;
            o.gain = c.gain;
            o.g_left = c.g_left;
            o.h_left = c.h_left;
        }
        out[node] = o;
    }
}

}  // namespace hgb
