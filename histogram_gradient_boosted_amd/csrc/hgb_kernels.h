// Device kernels of the hgb library (gfx950).  Internal header: included by
// hgb.hip only.  All integer work is exact; the floating-point work (the
// objective's (g, h) and the split scan's gain) is compiled without fused
// multiply-add.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "hgb_layout.h"

namespace hgb {

constexpr uint32_t kErrRowIndex = 1u;

// 64-bit values across a wave (two 32-bit shuffles each).
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

// Sums over a wave of int64 values.
__device__ inline long long wave_sum_i64(long long v)
{
    for (int off = kWave / 2; off > 0; off >>= 1) v += wave_shfl_xor_i64(v, off);
    return v;
}


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

// The error word into pinned host memory, in stream order (a store from the
// device instead of a copy command).
__global__ void k_post_u32(const uint32_t* __restrict__ src, uint32_t* __restrict__ host_dst)
{
    if (threadIdx.x == 0) *host_dst = *src;
}

__device__ inline uint32_t abs_pattern(float x) { return __float_as_uint(x) & 0x7fffffffu; }
__device__ inline uint32_t hess_pattern(float x)
{
    const uint32_t b = __float_as_uint(x);
    return b == 0x80000000u ? 0u : b;
}

// ---------------------------------------------------------------------------
// Row sources of begin_tree.  A source yields each row's fp32 (g, h), four
// rows at a time from 16-byte loads (fetch4) or one at a time (fetch1).
// ---------------------------------------------------------------------------
struct GradSource {   // (g, h) handed in directly
    // the quantize pass reads the pairs again (cheaper than writing guessed
    // codes in the max pass: both passes are memory-bound)
    static constexpr bool kGuess = false;
    const float* __restrict__ g;
    const float* __restrict__ h;
    __device__ void fetch4(int64_t i4, float4& a, float4& b) const
    {
        a = ((const float4*)g)[i4];
        b = ((const float4*)h)[i4];
    }
    __device__ void fetch1(int64_t i, float& a, float& b) const
    {
        a = g[i];
        b = h[i];
    }
};

// Device-resident objective: (g, h) derived from scores, labels and weights.
enum : int { kObjSquared = 0, kObjLogistic = 1, kObjPoisson = 2 };

// e^x in double.  Cody and Waite's reduction (Software Manual for the
// Elementary Functions, 1980): x = n ln2 + r, n = rint(x / ln2), with ln 2
// split into a head of 36 significant bits (n * head is exact for |n| < 2^17)
// and the double nearest the remainder; then the Taylor polynomial of degree
// 13 in r (|r| <= 0.347, first omitted term < 5e-18) in Horner form, scaled by
// 2^n with ldexp.  Every step is one IEEE operation (the library is built
// without contraction), so the bits do not depend on the compiler's choice of
// instructions.  |x| > 1000 saturates to +Inf / 0.
__device__ inline double cw_exp(double x)
{
    if (x != x) return x;
    if (x > 1000.0) return __builtin_huge_val();
    if (x < -1000.0) return 0.0;
    constexpr double kInvLn2 = 1.4426950408889634;
    constexpr double kLn2Head = 0x1.62e42fefa0000p-1;
    constexpr double kLn2Tail = 0x1.cf79abc9e3b3ap-40;
    const double n = __builtin_rint(x * kInvLn2);
    const double r = (x - n * kLn2Head) - n * kLn2Tail;
    // reciprocal factorials, degree 13 first (j! is exact in double for j <= 18)
    constexpr double kFact[14] = {6227020800.0, 479001600.0, 39916800.0, 3628800.0, 362880.0,
                                  40320.0,      5040.0,      720.0,      120.0,     24.0,
                                  6.0,          2.0,         1.0,        1.0};
    double p = 1.0 / kFact[0];
#pragma unroll
    for (int j = 1; j < 14; ++j) p = p * r + 1.0 / kFact[j];
    return __builtin_ldexp(p, (int)n);
}

template <int OBJ>
__device__ inline void objective_row(float m32, float y32, float w32, float& g, float& h)
{
    const double m = m32, y = y32, w = w32;
    double gd, hd;
    if constexpr (OBJ == kObjSquared) {
        gd = m - y;
        hd = 1.0;
    } else if constexpr (OBJ == kObjLogistic) {
        const double p = 1.0 / (1.0 + cw_exp(-m));
        gd = p - y;
        hd = p * (1.0 - p);
    } else {
        const double e = cw_exp(m);
        gd = e - y;
        hd = e;
    }
    g = (float)(gd * w);
    h = (float)(hd * w);
}

template <int OBJ, bool WEIGHTED>
struct ObjectiveSource {
    // deriving (g, h) costs fp64 work: the max pass also writes the codes at
    // the previous tree's scales, and the quantize pass reruns only when this
    // tree's scales differ
    static constexpr bool kGuess = true;
    const float* __restrict__ m;
    const float* __restrict__ y;
    const float* __restrict__ w;
    __device__ void fetch4(int64_t i4, float4& a, float4& b) const
    {
        const float4 mm = ((const float4*)m)[i4];
        const float4 yy = ((const float4*)y)[i4];
        const float4 ww = WEIGHTED ? ((const float4*)w)[i4] : make_float4(1.f, 1.f, 1.f, 1.f);
        objective_row<OBJ>(mm.x, yy.x, ww.x, a.x, b.x);
        objective_row<OBJ>(mm.y, yy.y, ww.y, a.y, b.y);
        objective_row<OBJ>(mm.z, yy.z, ww.z, a.z, b.z);
        objective_row<OBJ>(mm.w, yy.w, ww.w, a.w, b.w);
    }
    __device__ void fetch1(int64_t i, float& a, float& b) const
    {
        objective_row<OBJ>(m[i], y[i], WEIGHTED ? w[i] : 1.f, a, b);
    }
};

// Four rows per thread per step (16-byte loads, when `vec` says the source's
// arrays are 16-byte aligned); the leftover rows one by one at the end.  Each
// block writes its pair of maxima to out[2 * block], out[2 * block + 1].
// The fixed-point pair of one row at the given scales: exact power-of-two
// scaling of an fp32 value in double, then round half to even.  (A scale
// that is not the tree's own -- a guess -- may saturate the conversion; such
// codes are always rewritten.)
__device__ inline int2 encode_row(float a, float b, double scale_g, double scale_h)
{
    return make_int2((int)__builtin_rint((double)a * scale_g), (int)__builtin_rint((double)b * scale_h));
}

// Block maxima of |g| and h for k_max_final.  For a source with kGuess the
// same pass also writes each row's fixed-point pair at the previous tree's
// scales (scales[0..1], still in place): when this tree's scales turn out
// the same, k_max_final says so and the quantize pass has nothing to redo.
template <class Src>
__global__ __launch_bounds__(256) void k_grad_hess_max(Src src, int64_t n, int vec,
                                                       uint32_t* __restrict__ out,
                                                       const double* __restrict__ scales,
                                                       int2* __restrict__ q)
{
    uint32_t mg = 0, mh = 0;
    const double guess_g = scales[0], guess_h = scales[1];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = vec ? (n >> 2) : 0;
    int4* q4 = (int4*)q;
    auto fold = [&](int64_t i4, const float4& a, const float4& b) {
        mg = max(mg, max(max(abs_pattern(a.x), abs_pattern(a.y)), max(abs_pattern(a.z), abs_pattern(a.w))));
        mh = max(mh, max(max(hess_pattern(b.x), hess_pattern(b.y)), max(hess_pattern(b.z), hess_pattern(b.w))));
        if constexpr (!Src::kGuess) return;
        const int2 r0 = encode_row(a.x, b.x, guess_g, guess_h), r1 = encode_row(a.y, b.y, guess_g, guess_h);
        const int2 r2 = encode_row(a.z, b.z, guess_g, guess_h), r3 = encode_row(a.w, b.w, guess_g, guess_h);
        q4[2 * i4] = make_int4(r0.x, r0.y, r1.x, r1.y);
        q4[2 * i4 + 1] = make_int4(r2.x, r2.y, r3.x, r3.y);
    };
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // four strided groups in flight per thread
    for (; i + 3 * stride < n4; i += 4 * stride) {
        float4 a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) src.fetch4(i + u * stride, a[u], b[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u) fold(i + u * stride, a[u], b[u]);
    }
    for (; i < n4; i += stride) {
        float4 a, b;
        src.fetch4(i, a, b);
        fold(i, a, b);
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float a, b;
        src.fetch1(i, a, b);
        mg = max(mg, abs_pattern(a));
        mh = max(mh, hess_pattern(b));
        if constexpr (Src::kGuess) q[i] = encode_row(a, b, guess_g, guess_h);
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        mg = max(mg, (uint32_t)__shfl_xor((int)mg, off, kWave));
        mh = max(mh, (uint32_t)__shfl_xor((int)mh, off, kWave));
    }
    // one pair of maxima per block, reduced by k_max_final (no same-address
    // atomics, which serialize at the L2)
    __shared__ uint32_t red[2][256 / kWave];
    const int wv = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        red[0][wv] = mg;
        red[1][wv] = mh;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x / kWave); ++i) {
            mg = max(mg, red[0][i]);
            mh = max(mh, red[1][i]);
        }
        out[2 * blockIdx.x] = mg;
        out[2 * blockIdx.x + 1] = mh;
    }
}

// The maxima of the per-block pairs, into out[0..1].
// The scale 2^k of a maximum's fp32 bit pattern: k = precision - e with
// 2^(e-1) <= M < 2^e (frexp's exponent), k = 0 for M = 0.  Inf or NaN (the
// caller reports the error) gives 0.
__device__ inline double scale_of_max(uint32_t pat, int precision)
{
    if (pat >= 0x7f800000u) return 0.0;
    if (pat == 0u) return 1.0;
    int e = 0;
    (void)frexp((double)__uint_as_float(pat), &e);
    return ldexp(1.0, precision - e);
}

// Its inverse 2^-k, the factor that turns a fixed-point sum back into a value
// (1 for M = 0; 0 for Inf or NaN, as above).
__device__ inline double inv_scale_of_max(uint32_t pat, int precision)
{
    if (pat >= 0x7f800000u) return 0.0;
    if (pat == 0u) return 1.0;
    int e = 0;
    (void)frexp((double)__uint_as_float(pat), &e);
    return ldexp(1.0, e - precision);
}

// out[0..1]: the maxima's bit patterns; scales[0..1]: their scales 2^k (above),
// scales[2..3]: the inverses 2^-k that the split kernels read; *redo: 1 when
// the scales differ from the ones k_grad_hess_max encoded the rows with (the
// previous contents of scales[0..1]) or the max pass did not encode them
// (guessed 0), so that k_quantize must encode the rows.
__global__ __launch_bounds__(256) void k_max_final(const uint32_t* __restrict__ part, int n_blocks,
                                                   uint32_t* __restrict__ out, int precision,
                                                   double* __restrict__ scales,
                                                   uint32_t* __restrict__ host_out, uint32_t* __restrict__ redo,
                                                   int guessed, uint32_t* __restrict__ host_seq, uint32_t seq)
{
    __shared__ uint32_t red[2][256];
    uint32_t mg = 0, mh = 0;
    for (int i = threadIdx.x; i < n_blocks; i += blockDim.x) {
        mg = max(mg, part[2 * i]);
        mh = max(mh, part[2 * i + 1]);
    }
    red[0][threadIdx.x] = mg;
    red[1][threadIdx.x] = mh;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            red[0][threadIdx.x] = max(red[0][threadIdx.x], red[0][threadIdx.x + w]);
            red[1][threadIdx.x] = max(red[1][threadIdx.x], red[1][threadIdx.x + w]);
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        out[0] = red[0][0];
        out[1] = red[1][0];
        host_out[0] = red[0][0];   // pinned host memory: no read-back copy
        host_out[1] = red[1][0];
        const double sg = scale_of_max(red[0][0], precision), sh = scale_of_max(red[1][0], precision);
        *redo = (!guessed || sg != scales[0] || sh != scales[1]) ? 1u : 0u;
        scales[0] = sg;
        scales[1] = sh;
        scales[2] = inv_scale_of_max(red[0][0], precision);
        scales[3] = inv_scale_of_max(red[1][0], precision);
        // the tree's number last, once the maxima are visible to the host:
        // the host waits for it instead of for an event on the stream
        __threadfence_system();
        *host_seq = seq;
    }
}

// q = round-half-even(c * 2^k), both components packed per row as (qg, qh).
template <class Src>
__global__ __launch_bounds__(256) void k_quantize(Src src, int64_t n, int vec,
                                                  const double* __restrict__ scales,
                                                  const uint32_t* __restrict__ redo, int2* __restrict__ q)
{
    // the rows already hold their codes when the max pass guessed the scales
    if (*redo == 0u) return;
    // the scales k_max_final derived on the device (no host round trip)
    const double scale_g = scales[0], scale_h = scales[1];
    auto enc = [&](float a, float b) { return encode_row(a, b, scale_g, scale_h); };
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t n4 = vec ? (n >> 2) : 0;
    int4* q4 = (int4*)q;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 a, b;
        src.fetch4(i, a, b);
        const int2 r0 = enc(a.x, b.x), r1 = enc(a.y, b.y), r2 = enc(a.z, b.z), r3 = enc(a.w, b.w);
        q4[2 * i] = make_int4(r0.x, r0.y, r1.x, r1.y);
        q4[2 * i + 1] = make_int4(r2.x, r2.y, r3.x, r3.y);
    }
    for (int64_t i = 4 * n4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float a, b;
        src.fetch1(i, a, b);
        q[i] = enc(a, b);
    }
}

// upload_bins: the skipped slot of each feature (the slot holding the most
// rows; the smallest such slot on a tie), and the stored bins rotated so that
// it reads as 0.  Counts per row chunk in LDS (kCountCopies lane-interleaved
// copies, so a hot slot does not serialize), added into counts[f][S].
constexpr int kCountCopies = 4;
constexpr int64_t kCountChunk = 65536;

template <typename BinT>
__global__ __launch_bounds__(1024) void k_slot_counts(const BinT* __restrict__ bins, int64_t n, int S,
                                                      uint32_t* __restrict__ counts)
{
    extern __shared__ uint32_t cnt[];   // [S][kCountCopies]
    const int f = blockIdx.y;
    const int64_t r0 = (int64_t)blockIdx.x * kCountChunk;
    const int64_t r1 = min(n, r0 + kCountChunk);
    for (int i = threadIdx.x; i < S * kCountCopies; i += blockDim.x) cnt[i] = 0u;
    __syncthreads();
    const BinT* col = bins + (int64_t)f * n;
    const int cp = threadIdx.x & (kCountCopies - 1);
    for (int64_t r = r0 + threadIdx.x; r < r1; r += blockDim.x) {
        const int v = (int)col[r];   // validated: < S
        atomicAdd(&cnt[v * kCountCopies + cp], 1u);
    }
    __syncthreads();
    for (int sl = threadIdx.x; sl < S; sl += blockDim.x) {
        uint32_t t = 0;
        for (int k = 0; k < kCountCopies; ++k) t += cnt[sl * kCountCopies + k];
        if (t) atomicAdd(&counts[(int64_t)f * S + sl], t);
    }
}

__global__ __launch_bounds__(256) void k_hot_slot(const uint32_t* __restrict__ counts, int S,
                                                  int32_t* __restrict__ hot, uint32_t* __restrict__ hot_count)
{
    __shared__ uint32_t s_cnt[256];
    __shared__ int s_slot[256];
    const int f = blockIdx.x;
    uint32_t best = 0;
    int slot = 0;
    for (int sl = threadIdx.x; sl < S; sl += blockDim.x) {
        const uint32_t t = counts[(int64_t)f * S + sl];
        if (t > best) {   // slots visited in increasing order: the first maximum
            best = t;
            slot = sl;
        }
    }
    s_cnt[threadIdx.x] = best;
    s_slot[threadIdx.x] = slot;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            const uint32_t ob = s_cnt[threadIdx.x + w];
            const int os = s_slot[threadIdx.x + w];
            if (ob > s_cnt[threadIdx.x] || (ob == s_cnt[threadIdx.x] && os < s_slot[threadIdx.x])) {
                s_cnt[threadIdx.x] = ob;
                s_slot[threadIdx.x] = os;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        hot[f] = s_slot[0];
        hot_count[f] = s_cnt[0];
    }
}

template <typename BinT>
__global__ __launch_bounds__(256) void k_rotate(BinT* __restrict__ bins, int64_t n, int S,
                                                const int32_t* __restrict__ hot)
{
    const int f = blockIdx.y;
    const int h = hot[f];
    BinT* col = bins + (int64_t)f * n;
    for (int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < n;
         r += (int64_t)gridDim.x * blockDim.x) {
        int v = (int)col[r] - h;
        if (v < 0) v += S;
        col[r] = (BinT)v;
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

// upload_bins: row-major copy of the feature-major matrix, dst row r at byte
// r * row_stride (row_stride >= F * sizeof(BinT), padding zeroed beforehand),
// through a 64 x 64 LDS tile so both sides stay coalesced.  Blocks stride
// over the 64-row tiles (a launch's blocks times threads must stay below
// 2^32, fewer than 2^31 rows need up to 2^25 tiles).
template <typename BinT>
__global__ __launch_bounds__(256) void k_transpose(const BinT* __restrict__ src,
                                                   uint8_t* __restrict__ dst, int64_t n, int F,
                                                   int64_t row_stride)
{
    __shared__ BinT tile[64][65];
    const int f0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63;
    const int ty = threadIdx.x >> 6;
    const int64_t n_tiles = (n + 63) / 64;
    for (int64_t t = blockIdx.x; t < n_tiles; t += gridDim.x) {   // uniform across the block
        const int64_t r0 = t * 64;
        for (int j = ty; j < 64; j += 4) {
            const int f = f0 + j;
            const int64_t r = r0 + tx;
            if (f < F && r < n) tile[j][tx] = src[(int64_t)f * n + r];
        }
        __syncthreads();
        for (int j = ty; j < 64; j += 4) {
            const int64_t r = r0 + j;
            const int f = f0 + tx;
            if (r < n && f < F) ((BinT*)(dst + r * row_stride))[f] = tile[tx][j];
        }
        __syncthreads();   // the tile is rewritten next
    }
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

// A short merge list travels in the kernel's arguments (none to fetch).
struct MergeInline {
    MergeEntry e[kMergeInline];
};

__global__ __launch_bounds__(256) void k_merge(const longlong2* __restrict__ partial,
                                               longlong2* __restrict__ hist,
                                               const MergeEntry* __restrict__ plan, const MergeInline inl,
                                               int64_t node_vec)
{
    const MergeEntry m = plan ? plan[blockIdx.y] : inl.e[blockIdx.y];
    const longlong2* src = partial + (int64_t)m.first * node_vec;
    longlong2* dst = hist + (int64_t)m.out_slot * node_vec;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < node_vec; e += stride) {
        long long g = 0, h = 0;
#pragma unroll 8
        for (int j = 0; j < m.count; ++j) {
            const longlong2 v = src[(int64_t)j * node_vec + e];
            g += v.x;
            h += v.y;
        }
        if (m.atomic) {
            atomicAdd((unsigned long long*)&dst[e].x, (unsigned long long)g);
            atomicAdd((unsigned long long*)&dst[e].y, (unsigned long long)h);
        } else {
            dst[e] = make_longlong2(g, h);
        }
    }
}

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

// Work-item order for the fill: consecutive block ids are dispatched to the
// eight XCDs in turn, and each XCD has its own L2.  Give each XCD a contiguous
// run of items so that the feature tiles of one row chunk -- which share that
// chunk's (g, h) reads -- run at the same time on the same L2.
__device__ inline int xcd_item(int bid, int n_items)
{
    const int per = (n_items + 7) >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// ---------------------------------------------------------------------------
// Fill kernels
//
// Every fill block owns one FillItem and keeps a block-private histogram of its
// feature tile in LDS, with C = 2^lc copies interleaved at 8-byte granularity
// (word slot * C + copy); lane l adds into copy l mod C.  With C = 16 the 16 lanes
// that the LDS serves together always hit 16 different bank pairs, so random
// bins cause no bank conflicts and a hot bin shared by every lane (a skewed
// feature) costs no more than a uniform one.  At the end the copies are summed
// and the tile is written to the level buffer: a plain store when the item
// covers its whole node, an int64 atomic add otherwise.  Integer adds make the
// result independent of the order in which lanes, waves and blocks land.
//
// Two accumulation modes, kWide and kPacked (hgb_layout.h): [nf][2][S][C] u64
// gradient and hessian planes, or [nf][S][C] packed u64 words.
// ---------------------------------------------------------------------------

struct CellVal {
    unsigned long long a, b;
};

template <int ACC>
__device__ inline CellVal cell_val(int qg, int qh)
{
    CellVal v;
    if (ACC == kWide) {
        v.a = (unsigned long long)(long long)qg;
        v.b = (unsigned long long)(long long)qh;
    } else {
        v.a = ((unsigned long long)(uint32_t)qh << 32) + (unsigned long long)(long long)qg;
        v.b = 0ull;
    }
    return v;
}

template <int ACC>
__device__ inline void lds_add(unsigned long long* lcopy, int plane, int lc, int f, int b, CellVal v)
{
    unsigned long long* p = lcopy + f * (ACC == kWide ? 2 : 1) * plane + (b << lc);
    atomicAdd(p, v.a);
    if (ACC == kWide) atomicAdd(p + plane, v.b);
}

// The same add, addressed as feature base + (bin * C | copy): the per-lane copy
// joins the bin's offset instead of a per-lane base pointer, so an unrolled
// feature loop keeps one uniform base per feature rather than one per lane.
template <int ACC>
__device__ inline void lds_add_at(unsigned long long* lds, int cpy, int plane, int lc, int f, int b,
                                  CellVal v)
{
    const int idx = f * (ACC == kWide ? 2 : 1) * plane + ((b << lc) | cpy);
    atomicAdd(lds + idx, v.a);
    if (ACC == kWide) atomicAdd(lds + idx + plane, v.b);
}

// Zero the block's LDS tile: nf * planes * S * C words.
__device__ inline void lds_zero(unsigned long long* lds, int words)
{
    ulonglong2* l2 = (ulonglong2*)lds;
    for (int i = threadIdx.x; i < (words >> 1); i += blockDim.x) l2[i] = make_ulonglong2(0ull, 0ull);
    if ((words & 1) && threadIdx.x == 0) lds[words - 1] = 0ull;
}

// Packed mode keeps, after the copies, an int64 accumulator [nf][S][2] in LDS.
// Every `drain` steps the copies are decoded into it and zeroed, so a block
// can cover any number of rows while each copy-slot stays within
// kPackedRowsPerCopy rows between drains.
__device__ inline void lds_drain(unsigned long long* lds, int nf, int S, int plane, int lc)
{
    long long* acc = (long long*)(lds + nf * plane);
    const int cells = nf * S;
    const int C = 1 << lc;
    for (int i = threadIdx.x; i < cells; i += blockDim.x) {
        const int f = i / S;
        const int sl = i - f * S;
        unsigned long long* pg = lds + f * plane + (sl << lc);
        long long g = 0, h = 0;
        for (int cc = 0; cc < C; ++cc) {
            const int c = (cc + i) & (C - 1);   // rotated start: neighbouring lanes, other banks
            const long long v = (long long)pg[c];
            const long long lo = (long long)(int)(unsigned)(v & 0xffffffffll);
            g += lo;
            h += (v - lo) >> 32;
            pg[c] = 0ull;
        }
        acc[2 * i] += g;
        acc[2 * i + 1] += h;
    }
}

// ---------------------------------------------------------------------------
// The skipped slot.  Each feature has one slot -- the one holding the most
// rows of the matrix, found at upload -- whose adds the fills skip.  The
// stored bins are rotated per feature so that this slot reads as 0 (a compare
// with a constant), and each item recovers the slot's cell at the end as the
// item's row totals minus the feature's other cells.  A hot bin (a skewed
// feature, or the missing slot of a sparse column) would otherwise send most
// lanes of a wave to one LDS word, which serializes the atomics; here it costs
// nothing.  Exact: the recovery is an integer subtraction.
// ---------------------------------------------------------------------------

// The slot that rotated value s of a feature with rotation rot stands for.
__device__ inline int unrotate(int s, int rot, int S)
{
    const int r = s + rot;
    return r >= S ? r - S : r;
}

// The item's row totals into fix[0..1] (zeroed with the tile): each thread's
// sums, wave-reduced, then one LDS atomic pair per wave.  Every thread calls.
__device__ inline void add_item_totals(long long g, long long h, unsigned long long* fix)
{
    g = wave_sum_i64(g);
    h = wave_sum_i64(h);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        atomicAdd(&fix[0], (unsigned long long)g);
        atomicAdd(&fix[1], (unsigned long long)h);
    }
}

// Sum the tile's copies (wide) or take the drained accumulator (packed),
// recover each feature's skipped cell, and write the tile to the level
// buffer at the real slots: a plain store when the item covers its whole
// node, an int64 atomic add otherwise.  rot: the tile's rotations; fix: the
// item's totals (complete: callers synchronize after add_item_totals).
template <int ACC, bool SKIP>
__device__ inline void lds_finish(unsigned long long* lds, int nf, int S, int plane, int lc,
                                  unsigned long long* out, bool atomic_merge,
                                  const int32_t* __restrict__ rot, unsigned long long* fix)
{
    if (ACC == kPacked) {
        lds_drain(lds, nf, S, plane, lc);
        __syncthreads();
    }
    const int C = 1 << lc;
    const long long* acc = (const long long*)(lds + nf * plane);
    auto cell = [&](int f, int sl, long long& g, long long& h) {
        g = 0;
        h = 0;
        if (ACC == kWide) {
            const unsigned long long* pg = lds + f * 2 * plane + (sl << lc);
            for (int cc = 0; cc < C; ++cc) {
                const int c = (cc + sl) & (C - 1);   // rotated start: neighbouring lanes, other banks
                g += (long long)pg[c];
                h += (long long)pg[plane + c];
            }
        } else {
            g = acc[2 * (f * S + sl)];
            h = acc[2 * (f * S + sl) + 1];
        }
    };
    // each feature's skipped cell: the item's totals minus its other cells
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = (int)(blockDim.x / kWave);
    const long long tg = (long long)fix[0], th = (long long)fix[1];
    for (int f = (int)(threadIdx.x / kWave); SKIP && f < nf; f += waves) {
        long long sg = 0, sh = 0;
        for (int sl = 1 + lane; sl < S; sl += kWave) {
            long long g, h;
            cell(f, sl, g, h);
            sg += g;
            sh += h;
        }
        sg = wave_sum_i64(sg);
        sh = wave_sum_i64(sh);
        if (lane == 0) {
            fix[2 + 2 * f] = (unsigned long long)(tg - sg);
            fix[3 + 2 * f] = (unsigned long long)(th - sh);
        }
    }
    if (SKIP) __syncthreads();
    const int cells = nf * S;
    for (int i = threadIdx.x; i < cells; i += blockDim.x) {
        const int f = i / S;
        const int sl = i - f * S;
        long long g, h;
        if (SKIP && sl == 0) {
            g = (long long)fix[2 + 2 * f];
            h = (long long)fix[3 + 2 * f];
        } else {
            cell(f, sl, g, h);
        }
        const int o = SKIP ? f * S + unrotate(sl, rot[f], S) : i;
        if (atomic_merge) {
            if (g) atomicAdd(&out[2 * o], (unsigned long long)g);
            if (h) atomicAdd(&out[2 * o + 1], (unsigned long long)h);
        } else {
            out[2 * o] = (unsigned long long)g;
            out[2 * o + 1] = (unsigned long long)h;
        }
    }
}

// Slot-major ("interleaved") layout of a wide row-major tile of TF feature
// positions and C = 2^lc copies: word ((slot * 2 + plane) * C + copy) * TF + f.
// A wave's lanes take the features of a row in lane-rotated order (lane l adds
// feature (l + j) mod TF at its j-th add) and copy (l / TF) mod C, so when
// TF * C >= 32 the 64 lanes of one add land on 32 distinct u64 bank pairs,
// two lanes each, whatever the bins: the LDS's conflict-free rate.  The
// finish walks cells slot-major as well (lanes along features), so its LDS
// reads are conflict-free too.
template <bool SKIP, int TF>
__device__ inline void lds_finish_il(const unsigned long long* lds, int nf, int S, int lc,
                                     unsigned long long* out, bool atomic_merge,
                                     const int32_t* __restrict__ rot, unsigned long long* fix)
{
    const int C = 1 << lc;
    const int G = TF << lc;   // words per (slot, plane)
    const int total = S * TF;
    auto cell = [&](int i, long long& g, long long& h) {   // i = slot * TF + f
        const unsigned long long* pg = lds + (i / TF) * 2 * G + (i & (TF - 1));
        g = 0;
        h = 0;
        for (int c = 0; c < C; ++c) {
            g += (long long)pg[c * TF];
            h += (long long)pg[G + c * TF];
        }
    };
    // A thread's cells all have feature threadIdx.x mod TF (blockDim.x is a
    // multiple of TF): it sums its value cells, lanes of one feature combine
    // by shuffles, and one LDS atomic pair per wave and feature lands in fix.
    const int f_own = (int)(threadIdx.x & (TF - 1));
    if (SKIP) {
        long long sg = 0, sh = 0;
        for (int i = threadIdx.x; i < total; i += blockDim.x) {
            if (i < TF || f_own >= nf) continue;   // slot 0 is the skipped one
            long long g, h;
            cell(i, g, h);
            sg += g;
            sh += h;
        }
#pragma unroll
        for (int o = TF; o < kWave; o <<= 1) {
            sg += wave_shfl_xor_i64(sg, o);
            sh += wave_shfl_xor_i64(sh, o);
        }
        if ((threadIdx.x & (kWave - 1)) < (unsigned)TF && f_own < nf) {
            atomicAdd(&fix[2 + 2 * f_own], (unsigned long long)sg);
            atomicAdd(&fix[3 + 2 * f_own], (unsigned long long)sh);
        }
        __syncthreads();
    }
    const long long tg = (long long)fix[0], th = (long long)fix[1];
    for (int i = threadIdx.x; i < total; i += blockDim.x) {
        const int f = i & (TF - 1);
        if (f >= nf) continue;   // positions past the tile's features are never read
        const int sl = i / TF;
        long long g, h;
        if (SKIP && sl == 0) {
            g = tg - (long long)fix[2 + 2 * f];
            h = th - (long long)fix[3 + 2 * f];
        } else {
            cell(i, g, h);
        }
        const int o = f * S + (SKIP ? unrotate(sl, rot[f], S) : sl);
        if (atomic_merge) {
            if (g) atomicAdd(&out[2 * o], (unsigned long long)g);
            if (h) atomicAdd(&out[2 * o + 1], (unsigned long long)h);
        } else {
            out[2 * o] = (unsigned long long)g;
            out[2 * o + 1] = (unsigned long long)h;
        }
    }
}

// Root fill: the level's one node holds every row in order, so each thread
// reads 4 consecutive rows per step -- a 16-byte (g, h) load per two rows and
// one 4- or 8-byte bin load per feature -- and loads the next step while it
// adds the current one.  NF features per block.  (4 rows beat 8 and 2 on the
// MI355X: fewer registers in flight per wave, the LDS adds interleave better.)
// (kRootRows = 4, hgb_layout.h)

// A thread's kRootRows consecutive bins of one feature, from one load.
template <typename BinT>
struct RootBins;
template <>
struct RootBins<uint8_t> {
    uint32_t w;
    __device__ inline void load(const uint8_t* p) { w = *(const uint32_t*)p; }
    __device__ inline int at(int j) const { return (int)((w >> (8 * j)) & 0xffu); }
    // on ? a : b, selected by value (a select of the structs' addresses would
    // put a register array in scratch memory)
    __device__ static inline RootBins pick(bool on, RootBins a, RootBins b)
    {
        RootBins r;
        r.w = on ? a.w : b.w;
        return r;
    }
};
template <>
struct RootBins<uint16_t> {
    uint2 w;
    __device__ inline void load(const uint16_t* p) { w = *(const uint2*)p; }
    __device__ inline int at(int j) const
    {
        const uint32_t x = j < 2 ? w.x : w.y;
        return (int)((x >> (16 * (j & 1))) & 0xffffu);
    }
    __device__ static inline RootBins pick(bool on, RootBins a, RootBins b)
    {
        RootBins r;
        r.w.x = on ? a.w.x : b.w.x;
        r.w.y = on ? a.w.y : b.w.y;
        return r;
    }
};
static_assert(kRootRows == 4, "RootBins loads 4 rows");

template <typename BinT, int NF>
struct RootStep {
    int4 q[kRootRows / 2];
    RootBins<BinT> b[NF];
};

template <typename BinT, int NF, int ACC, bool SKIP>
__global__ __launch_bounds__(1024) void k_fill_root(const BinT* __restrict__ bins, int64_t n,
                                                    int n_features, int S, int lc,
                                                    const int2* __restrict__ q,
                                                    const FillItem* __restrict__ items, int n_items,
                                                    int vec_ok, int drain,
                                                    unsigned long long* __restrict__ hist,
                                                    const int32_t* __restrict__ rot)
{
    extern __shared__ unsigned long long lds[];
    const int item = xcd_item(blockIdx.x, n_items);
    if (item >= n_items) return;
    const FillItem it = items[item];
    const int f0 = it.f0_nf & 0xffff;   // every item of this launch has exactly NF features
    const int plane = S << lc;
    unsigned long long* const fix = lds + tile_words(ACC, NF, S, lc);
    lds_zero(lds, tile_words(ACC, NF, S, lc) + kFixWords);
    __syncthreads();
    long long tg = 0, th = 0;   // the item's row totals (this thread's share)

    unsigned long long* const lcopy = lds + (threadIdx.x & ((1 << lc) - 1));
    const BinT* const col0 = bins + (int64_t)f0 * n;
    const int64_t rb = it.row_begin, re = it.row_end;
    constexpr int R = kRootRows;
    const int64_t step = (int64_t)blockDim.x * R;
    const int64_t off = (int64_t)threadIdx.x * R;

    auto load = [&](int64_t at, RootStep<BinT, NF>& st) {
        const int4* g4 = (const int4*)(q + at);
#pragma unroll
        for (int j = 0; j < R / 2; ++j) st.q[j] = g4[j];
#pragma unroll
        for (int f = 0; f < NF; ++f) st.b[f].load(col0 + (int64_t)f * n + at);
    };
    // `live` is false for a thread whose group lies past the item: it then
    // adds zeros (to valid bins), which keeps the loop free of divergence.
    // Only an item's last step can hold such threads; the others take
    // ALL_LIVE and skip the selects.
    auto accumulate = [&](const RootStep<BinT, NF>& st, bool live, auto all_live) {
        constexpr bool ALL_LIVE = decltype(all_live)::value;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int4 qq = st.q[j >> 1];
            const int gv = (ALL_LIVE || live) ? ((j & 1) ? qq.z : qq.x) : 0;
            const int hv = (ALL_LIVE || live) ? ((j & 1) ? qq.w : qq.y) : 0;
            if (SKIP) {
                tg += gv;
                th += hv;
            }
            const CellVal v = cell_val<ACC>(gv, hv);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int b = st.b[f].at(j);
                if (!SKIP || b != 0) lds_add<ACC>(lcopy, plane, lc, f, b, v);   // 0: the skipped slot
            }
        }
    };
    auto add_row = [&](int64_t r) {
        const int2 g = q[r];
        if (SKIP) {
            tg += g.x;
            th += g.y;
        }
        const CellVal v = cell_val<ACC>(g.x, g.y);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int b = (int)col0[(int64_t)f * n + r];
            if (!SKIP || b != 0) lds_add<ACC>(lcopy, plane, lc, f, b, v);
        }
    };
    // packed: decode the copies into the accumulator every `drain` steps (the
    // step loop is uniform across the block, so the barriers are too)
    auto drain_now = [&]() {
        __syncthreads();
        lds_drain(lds, NF, S, plane, lc);
        __syncthreads();
    };

    if (vec_ok) {
        // Whole R-row groups; the rows after the last whole group are added
        // one by one afterwards.  Loads are issued unconditionally (clamped to
        // a valid group), since a load under a branch would make the compiler
        // wait for it at the join; the next step's loads are in flight while
        // the current step adds.
        const int64_t full = (re - rb) / R;
        const int64_t gend = rb + full * R;
        const int64_t n_steps = (full + blockDim.x - 1) / blockDim.x;
        const int64_t last = full > 0 ? gend - R : rb;
        int dcount = 0;
        RootStep<BinT, NF> A, B;
        // Steps before the item's last have every thread's group inside the
        // item (n_steps = ceil(full / threads)): their loads need no clamp
        // and their adds no select.  The step loop is uniform across the
        // block, so these branches do not diverge.
        using Live = std::true_type;
        using Maybe = std::false_type;
        auto at_of = [&](int64_t at, int64_t s) { return s < n_steps - 1 || at + R <= gend ? at : last; };
        if (n_steps > 0) load(at_of(rb + off, 0), A);
        for (int64_t s = 0; s < n_steps; s += 2) {
            const int64_t a_at = rb + s * step + off;
            const int64_t b_at = a_at + step;
            load(at_of(b_at, s + 1), B);
            if (s + 1 < n_steps) accumulate(A, true, Live{});
            else accumulate(A, a_at + R <= gend, Maybe{});
            if (ACC == kPacked && ++dcount == drain) { drain_now(); dcount = 0; }
            if (s + 1 >= n_steps) break;
            const int64_t c_at = b_at + step;
            load(at_of(c_at, s + 2), A);
            if (s + 2 < n_steps) accumulate(B, true, Live{});
            else accumulate(B, b_at + R <= gend, Maybe{});
            if (ACC == kPacked && ++dcount == drain) { drain_now(); dcount = 0; }
        }
        if (threadIdx.x == 0)
            for (int64_t r = gend; r < re; ++r) add_row(r);
    } else {
        const int64_t n_steps = (re - rb + blockDim.x - 1) / blockDim.x;
        int dcount = 0;
        for (int64_t s = 0; s < n_steps; ++s) {
            const int64_t r = rb + s * blockDim.x + threadIdx.x;
            if (r < re) add_row(r);
            if (ACC == kPacked && ++dcount == drain * R) { drain_now(); dcount = 0; }
        }
    }
    if (SKIP) add_item_totals(tg, th, fix);
    __syncthreads();
    lds_finish<ACC, SKIP>(lds, NF, S, plane, lc,
                          hist + ((int64_t)it.out_slot * n_features + f0) * (int64_t)S * 2,
                          it.dest == kDestAtomic, rot + f0, fix);
}

// Root fill with the interleaved (slot-major) tile: an item covers TF feature
// positions, of which the first nf are real features.  Each thread loads
// kRootRows consecutive rows of every position (positions past nf re-load the
// last real feature, and their adds land in words nothing reads), rotates its
// registers so that lane l visits feature (l + p) mod TF at its p-th
// position, and adds -- every wave-wide add spreads over the tile's TF * 2^lc
// bank pairs whatever the bins.  One (g, h) load per row serves all TF
// features.
//
// Wide sums (ACC = kWide) keep G and H planes: word ((slot * 2 + plane) * C +
// copy) * TF + f, two adds per cell.  Packed sums (ACC = kPacked, P <= 19)
// add qh * 2^32 + qg once per cell into word (slot * C + copy) * TF + f; every
// `drain` steps -- few enough rows per copy-slot for both halves to decode
// exactly -- each thread takes the words of its own RA cells (cell i = slot *
// TF + f, i = threadIdx.x + k * blockDim.x) out of the tile into int64
// registers, zeroing them.  At the end the registers are written into the
// wide layout with one copy, and the wide finish writes the tile out.
template <typename BinT, int TF>
struct RootStepIL {
    int4 q[kRootRows / 2];
    RootBins<BinT> b[TF];
};

template <typename BinT, int TF>
__device__ inline void rotate_root_bins(RootBins<BinT> (&b)[TF], int k)
{
#pragma unroll
    for (int s = 1; s < TF; s <<= 1) {
        const bool on = (k & s) != 0;
        RootBins<BinT> t[TF];
#pragma unroll
        for (int i = 0; i < TF; ++i) t[i] = RootBins<BinT>::pick(on, b[(i + s) % TF], b[i]);
#pragma unroll
        for (int i = 0; i < TF; ++i) b[i] = t[i];
    }
}


// LC0: one copy (lc_arg = 0), so that the H plane's offset from the G plane
// is a constant the LDS instruction carries (no vector add per cell).
template <typename BinT, int TF, bool SKIP, int ACC, bool LC0>
__global__ __launch_bounds__(1024) void k_fill_root_il(const BinT* __restrict__ bins, int64_t n,
                                                       int n_features, int S, int lc_arg,
                                                       const int2* __restrict__ q,
                                                       const FillItem* __restrict__ items, int n_items,
                                                       int vec_ok, int drain,
                                                       unsigned long long* __restrict__ hist,
                                                       unsigned long long* __restrict__ partial,
                                                       const int32_t* __restrict__ rot)
{
    static_assert(TF <= (kFixWords - 2) / 2, "a recovered cell per feature of the tile");
    constexpr int kLogTF = TF >= 32 ? 5 : TF >= 16 ? 4 : TF >= 8 ? 3 : TF >= 4 ? 2 : TF >= 2 ? 1 : 0;
    static_assert((1 << kLogTF) == TF, "feature positions per tile: a power of two");
    const int lc = LC0 ? 0 : lc_arg;
    constexpr bool kPack = ACC == kPacked;
    static_assert(!kPack || TF == 16, "packed sums: 16 positions, whose 256 slots the register cells cover");
    constexpr int RA = kPack ? kRootIlPackedCells : 1;
    extern __shared__ unsigned long long lds[];
    const int item = xcd_item(blockIdx.x, n_items);
    if (item >= n_items) return;
    const FillItem it = items[item];
    const int f0 = it.f0_nf & 0xffff;
    const int nf = it.f0_nf >> 16;   // 1 <= nf <= TF
    const int G = TF << lc;
    const int tile_w = root_il_words(ACC, TF, S, lc);
    unsigned long long* const fix = lds + tile_w;
    lds_zero(lds, tile_w + kFixWords);
    __syncthreads();
    long long tg = 0, th = 0;   // the item's row totals (this thread's share)
    const int lane = threadIdx.x & (kWave - 1);
    const int rl = lane & (TF - 1);                             // the lane's first feature
    const int cb = ((lane >> kLogTF) & ((1 << lc) - 1)) * TF;   // and its copy's offset
    const int gsh = (kPack ? 0 : 1) + lc + kLogTF;              // slot stride: 2G words (G packed)
    // packed: this thread's cells, drained out of the copies
    long long ag[RA], ah[RA];
#pragma unroll
    for (int k = 0; k < RA; ++k) ag[k] = ah[k] = 0;
    // Each thread takes its cells' words of every copy, so between the two
    // barriers every word has one reader.  A wave's 64 cells span four slots
    // of the 16 positions; starting each slot at copy (slot mod C) spreads
    // the lanes over the bank pairs.  (The host keeps S * 16 within the
    // block's 1024 x RA cells.)
    auto drain_cells = [&]() {
        __syncthreads();
        const int C = 1 << lc;
#pragma unroll
        for (int k = 0; k < RA; ++k) {
            const int i = (int)threadIdx.x + k * (int)blockDim.x;
            if (i < S * TF) {
                const int sl = i >> kLogTF;
                unsigned long long* const base = lds + sl * G + (i & (TF - 1));
                for (int cc = 0; cc < C; ++cc) {
                    const int cp = (cc + sl) & (C - 1);
                    const long long v = (long long)atomicExch(base + cp * TF, 0ull);
                    const long long lo = (long long)(int)(uint32_t)(unsigned long long)v;
                    ag[k] += lo;
                    ah[k] += (v - lo) >> 32;
                }
            }
        }
        __syncthreads();
    };
    int dcount = 0;

    const BinT* const col0 = bins + (int64_t)f0 * n;
    const int64_t rb = it.row_begin, re = it.row_end;
    constexpr int R = kRootRows;
    const int64_t step = (int64_t)blockDim.x * R;
    const int64_t off = (int64_t)threadIdx.x * R;

    auto load = [&](int64_t at, RootStepIL<BinT, TF>& st) {
        const int4* g4 = (const int4*)(q + at);
#pragma unroll
        for (int j = 0; j < R / 2; ++j) st.q[j] = g4[j];
#pragma unroll
        for (int f = 0; f < TF; ++f) st.b[f].load(col0 + (int64_t)(f < nf ? f : nf - 1) * n + at);
    };
    // A step's work, taken out of its loads: the rows' cell values and the
    // rotated bins (b[p] holds feature (rl + p) mod TF).  `live` is false for
    // a thread whose group lies past the item: it then adds zeros (to valid
    // bins), which keeps the loop free of divergence.  Only an item's last
    // step can hold such threads; the others take ALL_LIVE and skip the
    // selects.
    struct Work {
        CellVal v[R];
        RootBins<BinT> b[TF];
    };
    auto prepare = [&](const RootStepIL<BinT, TF>& st, bool live, Work& wk, auto all_live) {
        constexpr bool ALL_LIVE = decltype(all_live)::value;
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const int4 qq = st.q[j >> 1];
            const int gv = (ALL_LIVE || live) ? ((j & 1) ? qq.z : qq.x) : 0;
            const int hv = (ALL_LIVE || live) ? ((j & 1) ? qq.w : qq.y) : 0;
            if (SKIP) {
                tg += gv;
                th += hv;
            }
            wk.v[j] = cell_val<ACC>(gv, hv);
        }
#pragma unroll
        for (int f = 0; f < TF; ++f) wk.b[f] = st.b[f];
        rotate_root_bins<BinT, TF>(wk.b, rl);
    };
    auto accumulate = [&](const Work& wk) {
        // The TF feature offsets are recomputed every step: hoisted out of the
        // loop they would hold TF registers for the whole kernel.
        int rs = rl;
        asm volatile("" : "+v"(rs));
#pragma unroll
        for (int p = 0; p < TF; ++p) {
            const int fo = cb + ((rs + p) & (TF - 1));
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const int bin = wk.b[p].at(j);
                if (!SKIP || bin != 0) {   // 0: the skipped slot
                    const int word = (bin << gsh) + fo;
                    atomicAdd(lds + word, wk.v[j].a);
                    if (!kPack) atomicAdd(lds + word + G, wk.v[j].b);
                }
            }
        }
    };
    // One row, every real feature, in the lane's rotated order.
    auto add_row = [&](int64_t r) {
        const int2 g = q[r];
        if (SKIP) {
            tg += g.x;
            th += g.y;
        }
        const CellVal v = cell_val<ACC>(g.x, g.y);
        for (int p = 0; p < TF; ++p) {
            const int f = (rl + p) & (TF - 1);
            if (f >= nf) continue;
            const int bin = (int)col0[(int64_t)f * n + r];
            if (!SKIP || bin != 0) {
                const int word = (bin << gsh) + cb + f;
                atomicAdd(lds + word, v.a);
                if (!kPack) atomicAdd(lds + word + G, v.b);
            }
        }
    };

    if (vec_ok) {
        // Whole groups of R rows; the rows after the last whole group are
        // added one by one afterwards.  Loads are issued unconditionally
        // (clamped to a valid group).  Each step first takes its work out of
        // the load registers, then issues the next step's loads into them, so
        // those are in flight while this step adds, with one set of load
        // registers instead of two.
        const int64_t full = (re - rb) / R;
        const int64_t gend = rb + full * R;
        const int64_t n_steps = (full + blockDim.x - 1) / blockDim.x;
        const int64_t last = full > 0 ? gend - R : rb;
        RootStepIL<BinT, TF> st;
        Work wk;
        // Steps before the item's last have every thread's group inside the
        // item (n_steps = ceil(full / threads)): no clamp, no select.  The
        // step loop is uniform across the block.
        auto at_of = [&](int64_t a, int64_t s) { return s < n_steps - 1 || a + R <= gend ? a : last; };
        if (n_steps > 0) load(at_of(rb + off, 0), st);
        for (int64_t s = 0; s < n_steps; ++s) {
            const int64_t at = rb + s * step + off;
            const int64_t nx = at + step;
            if (s + 1 < n_steps) prepare(st, true, wk, std::true_type{});
            else prepare(st, at + R <= gend, wk, std::false_type{});
            __builtin_amdgcn_sched_barrier(0);   // keep the issue order
            load(at_of(nx, s + 1), st);
            __builtin_amdgcn_sched_barrier(0);
            accumulate(wk);
            if (kPack && ++dcount == drain) {
                drain_cells();
                dcount = 0;
            }
        }
        // (at most kRootRows - 1 rows on one copy: the drain period allows them)
        if (threadIdx.x == 0)
            for (int64_t r = gend; r < re; ++r) add_row(r);
    } else {
        const int64_t n_steps = (re - rb + blockDim.x - 1) / blockDim.x;
        for (int64_t s = 0; s < n_steps; ++s) {
            const int64_t r = rb + s * blockDim.x + threadIdx.x;
            if (r < re) add_row(r);
            if (kPack && ++dcount == drain) {   // one row per thread and step: within the period
                drain_cells();
                dcount = 0;
            }
        }
    }
    if (kPack) {
        // the last rows, then the cells into the one-copy wide layout (word
        // (slot * 2 + plane) * TF + f; every word was zeroed by the drain)
        drain_cells();
#pragma unroll
        for (int k = 0; k < RA; ++k) {
            const int i = (int)threadIdx.x + k * (int)blockDim.x;
            if (i < S * TF) {
                unsigned long long* const w = lds + (i >> kLogTF) * 2 * TF + (i & (TF - 1));
                w[0] = (unsigned long long)ag[k];
                w[TF] = (unsigned long long)ah[k];
            }
        }
    }
    if (SKIP) add_item_totals(tg, th, fix);
    __syncthreads();
    unsigned long long* const out = (it.dest == kDestPartial ? partial : hist) +
                                    ((int64_t)it.out_slot * n_features + f0) * (int64_t)S * 2;
    lds_finish_il<SKIP, TF>(lds, nf, S, kPack ? 0 : lc, out, it.dest == kDestAtomic, rot + f0, fix);
}

// Level fills read their rows through the row index.  Each thread takes
// kLevelEntries entries per step, strided by the block size so that index and
// (g, h) loads stay coalesced and only the bin loads scatter, in a two-stage
// pipeline: the next step's indices are in flight while this step's bins
// load, and this step's bins while the previous step adds.
// (kLevelEntries, cols_entries: hgb_layout.h)

template <int E>
struct Entries {
    int32_t r[E];
    int2 g[E];
    bool ok[E];
};

template <int E>
__device__ inline void load_entries(Entries<E>& en, const int32_t* __restrict__ row_index,
                                    const int2* __restrict__ gh, int64_t base, int64_t rb,
                                    int64_t re)
{
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t kk = base + (int64_t)e * blockDim.x + threadIdx.x;
        en.ok[e] = kk < re;
        const int64_t kc = en.ok[e] ? kk : rb;   // past the end: a valid address, masked below
        en.r[e] = row_index[kc];
        en.g[e] = gh[kc];
    }
}

template <int E>
__device__ inline void check_entries(Entries<E>& en, int64_t n)
{
#pragma unroll
    for (int e = 0; e < E; ++e) {
        en.ok[e] = en.ok[e] && (uint32_t)en.r[e] < (uint64_t)n;
        if (!en.ok[e]) en.r[e] = 0;
    }
}

// Feature-major level fill (wide matrices): NF features per block, each bin a
// scattered one-element load.
template <typename BinT, int NF, int ACC, bool SKIP>
__device__ inline void fill_cols_item(unsigned long long* lds, const FillItem& it,
                                      const BinT* __restrict__ bins, int64_t n, int n_features,
                                      int S, int lc, const int2* __restrict__ gh,
                                      const int32_t* __restrict__ row_index, int drain,
                                      unsigned long long* __restrict__ hist,
                                      unsigned long long* __restrict__ partial,
                                      const int32_t* __restrict__ rot)
{
    const int f0 = it.f0_nf & 0xffff;
    const int nf = it.f0_nf >> 16;   // <= NF
    const int plane = S << lc;
    unsigned long long* const fix = lds + tile_words(ACC, nf, S, lc);
    lds_zero(lds, tile_words(ACC, nf, S, lc) + kFixWords);
    __syncthreads();
    long long tg = 0, th = 0;   // the item's row totals (this thread's share)

    unsigned long long* const lcopy = lds + (threadIdx.x & ((1 << lc) - 1));
    const int idle_bin = SKIP ? 0 : (int)((threadIdx.x >> lc) % (unsigned)S);
    const BinT* const col0 = bins + (int64_t)f0 * n;
    const int64_t rb = it.row_begin, re = it.row_end;
    constexpr int E = cols_entries(NF);
    const int64_t step = (int64_t)blockDim.x * E;

    struct Data {
        int b[NF][E];
    };
    auto load_data = [&](const Entries<E>& en, Data& d) {
#pragma unroll
        for (int f = 0; f < NF; ++f)   // a feature past the tile re-reads the last one
#pragma unroll
            for (int e = 0; e < E; ++e) d.b[f][e] = (int)col0[(int64_t)(f < nf ? f : nf - 1) * n + en.r[e]];
    };
    // An idle entry adds zero to a lane's own bin (SKIP: reads as the skipped
    // slot 0, so it adds nothing).
    auto accumulate = [&](const Entries<E>& en, const Data& d) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const bool ok = en.ok[e];
            const int gv = ok ? en.g[e].x : 0, hv = ok ? en.g[e].y : 0;
            if (SKIP) {
                tg += gv;
                th += hv;
            }
            const CellVal v = cell_val<ACC>(gv, hv);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int b = ok ? d.b[f][e] : idle_bin;
                if (f < nf && (!SKIP || b != 0)) lds_add<ACC>(lcopy, plane, lc, f, b, v);
            }
        }
    };

    Entries<E> ea, eb;
    Data da;
    int64_t base = rb;
    load_entries<E>(ea, row_index, gh, base, rb, re);
    check_entries<E>(ea, n);
    load_data(ea, da);
    for (int64_t s = 0;; ++s) {   // uniform across the block
        const int64_t nb = base + step;
        const bool more = nb < re;
        load_entries<E>(eb, row_index, gh, nb, rb, re);   // unconditional, see k_fill_root
        accumulate(ea, da);
        if (ACC == kPacked && (s + 1) % drain == 0) {
            __syncthreads();
            lds_drain(lds, nf, S, plane, lc);
            __syncthreads();
        }
        if (!more) break;
        check_entries<E>(eb, n);
        load_data(eb, da);
        ea = eb;
        base = nb;
    }
    if (SKIP) add_item_totals(tg, th, fix);
    __syncthreads();
    lds_finish<ACC, SKIP>(lds, nf, S, plane, lc,
                          (it.dest == kDestPartial ? partial : hist) +
                              ((int64_t)it.out_slot * n_features + f0) * (int64_t)S * 2,
                          it.dest == kDestAtomic, rot + f0, fix);
}


// Level fills run one block per CU-sized share of the level: block b takes
// the items [block_first[b], block_first[b + 1]) in turn -- consecutive pieces
// of the level order, one per node that the share touches.
// Node slots of the level buffer to clear (those k_merge adds into with
// atomics, and empty nodes), cleared by the level fill itself: k_merge runs
// after it, so no separate launch is needed.
struct ZeroList {
    const int32_t* slots;   // device
    int n;
    int64_t node_vec;       // longlong2 per node slot
};

__device__ inline void zero_listed(const ZeroList& z, unsigned long long* hist)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int k = 0; k < z.n; ++k) {
        longlong2* dst = (longlong2*)hist + (int64_t)z.slots[k] * z.node_vec;
        for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < z.node_vec; e += stride)
            dst[e] = make_longlong2(0, 0);
    }
}

template <typename BinT, int NF, int ACC, bool SKIP>
__global__ __launch_bounds__(1024) void k_fill_cols(const BinT* __restrict__ bins, int64_t n,
                                                   int n_features, int S, int lc,
                                                   const int2* __restrict__ gh,
                                                   const int32_t* __restrict__ row_index,
                                                   const FillItem* __restrict__ items,
                                                   const int32_t* __restrict__ block_first, int n_blocks,
                                                   int drain, unsigned long long* __restrict__ hist,
                                                   unsigned long long* __restrict__ partial,
                                                   const int32_t* __restrict__ rot, const ZeroList zl)
{
    extern __shared__ unsigned long long lds[];
    zero_listed(zl, hist);
    const int blk = xcd_item(blockIdx.x, n_blocks);
    if (blk >= n_blocks) return;
    const int i1 = block_first[blk + 1];
    for (int ii = block_first[blk]; ii < i1; ++ii) {
        fill_cols_item<BinT, NF, ACC, SKIP>(lds, items[ii], bins, n, n_features, S, lc, gh, row_index,
                                      drain, hist, partial, rot);
        __syncthreads();
    }
}

// Row-major level fill (narrow matrices).  The resident row-major copy pads
// each row to a multiple of 16 bytes, so a row sits in one or two 64-byte
// sectors and a sparse node costs about a sector per row instead of a cache
// line per row and feature.  Each block covers the LT bytes of a row that hold
// its feature tile (LT / sizeof(BinT) features), read with one load per row.
template <int LT>
struct Chunk;
// Rotate N dwords as one little-endian byte string: afterwards byte i holds
// what byte (i + k) mod 4N held (0 <= k < 4N).  Whole dwords move in log2(N)
// conditional stages, then one alignbyte per dword shifts the remaining 0-3
// bytes.  Each lane may rotate by its own k.  A stage is one bitfield insert
// per dword under an all-ones or all-zero mask that the compiler cannot see
// through: with plain selects it merges the stages into an N-way select per
// dword (N - 1 compares and N - 1 selects each, four times the work).
template <int N>
__device__ inline void rotate_bytes(uint32_t (&d)[N], int k)
{
    const int kd = k >> 2;
#pragma unroll
    for (int s = 1; s < N; s <<= 1) {
        uint32_t m = (kd & s) != 0 ? ~0u : 0u;
        asm("" : "+v"(m));   // opaque; a function of k alone, so hoisted out of row loops
        uint32_t t[N];
#pragma unroll
        for (int i = 0; i < N; ++i) t[i] = (d[(i + s) % N] & m) | (d[i] & ~m);
#pragma unroll
        for (int i = 0; i < N; ++i) d[i] = t[i];
    }
    const uint32_t kb = (uint32_t)k & 3u;
    uint32_t t[N];
#pragma unroll
    for (int i = 0; i < N; ++i) t[i] = __builtin_amdgcn_alignbyte(d[(i + 1) % N], d[i], kb);
#pragma unroll
    for (int i = 0; i < N; ++i) d[i] = t[i];
}

template <>
struct Chunk<32> {
    uint4 w0, w1;
    __device__ inline void load(const uint8_t* p)
    {
        w0 = *(const uint4*)p;
        w1 = *(const uint4*)(p + 16);
    }
    __device__ inline uint32_t word(int i) const
    {
        const uint4& w = i < 4 ? w0 : w1;
        const int j = i & 3;
        return j == 0 ? w.x : (j == 1 ? w.y : (j == 2 ? w.z : w.w));
    }
    __device__ inline void rotate(int k)
    {
        uint32_t d[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        rotate_bytes(d, k);
        w0 = make_uint4(d[0], d[1], d[2], d[3]);
        w1 = make_uint4(d[4], d[5], d[6], d[7]);
    }
};
template <>
struct Chunk<16> {
    uint4 w;
    __device__ inline void load(const uint8_t* p) { w = *(const uint4*)p; }
    __device__ inline uint32_t word(int i) const { return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w)); }
    __device__ inline void rotate(int k)
    {
        uint32_t d[4] = {w.x, w.y, w.z, w.w};
        rotate_bytes(d, k);
        w = make_uint4(d[0], d[1], d[2], d[3]);
    }
};
template <>
struct Chunk<8> {
    uint2 w;
    __device__ inline void load(const uint8_t* p) { w = *(const uint2*)p; }
    __device__ inline uint32_t word(int i) const { return i == 0 ? w.x : w.y; }
    __device__ inline void rotate(int k)
    {
        uint32_t d[2] = {w.x, w.y};
        rotate_bytes(d, k);
        w = make_uint2(d[0], d[1]);
    }
};
template <>
struct Chunk<4> {
    uint32_t w;
    __device__ inline void load(const uint8_t* p) { w = *(const uint32_t*)p; }
    __device__ inline uint32_t word(int) const { return w; }
    __device__ inline void rotate(int k)
    {
        uint32_t d[1] = {w};
        rotate_bytes(d, k);
        w = d[0];
    }
};
template <>
struct Chunk<2> {
    uint32_t w;   // low 16 bits hold the data
    __device__ inline void load(const uint8_t* p) { w = (uint32_t)*(const uint16_t*)p; }
    __device__ inline uint32_t word(int) const { return w; }
    __device__ inline void rotate(int k) { w = k ? ((w >> 8) | (w << 8)) & 0xffffu : w; }   // k in {0, 1}
};

// Packed sums with the int64 accumulator in registers instead of LDS: thread t
// owns the cells t + k * blockDim.x, k < RA, of the tile.  The whole LDS then
// holds copies, so one block covers a whole narrow row (every feature of a
// row-major line) and each row's line is fetched once per level.
template <int RA>
struct RegAcc {
    long long g[RA], h[RA];
};

template <int RA>
__device__ inline void reg_drain(unsigned long long* lds, int cells, int S, int plane, int lc,
                                 RegAcc<RA>& a)
{
    const int C = 1 << lc;
#pragma unroll
    for (int k = 0; k < RA; ++k) {
        const int i = threadIdx.x + k * blockDim.x;
        if (i < cells) {
            const int f = i / S;
            const int sl = i - f * S;
            unsigned long long* pg = lds + f * plane + (sl << lc);
            for (int c = 0; c < C; ++c) {
                const long long v = (long long)pg[c];
                const long long lo = (long long)(int)(unsigned)(v & 0xffffffffll);
                a.g[k] += lo;
                a.h[k] += (v - lo) >> 32;
                pg[c] = 0ull;
            }
        }
    }
}

// Write the register accumulator: each feature's skipped cell is the item's
// totals minus the feature's other cells (summed into fix[2 + 2f], zeroed with
// the tile; one LDS atomic pair per wave when a wave's cells share a feature),
// and every cell goes to its real slot.
template <int RA, bool SKIP>
__device__ inline void reg_finish(const RegAcc<RA>& a, int cells, int S, unsigned long long* out,
                                  bool atomic_merge, const int32_t* __restrict__ rot,
                                  unsigned long long* fix)
{
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int k = 0; k < (SKIP ? RA : 0); ++k) {
        const int i = threadIdx.x + k * blockDim.x;
        const bool live = i < cells;
        const int f = live ? i / S : -1;
        const int sl = live ? i - f * S : 0;
        long long g = (live && sl != 0) ? a.g[k] : 0;
        long long h = (live && sl != 0) ? a.h[k] : 0;
        const int fw = __shfl(f, 0, kWave);
        if (__all(f == fw)) {   // wave-uniform: one atomic pair
            g = wave_sum_i64(g);
            h = wave_sum_i64(h);
            if (lane == 0 && fw >= 0) {
                atomicAdd(&fix[2 + 2 * fw], (unsigned long long)g);
                atomicAdd(&fix[3 + 2 * fw], (unsigned long long)h);
            }
        } else if (live && sl != 0) {
            atomicAdd(&fix[2 + 2 * f], (unsigned long long)g);
            atomicAdd(&fix[3 + 2 * f], (unsigned long long)h);
        }
    }
    if (SKIP) __syncthreads();
    const long long tg = (long long)fix[0], th = (long long)fix[1];
#pragma unroll
    for (int k = 0; k < RA; ++k) {
        const int i = threadIdx.x + k * blockDim.x;
        if (i < cells) {
            const int f = i / S;
            const int sl = i - f * S;
            long long g = a.g[k], h = a.h[k];
            if (SKIP && sl == 0) {
                g = tg - (long long)fix[2 + 2 * f];
                h = th - (long long)fix[3 + 2 * f];
            }
            const int o = SKIP ? f * S + unrotate(sl, rot[f], S) : i;
            if (atomic_merge) {
                if (g) atomicAdd(&out[2 * o], (unsigned long long)g);
                if (h) atomicAdd(&out[2 * o + 1], (unsigned long long)h);
            } else {
                out[2 * o] = (unsigned long long)g;
                out[2 * o + 1] = (unsigned long long)h;
            }
        }
    }
}

// RA > 0 (packed only): register accumulator of RA cells per thread; E
// entries per thread and step.  IL: 0 feature-major tile; 1 interleaved tile,
// one lane per row; 2 interleaved tile over 32-byte chunks, two lanes per row
// (one kPairHalfBytes half each).  LC0: the plan has one copy (lc_arg = 0),
// so the interleaved tile's H plane is a constant offset from its G plane,
// which the LDS instruction carries instead of a vector add per cell.
template <typename BinT, int LT, int ACC, int RA, int E, bool SKIP, int IL, bool LC0>
__device__ inline void fill_rows_item(unsigned long long* lds, const FillItem& it,
                                      const uint8_t* __restrict__ bins_rm, int64_t row_stride,
                                      int64_t n, int n_features, int S, int lc_arg,
                                      const int2* __restrict__ q,
                                      const int32_t* __restrict__ row_index, int drain,
                                      unsigned long long* __restrict__ hist,
                                      unsigned long long* __restrict__ partial, int& bad,
                                      const int32_t* __restrict__ rot)
{
    const int lc = LC0 ? 0 : lc_arg;
    static_assert((RA > 0) == (ACC == kPacked), "packed sums live in registers, wide sums in LDS");
    static_assert(LT / (int)sizeof(BinT) <= (kFixWords - 2) / 2, "a recovered cell per feature of the tile");
    static_assert(!IL || (ACC == kWide && RA == 0), "the interleaved layout holds wide sums in LDS");
    const int f0 = it.f0_nf & 0xffff;
    const int nf = it.f0_nf >> 16;   // <= LT / sizeof(BinT)
    constexpr int TF = LT / (int)sizeof(BinT);
    constexpr int kLogTF = TF >= 32 ? 5 : TF >= 16 ? 4 : TF >= 8 ? 3 : TF >= 4 ? 2 : TF >= 2 ? 1 : 0;
    static_assert((1 << kLogTF) == TF, "feature positions per tile: a power of two");
    // Lane pairs: lanes 2i and 2i + 1 take the two halves of one row's chunk
    // (HT positions each), so one load instruction reads a row's whole chunk
    // and the pair's two 16-byte pieces of a line go out as one request.
    constexpr bool PAIR = IL == 2;
    static_assert(!PAIR || LT == 2 * kPairHalfBytes, "lane pairs split a 32-byte chunk");
    constexpr int HT = PAIR ? TF / 2 : TF;       // positions a lane adds per row
    constexpr int kLanesPerRow = PAIR ? 2 : 1;
    const int plane = S << lc;
    const int cells = nf * S;
    // Interleaved: every one of the TF positions has its words, even past nf
    // (those lanes add the row's padding or the next tile's bins there, and
    // nothing reads them back).
    const int G = TF << lc;
    const int tile_w = IL ? 2 * S * G : nf * (ACC == kWide ? 2 : 1) * plane;
    unsigned long long* const fix = lds + tile_w;
    lds_zero(lds, tile_w + kFixWords);
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    // interleaved: the lane's first position (of its half with lane pairs),
    // the half's first position, and the lane's copy's offset.  Either way
    // the 64 lanes of one add meet every (copy, position) word equally often.
    // The LDS serves 16 lanes of a 64-bit add at a time, and positions 16
    // apart share a bank pair: a pair's second lane starts HT / 2 further on,
    // so that any 16 consecutive lanes meet 16 positions distinct mod 16 (the
    // halves' own offsets, 0 and HT, do not separate them when HT = 16).
    const int rl = PAIR ? ((lane >> 1) + (lane & 1) * (HT / 2)) & (HT - 1) : lane & (TF - 1);
    const int hb = PAIR ? (lane & 1) * HT : 0;
    const int cb = ((lane >> kLogTF) & ((1 << lc) - 1)) * TF;
    const int gsh = 1 + lc + kLogTF;                       // slot stride: 2G words
    long long tg = 0, th = 0;   // the item's row totals (this thread's share)
    RegAcc<(RA > 0 ? RA : 1)> racc;
#pragma unroll
    for (int k = 0; k < (RA > 0 ? RA : 1); ++k) racc.g[k] = racc.h[k] = 0;

    const int cpy = threadIdx.x & ((1 << lc) - 1);
    const uint8_t* const tile = bins_rm + (int64_t)f0 * sizeof(BinT) + (PAIR ? (lane & 1) * kPairHalfBytes : 0);
    const int64_t rb = it.row_begin, re = it.row_end;
    const int rows_per_pass = (int)blockDim.x / kLanesPerRow;   // entries one pass of the block takes
    const int my_entry = (int)threadIdx.x / kLanesPerRow;
    const int64_t step = (int64_t)rows_per_pass * E;

    // Per step: the row chunks and (g, h) pairs of E entries per thread, the
    // entries strided by the block size (index and (g, h) loads coalesced).
    struct Data {
        Chunk<(PAIR ? LT / 2 : LT)> c[E];
        int2 g[E];
        bool ok[E];
    };
    // Row indices of a step: loaded one step ahead of its rows.
    struct Index {
        int32_t r[E];
        bool in[E];   // inside the item
    };
    auto load_index = [&](int64_t s, Index& x) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int64_t kk = rb + s * step + (int64_t)e * rows_per_pass + my_entry;
            x.in[e] = kk < re;
            x.r[e] = row_index[x.in[e] ? kk : rb];   // past the end: a valid address, masked
        }
    };
    auto load_rows = [&](int64_t s, const Index& x, Data& d) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            d.ok[e] = x.in[e] && (uint32_t)x.r[e] < (uint64_t)n;
            bad |= (int)x.in[e] & (int)!d.ok[e];
            const int64_t r = d.ok[e] ? x.r[e] : 0;
            d.c[e].load(tile + r * row_stride);
            d.g[e] = q[r];   // the level-order gather, fused: the row's (g, h) beside its bins
        }
    };
    // Idle entries and features past the tile's nf are skipped.  (The loads
    // that a step's adds use were issued a whole step earlier, ahead of the
    // previous adds, so the compiler cannot sink them into these branches.)
    auto accumulate = [&](const Data& d) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (!d.ok[e]) continue;
            if (SKIP && hb == 0) {   // a row's (g, h) counted once, by its first lane
                tg += d.g[e].x;
                th += d.g[e].y;
            }
            const CellVal v = cell_val<ACC>(d.g[e].x, d.g[e].y);
            if (IL) {
                auto ch = d.c[e];
                ch.rotate(rl * (int)sizeof(BinT));   // position j now holds the half's feature (rl + j) mod HT
#pragma unroll
                for (int j = 0; j < HT; ++j) {
                    const uint32_t w = ch.word((j * (int)sizeof(BinT)) >> 2);
                    const int b = sizeof(BinT) == 1 ? (int)((w >> (8 * (j & 3))) & 0xffu)
                                                    : (int)((w >> (16 * (j & 1))) & 0xffffu);
                    const int word = (b << gsh) + cb + hb + ((rl + j) & (HT - 1));
                    if (!SKIP || b != 0) {   // 0: skipped
                        atomicAdd(lds + word, v.a);
                        atomicAdd(lds + word + G, v.b);
                    }
                }
                continue;
            }
            // The feature's base offset is stepped here rather than hoisted:
            // 32 hoisted values would not fit the scalar registers.
            int fb = 0;
#pragma unroll
            for (int f = 0; f < TF; ++f) {
                if (f >= nf) break;
                const uint32_t w = d.c[e].word((f * (int)sizeof(BinT)) >> 2);
                const int b = sizeof(BinT) == 1 ? (int)((w >> (8 * (f & 3))) & 0xffu)
                                                : (int)((w >> (16 * (f & 1))) & 0xffffu);
                if (!SKIP || b != 0) lds_add_at<ACC>(lds + fb, cpy, plane, lc, 0, b, v);   // 0: skipped
                fb += (ACC == kWide ? 2 : 1) * plane;
                asm volatile("" : "+s"(fb));
            }
        }
    };

    // Pipeline: step s waits for what step s - 1 issued (its own rows and
    // (g, h), and the indices of s + 1), issues the rows of s + 1 and the
    // indices of s + 2, then adds.  The memory counter retires in issue
    // order, and that one wait is all a step needs: every load it covers had
    // a whole step of adds to land.  Two data buffers alternate (the loop is
    // unrolled by two), so no register copy waits on a load in flight; the
    // index buffer is consumed before it is reloaded.  Loads past the item
    // are clamped to valid addresses and masked (unconditional, see
    // k_fill_root).
    const int64_t n_steps = (re - rb + step - 1) / step;
    Index x;
    Data d0, d1;
    load_index(0, x);
    load_rows(0, x, d0);
    load_index(1, x);
    auto run_step = [&](int64_t s, Data& cur, Data& next) {
        load_rows(s + 1, x, next);
        __builtin_amdgcn_sched_barrier(0);   // keep the issue order
        load_index(s + 2, x);
        __builtin_amdgcn_sched_barrier(0);
        accumulate(cur);
        if (ACC == kPacked && (s + 1) % drain == 0) {
            __syncthreads();
            reg_drain(lds, cells, S, plane, lc, racc);
            __syncthreads();
        }
    };
    for (int64_t s = 0; s < n_steps; s += 2) {   // uniform across the block
        run_step(s, d0, d1);
        if (s + 1 >= n_steps) break;
        run_step(s + 1, d1, d0);
    }
    if (SKIP) add_item_totals(tg, th, fix);
    __syncthreads();
    unsigned long long* const out = (it.dest == kDestPartial ? partial : hist) +
                                    ((int64_t)it.out_slot * n_features + f0) * (int64_t)S * 2;
    if (RA > 0) {
        reg_drain(lds, cells, S, plane, lc, racc);
        reg_finish<(RA > 0 ? RA : 1), SKIP>(racc, cells, S, out, it.dest == kDestAtomic, rot + f0, fix);
    } else if (IL) {
        lds_finish_il<SKIP, TF>(lds, nf, S, lc, out, it.dest == kDestAtomic, rot + f0, fix);
    } else {
        lds_finish<ACC, SKIP>(lds, nf, S, plane, lc, out, it.dest == kDestAtomic, rot + f0, fix);
    }
}


template <typename BinT, int LT, int ACC, int RA, int E, bool SKIP, int IL, bool LC0>
__global__ __launch_bounds__(1024) void k_fill_rows(const uint8_t* __restrict__ bins_rm,
                                                   int64_t row_stride, int64_t n, int n_features,
                                                   int S, int lc, const int2* __restrict__ q,
                                                   const int32_t* __restrict__ row_index,
                                                   const FillItem* __restrict__ items,
                                                   const int32_t* __restrict__ block_first, int n_blocks,
                                                   int drain, unsigned long long* __restrict__ hist,
                                                   unsigned long long* __restrict__ partial,
                                                   uint32_t* __restrict__ err,
                                                   const int32_t* __restrict__ rot, const ZeroList zl)
{
    extern __shared__ unsigned long long lds[];
    zero_listed(zl, hist);
    const int blk = xcd_item(blockIdx.x, n_blocks);
    if (blk >= n_blocks) return;
    const int i1 = block_first[blk + 1];
    int bad = 0;   // a row index outside [0, n): skipped, and flagged
    for (int ii = block_first[blk]; ii < i1; ++ii) {
        fill_rows_item<BinT, LT, ACC, RA, E, SKIP, IL, LC0>(lds, items[ii], bins_rm, row_stride, n, n_features, S,
                                             lc, q, row_index, drain, hist, partial, bad, rot);
        __syncthreads();
    }
    if (bad) atomicOr(err, kErrRowIndex);
}

// ---------------------------------------------------------------------------
// subtract_siblings: other = parent - built, for every pair, elementwise.
// ---------------------------------------------------------------------------
// A small plan travels in the kernel's arguments (no upload).
struct SubtractInline {
    int32_t v[2 * kSubtractInlinePairs];   // per pair: parent slot, built side
};

__global__ __launch_bounds__(256) void k_subtract(const longlong2* __restrict__ parent,
                                                  longlong2* __restrict__ child,
                                                  const int32_t* __restrict__ plan,
                                                  const SubtractInline inl, int64_t pair_vec)
{
    const int pair = blockIdx.y;
    const int32_t pslot = plan ? plan[2 * pair] : inl.v[2 * pair];
    const int r = plan ? plan[2 * pair + 1] : inl.v[2 * pair + 1];
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
    int32_t code;      // 2 * bin + (default left ? 1 : 0); -1 when no valid candidate
    int32_t feature;   // the feature the candidate belongs to
    long long g_left;
    long long h_left;
};



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

// The best of a block's waves (one feature each, in feature order), in the
// serial order: larger gain, then the smaller feature.  s holds one entry per
// wave; thread 0 returns the winner.
__device__ inline FeatureBest block_feature_best(const FeatureBest* s, int waves)
{
    FeatureBest b = s[0];
    for (int i = 1; i < waves; ++i)
        if (better(s[i].gain, s[i].code < 0 ? -1 : s[i].feature, b.gain, b.code < 0 ? -1 : b.feature))
            b = s[i];
    return b;
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

// One wave, one (node, feature): totals, a lane-contiguous prefix scan of the
// value bins, the gain of every (bin, direction) candidate, a wave argmax.
// Every lane returns the result (gain -inf and code -1 when no candidate).
struct WaveBest {
    FeatureBest fb;
    long long G, H;   // the feature's slot sums: the node totals
};

// A lane's value slots [lane * PER, lane * PER + PER) (zeros past n_bins) and
// the feature's missing slot, held in registers.
template <int PER>
struct LaneSlots {
    longlong2 v[PER > 0 ? PER : 1];
    longlong2 miss;
};

// Read the lane's slots, 16 bytes at a time (PER > 0; the buffer 16-byte
// aligned), or only the missing slot (PER == 0: the scan reads memory).
template <int PER>
__device__ inline void load_lane_slots(const long long* __restrict__ hf, int n_bins, int has_missing,
                                       LaneSlots<PER>& s)
{
    const int lane = threadIdx.x & (kWave - 1);
    if (PER > 0) {
        const longlong2* h2 = (const longlong2*)hf;
        const int b0 = lane * PER;
        const int b1 = min(b0 + PER, n_bins);
#pragma unroll
        for (int j = 0; j < (PER > 0 ? PER : 1); ++j) {
            const int b = b0 + j;
            const longlong2 t = h2[min(b, n_bins - 1)];   // unconditional, masked below
            s.v[j] = b < b1 ? t : make_longlong2(0, 0);
        }
    }
    s.miss = has_missing ? make_longlong2(hf[2 * n_bins], hf[2 * n_bins + 1]) : make_longlong2(0, 0);
}

// The prefix scan of one feature's value slots across a wave.  Each lane owns
// the value bins [b0, b1) = [lane * per, lane * per + per) clipped to n_bins.
// wave_prefix scans the lane sums across the wave and returns the feature's
// totals G, H (missing slot included) and the lane's exclusive prefix;
// prefix_visit then calls visit(b, GL, HL) for each of the lane's bins in
// increasing order, with the inclusive prefix sums of the value slots 0..b.
// PER > 0 scans the registers in s; PER == 0 reads the slots from hf (any bin
// count).
struct WavePrefix {
    long long G, H;     // totals
    long long pg, ph;   // sums of the value slots before the lane's first bin
    int b0, b1;
};

template <int PER>
__device__ inline WavePrefix wave_prefix(const long long* __restrict__ hf, const LaneSlots<PER>& s, int n_bins)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int per = PER > 0 ? PER : (n_bins + kWave - 1) / kWave;
    WavePrefix p;
    p.b0 = lane * per;
    p.b1 = min(p.b0 + per, n_bins);
    long long sg = 0, sh = 0;
    if (PER > 0) {
#pragma unroll
        for (int j = 0; j < (PER > 0 ? PER : 1); ++j) { sg += s.v[j].x; sh += s.v[j].y; }
    } else {
        for (int b = p.b0; b < p.b1; ++b) { sg += hf[2 * b]; sh += hf[2 * b + 1]; }
    }
    // inclusive scan of lane sums
    long long ig = sg, ih = sh;
    for (int d = 1; d < kWave; d <<= 1) {
        long long tg = wave_shfl_up_i64(ig, d);
        long long th = wave_shfl_up_i64(ih, d);
        if (lane >= d) { ig += tg; ih += th; }
    }
    p.G = wave_shfl_i64(ig, kWave - 1) + s.miss.x;
    p.H = wave_shfl_i64(ih, kWave - 1) + s.miss.y;
    p.pg = ig - sg;
    p.ph = ih - sh;
    return p;
}

template <int PER, class Visit>
__device__ inline void prefix_visit(const long long* __restrict__ hf, const LaneSlots<PER>& s,
                                    const WavePrefix& p, Visit&& visit)
{
    long long pg = p.pg, ph = p.ph;
    if (PER > 0) {
#pragma unroll
        for (int j = 0; j < (PER > 0 ? PER : 1); ++j)
            if (p.b0 + j < p.b1) {
                pg += s.v[j].x;
                ph += s.v[j].y;
                visit(p.b0 + j, pg, ph);
            }
    } else {
        for (int b = p.b0; b < p.b1; ++b) {
            pg += hf[2 * b];
            ph += hf[2 * b + 1];
            visit(b, pg, ph);
        }
    }
}

// The wave's best (bin, direction) of one feature: the gain of every
// candidate from the prefix scan, then a wave argmax.  Every lane returns the
// result (gain -inf and code -1 when no candidate).
template <int PER>
__device__ inline WaveBest scan_best(const long long* __restrict__ hf, const LaneSlots<PER>& s,
                                     const WavePrefix& p, int has_missing, double scale_g, double scale_h,
                                     double lam, double gamma)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long long miss_g = s.miss.x;
    const long long miss_h = s.miss.y;
    const long long G = p.G, H = p.H;
    const double g = (double)G * scale_g;
    const double h = (double)H * scale_h;
    const double parent = g * g / (h + lam);
    double bgain = 0.0;
    int bcode = -1;
    long long bgl = 0, bhl = 0;
    const int n_dirs = has_missing ? 2 : 1;
    prefix_visit<PER>(hf, s, p, [&](int b, long long pg, long long ph) {
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
    });
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
    WaveBest r;
    r.fb.gain = rc < 0 ? -__builtin_inf() : rg;
    r.fb.code = rc;
    r.fb.feature = -1;   // set by the caller
    r.fb.g_left = rc < 0 ? 0 : wgl;
    r.fb.h_left = rc < 0 ? 0 : whl;
    r.G = G;
    r.H = H;
    return r;
}

template <int PER>
__device__ inline WaveBest wave_scan(const long long* __restrict__ hf, const LaneSlots<PER>& s, int n_bins,
                                     int has_missing, double scale_g, double scale_h, double lam,
                                     double gamma)
{
    return scan_best<PER>(hf, s, wave_prefix<PER>(hf, s, n_bins), has_missing, scale_g, scale_h, lam, gamma);
}

// Features with more bins than 64 * 4 (up to 1,024): one block of
// kSliceWaves waves per feature, wave q owning the bins [q * 64 * PER,
// (q + 1) * 64 * PER) in contiguous lane runs of PER <= 4.  A single wave
// would hold up to 16 bins per lane and leave the chip with few waves; here
// the slices' sums meet in LDS (the carry into each slice and the feature's
// totals) and each wave scans its own slice.  (kSliceWaves: hgb_layout.h)

template <int PER>
__device__ inline void load_slice_slots(const long long* __restrict__ hf, int n_bins, int has_missing,
                                        int bin0, LaneSlots<PER>& s)
{
    const int lane = threadIdx.x & (kWave - 1);
    const longlong2* h2 = (const longlong2*)hf;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        const int b = bin0 + lane * PER + j;
        const longlong2 t = h2[min(b, n_bins - 1)];   // unconditional, masked below
        s.v[j] = b < n_bins ? t : make_longlong2(0, 0);
    }
    s.miss = has_missing ? make_longlong2(hf[2 * n_bins], hf[2 * n_bins + 1]) : make_longlong2(0, 0);
}

// The slice's prefix: the lane's exclusive prefix within the wave plus the
// earlier slices' sums, and the feature's totals.  s_sum holds 2 * kSliceWaves
// values; every thread of the block calls (one barrier).
template <int PER>
__device__ inline WavePrefix slice_prefix(const LaneSlots<PER>& s, int n_bins, int bin0, long long* s_sum)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x / kWave;
    WavePrefix p;
    p.b0 = bin0 + lane * PER;
    p.b1 = min(p.b0 + PER, n_bins);
    long long sg = 0, sh = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) { sg += s.v[j].x; sh += s.v[j].y; }
    long long ig = sg, ih = sh;
    for (int d = 1; d < kWave; d <<= 1) {
        const long long tg = wave_shfl_up_i64(ig, d);
        const long long th = wave_shfl_up_i64(ih, d);
        if (lane >= d) { ig += tg; ih += th; }
    }
    if (lane == kWave - 1) {
        s_sum[2 * q] = ig;
        s_sum[2 * q + 1] = ih;
    }
    __syncthreads();
    long long cg = 0, ch = 0, tg = 0, th = 0;
#pragma unroll
    for (int k = 0; k < kSliceWaves; ++k) {
        const long long xg = s_sum[2 * k], xh = s_sum[2 * k + 1];
        cg += k < q ? xg : 0;
        ch += k < q ? xh : 0;
        tg += xg;
        th += xh;
    }
    p.G = tg + s.miss.x;
    p.H = th + s.miss.y;
    p.pg = cg + ig - sg;
    p.ph = ch + ih - sh;
    return p;
}

template <int PER>
__device__ inline WaveBest wave_feature_best(const long long* __restrict__ hf, int n_bins,
                                             int has_missing, double scale_g, double scale_h,
                                             double lam, double gamma)
{
    LaneSlots<PER> s;
    load_lane_slots<PER>(hf, n_bins, has_missing, s);
    return wave_scan<PER>(hf, s, n_bins, has_missing, scale_g, scale_h, lam, gamma);
}

// One wave per (node, feature); the block's best of its features to
// best[node][block]; node totals from feature 0.
template <int PER>
__global__ __launch_bounds__(256) void k_split_feature(const long long* __restrict__ hist,
                                                       int n_features, int n_bins, int S,
                                                       int has_missing, const double* __restrict__ inv_scale,
                                                       double lam, double gamma,
                                                       FeatureBest* __restrict__ best,
                                                       long long* __restrict__ totals)
{
    const double scale_g = inv_scale[0], scale_h = inv_scale[1];   // 2^-k, from k_max_final
    __shared__ FeatureBest s_fb[256 / kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int f = blockIdx.x * (blockDim.x / kWave) + wv;
    const int node = blockIdx.y;
    if (f < n_features) {   // uniform per wave
        const long long* hf = hist + ((int64_t)node * n_features + f) * (int64_t)S * 2;
        const WaveBest r = wave_feature_best<PER>(hf, n_bins, has_missing, scale_g, scale_h, lam, gamma);
        if (lane == 0) {
            s_fb[wv] = r.fb;
            s_fb[wv].feature = f;
            if (f == 0) { totals[2 * node] = r.G; totals[2 * node + 1] = r.H; }
        }
    } else if (lane == 0) {
        s_fb[wv].code = -1;
        s_fb[wv].feature = -1;
        s_fb[wv].gain = -__builtin_inf();
    }
    __syncthreads();
    if (threadIdx.x == 0)
        best[(int64_t)node * gridDim.x + blockIdx.x] = block_feature_best(s_fb, blockDim.x / kWave);
}

// The level tail in one pass: one wave per (pair, feature) reads the parent
// and the built child, writes the other child (parent - built) and scans both
// children, so the children are not read again by a separate split pass.
template <int PER>
__global__ __launch_bounds__(256) void k_subtract_split(const long long* __restrict__ parent,
                                                        long long* __restrict__ child,
                                                        const int32_t* __restrict__ plan,
                                                        const SubtractInline inl, int n_features,
                                                        int n_bins, int S, int has_missing,
                                                        const double* __restrict__ inv_scale, double lam,
                                                        double gamma, FeatureBest* __restrict__ best,
                                                        long long* __restrict__ totals)
{
    const double scale_g = inv_scale[0], scale_h = inv_scale[1];   // 2^-k, from k_max_final
    static_assert(PER > 0, "the fused pass keeps the slots in registers");
    __shared__ FeatureBest s_fb[2][256 / kWave];   // [0] the built child, [1] the other
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int f = blockIdx.x * (blockDim.x / kWave) + wv;
    const int pair = blockIdx.y;
    const int32_t pslot = plan ? plan[2 * pair] : inl.v[2 * pair];
    const int r = plan ? plan[2 * pair + 1] : inl.v[2 * pair + 1];
    const int nb = 2 * pair + r, no = 2 * pair + 1 - r;
    if (f >= n_features) {   // uniform per wave: no feature, no candidate
        if (lane == 0)
            for (int k = 0; k < 2; ++k) {
                s_fb[k][wv].code = -1;
                s_fb[k][wv].feature = -1;
                s_fb[k][wv].gain = -__builtin_inf();
            }
    } else {
        const int64_t fs = (int64_t)S * 2;
        const long long* hp = parent + ((int64_t)pslot * n_features + f) * fs;
        const long long* hb = child + ((int64_t)nb * n_features + f) * fs;
        long long* ho = child + ((int64_t)no * n_features + f) * fs;
        // the parent's slots become the other child's in place (fewer registers)
        LaneSlots<PER> so, sb;
        load_lane_slots<PER>(hp, n_bins, has_missing, so);
        load_lane_slots<PER>(hb, n_bins, has_missing, sb);
#pragma unroll
        for (int j = 0; j < PER; ++j) so.v[j] = make_longlong2(so.v[j].x - sb.v[j].x, so.v[j].y - sb.v[j].y);
        so.miss = make_longlong2(so.miss.x - sb.miss.x, so.miss.y - sb.miss.y);
        longlong2* o2 = (longlong2*)ho;
        const int b0 = lane * PER;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            if (b0 + j < n_bins) o2[b0 + j] = so.v[j];
        if (has_missing && lane == 0) o2[n_bins] = so.miss;
        const WaveBest wb = wave_scan<PER>(hb, sb, n_bins, has_missing, scale_g, scale_h, lam, gamma);
        const WaveBest wo = wave_scan<PER>(ho, so, n_bins, has_missing, scale_g, scale_h, lam, gamma);
        if (lane == 0) {
            s_fb[0][wv] = wb.fb;
            s_fb[0][wv].feature = f;
            s_fb[1][wv] = wo.fb;
            s_fb[1][wv].feature = f;
            if (f == 0) {
                totals[2 * nb] = wb.G;
                totals[2 * nb + 1] = wb.H;
                totals[2 * no] = wo.G;
                totals[2 * no + 1] = wo.H;
            }
        }
    }
    __syncthreads();
    if (threadIdx.x < 2)
        best[(int64_t)(threadIdx.x == 0 ? nb : no) * gridDim.x + blockIdx.x] =
            block_feature_best(s_fb[threadIdx.x], blockDim.x / kWave);
}

// One feature per block of kSliceWaves waves (wide bins): the feature's best
// to best[node][feature]; node totals from feature 0.
template <int PER>
__global__ __launch_bounds__(kSliceWaves * kWave) void k_split_feature_sliced(
    const long long* __restrict__ hist, int n_features, int n_bins, int S, int has_missing,
    const double* __restrict__ inv_scale, double lam, double gamma, FeatureBest* __restrict__ best,
    long long* __restrict__ totals)
{
    const double scale_g = inv_scale[0], scale_h = inv_scale[1];   // 2^-k, from k_max_final
    __shared__ long long s_sum[2 * kSliceWaves];
    __shared__ FeatureBest s_fb[kSliceWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x / kWave;
    const int f = blockIdx.x;
    const int node = blockIdx.y;
    const long long* hf = hist + ((int64_t)node * n_features + f) * (int64_t)S * 2;
    const int bin0 = q * kWave * PER;
    LaneSlots<PER> sl;
    load_slice_slots<PER>(hf, n_bins, has_missing, bin0, sl);
    const WavePrefix p = slice_prefix<PER>(sl, n_bins, bin0, s_sum);
    const WaveBest r = scan_best<PER>(hf, sl, p, has_missing, scale_g, scale_h, lam, gamma);
    if (lane == 0) {
        s_fb[q] = r.fb;
        s_fb[q].feature = f;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        // slices in bin order: on equal gains the earlier (smaller code) stays
        best[(int64_t)node * gridDim.x + blockIdx.x] = block_feature_best(s_fb, kSliceWaves);
        if (f == 0) { totals[2 * node] = r.G; totals[2 * node + 1] = r.H; }
    }
}

// The fused level tail for wide bins: one (pair, feature) per block of
// kSliceWaves waves, each wave a slice of both children.
template <int PER>
__global__ __launch_bounds__(kSliceWaves * kWave) void k_subtract_split_sliced(
    const long long* __restrict__ parent, long long* __restrict__ child, const int32_t* __restrict__ plan,
    const SubtractInline inl, int n_features, int n_bins, int S, int has_missing,
    const double* __restrict__ inv_scale, double lam, double gamma, FeatureBest* __restrict__ best,
    long long* __restrict__ totals)
{
    const double scale_g = inv_scale[0], scale_h = inv_scale[1];   // 2^-k, from k_max_final
    __shared__ long long s_sum[2][2 * kSliceWaves];
    __shared__ FeatureBest s_fb[2][kSliceWaves];   // [0] the built child, [1] the other
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x / kWave;
    const int f = blockIdx.x;
    const int pair = blockIdx.y;
    const int32_t pslot = plan ? plan[2 * pair] : inl.v[2 * pair];
    const int r = plan ? plan[2 * pair + 1] : inl.v[2 * pair + 1];
    const int nb = 2 * pair + r, no = 2 * pair + 1 - r;
    const int64_t fs = (int64_t)S * 2;
    const long long* hp = parent + ((int64_t)pslot * n_features + f) * fs;
    const long long* hb = child + ((int64_t)nb * n_features + f) * fs;
    long long* ho = child + ((int64_t)no * n_features + f) * fs;
    const int bin0 = q * kWave * PER;
    LaneSlots<PER> so, sb;
    load_slice_slots<PER>(hp, n_bins, has_missing, bin0, so);
    load_slice_slots<PER>(hb, n_bins, has_missing, bin0, sb);
#pragma unroll
    for (int j = 0; j < PER; ++j) so.v[j] = make_longlong2(so.v[j].x - sb.v[j].x, so.v[j].y - sb.v[j].y);
    so.miss = make_longlong2(so.miss.x - sb.miss.x, so.miss.y - sb.miss.y);
    longlong2* o2 = (longlong2*)ho;
    const int b0 = bin0 + lane * PER;
#pragma unroll
    for (int j = 0; j < PER; ++j)
        if (b0 + j < n_bins) o2[b0 + j] = so.v[j];
    if (has_missing && threadIdx.x == 0) o2[n_bins] = so.miss;
    const WavePrefix pb = slice_prefix<PER>(sb, n_bins, bin0, s_sum[0]);
    const WavePrefix po = slice_prefix<PER>(so, n_bins, bin0, s_sum[1]);
    const WaveBest wb = scan_best<PER>(hb, sb, pb, has_missing, scale_g, scale_h, lam, gamma);
    const WaveBest wo = scan_best<PER>(ho, so, po, has_missing, scale_g, scale_h, lam, gamma);
    if (lane == 0) {
        s_fb[0][q] = wb.fb;
        s_fb[0][q].feature = f;
        s_fb[1][q] = wo.fb;
        s_fb[1][q].feature = f;
    }
    __syncthreads();
    if (threadIdx.x < 2)
        best[(int64_t)(threadIdx.x == 0 ? nb : no) * gridDim.x + blockIdx.x] =
            block_feature_best(s_fb[threadIdx.x], kSliceWaves);
    if (threadIdx.x == 0 && f == 0) {
        totals[2 * nb] = wb.G;
        totals[2 * nb + 1] = wb.H;
        totals[2 * no] = wo.G;
        totals[2 * no + 1] = wo.H;
    }
}

struct SplitOut {
    int32_t feature, bin, default_left, pad;
    double gain;
    long long g_left, h_left, g_total, h_total;
};

// A node's record: no candidate (f < 0) reads feature and bin -1, gain -inf.
__device__ inline void split_out_write(SplitOut* out, int node, int f, int code, double gain, long long gl,
                                       long long hl, long long tg, long long th)
{
    SplitOut o;
    o.pad = 0;
    o.g_total = tg;
    o.h_total = th;
    if (f < 0) {
        o.feature = -1; o.bin = -1; o.default_left = 0;
        o.gain = -__builtin_inf();
        o.g_left = 0; o.h_left = 0;
    } else {
        o.feature = f;
        o.bin = code >> 1;
        o.default_left = code & 1;
        o.gain = gain;
        o.g_left = gl;
        o.h_left = hl;
    }
    out[node] = o;
}

// k_split_reduce for at most kWave entries: lane e holds entry e, and the
// lanes exchange (gain, feature) with the winner's record through xor
// shuffles, 32 apart first.  Lane 0 then has combined the same pairs, in the
// same order and orientation, as the block-wide tree below does with one
// wave, so it picks the same entry; the record needs no second load.
__device__ inline void split_reduce_wave(const FeatureBest* __restrict__ nb, const long long* __restrict__ totals,
                                         int n_entries, int node, SplitOut* __restrict__ out)
{
    const int lane = (int)threadIdx.x;
    const long long tg = totals[2 * node], th = totals[2 * node + 1];
    double bg = 0.0;
    int bf = -1, code = -1;
    long long gl = 0, hl = 0;
    if (lane < n_entries) {
        const FeatureBest c = nb[lane];
        if (c.code >= 0) {
            bg = c.gain;
            bf = c.feature;
            code = c.code;
            gl = c.g_left;
            hl = c.h_left;
        }
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const double og = __shfl_xor(bg, off, kWave);
        const int of = __shfl_xor(bf, off, kWave);
        const int oc = __shfl_xor(code, off, kWave);
        const long long ogl = __shfl_xor(gl, off, kWave);
        const long long ohl = __shfl_xor(hl, off, kWave);
        if (better(og, of, bg, bf)) {
            bg = og;
            bf = of;
            code = oc;
            gl = ogl;
            hl = ohl;
        }
    }
    if (lane == 0) split_out_write(out, node, bf, code, bg, gl, hl, tg, th);
}

// One block per node (64, 256 or 1,024 threads, a power of two): the best feature,
// scanning features in order per thread -- four entries loaded before any is
// compared -- and then reducing across threads with the same (gain, feature)
// order.  (kSplitReduceMaxThreads: hgb_layout.h)
__global__ __launch_bounds__(kSplitReduceMaxThreads) void k_split_reduce(
    const FeatureBest* __restrict__ best, const long long* __restrict__ totals, int n_entries,
    SplitOut* __restrict__ out)
{
    __shared__ double s_gain[kSplitReduceMaxThreads];
    __shared__ int s_feat[kSplitReduceMaxThreads];
    __shared__ int s_entry[kSplitReduceMaxThreads];
    const int node = blockIdx.x;
    const FeatureBest* nb = best + (int64_t)node * n_entries;
    if (blockDim.x == kWave && n_entries <= kWave) {   // one wave, at most one entry per lane
        split_reduce_wave(nb, totals, n_entries, node, out);
        return;
    }
    double bg = 0.0;
    int bf = -1, be = -1;
    auto take = [&](const FeatureBest& c, int e) {
        if (c.code < 0) return;
        if (bf < 0 || c.gain > bg) { bg = c.gain; bf = c.feature; be = e; }
    };
    const int bd = (int)blockDim.x;
    int e = threadIdx.x;   // entries in feature order
    for (; e + 3 * bd < n_entries; e += 4 * bd) {
        FeatureBest c[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) c[u] = nb[e + u * bd];
#pragma unroll
        for (int u = 0; u < 4; ++u) take(c[u], e + u * bd);
    }
    for (; e < n_entries; e += bd) take(nb[e], e);
    s_gain[threadIdx.x] = bg;
    s_feat[threadIdx.x] = bf;
    s_entry[threadIdx.x] = be;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            double og = s_gain[threadIdx.x + w];
            int of = s_feat[threadIdx.x + w];
            if (better(og, of, s_gain[threadIdx.x], s_feat[threadIdx.x])) {
                s_gain[threadIdx.x] = og;
                s_feat[threadIdx.x] = of;
                s_entry[threadIdx.x] = s_entry[threadIdx.x + w];
            }
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        const int f = s_feat[0];
        if (f < 0) {
            split_out_write(out, node, -1, -1, 0.0, 0, 0, totals[2 * node], totals[2 * node + 1]);
        } else {
            const FeatureBest c = nb[s_entry[0]];
            split_out_write(out, node, f, c.code, c.gain, c.g_left, c.h_left, totals[2 * node],
                            totals[2 * node + 1]);
        }
    }
}

// ---------------------------------------------------------------------------
// find_level_split: one (feature, bin, direction) for every node of a level
// (the oblivious tree).  A candidate's level score is the sum, in node order
// from 0.0, of its gain in each node where it is valid; a floating-point sum
// depends on its order, so the three passes keep that order exactly:
//   k_level_gain   one wave per (node, feature): the gain of every candidate
//                  in that node (-inf where invalid) into terms[node][c], with
//                  c = (feature * n_bins + bin) * n_dirs + direction;
//   k_level_sum    one thread per candidate: its terms added node by node,
//                  then a block argmax (larger score, then smaller c);
//   k_level_pick   one block: the argmax over the block winners, into the
//                  level's record;
//   k_level_records  one wave per node: the node's record under the level's
//                  split, and the level record's integer sums.
// ---------------------------------------------------------------------------
struct LevelBest {
    double score;
    int32_t code;    // candidate index c; -1 when no candidate in the block
    int32_t pad;
};

template <int PER>
__global__ __launch_bounds__(256) void k_level_gain(const long long* __restrict__ hist, int n_features,
                                                    int n_bins, int S, int has_missing,
                                                    const double* __restrict__ inv_scale, double lam, double gamma,
                                                    double* __restrict__ terms)
{
    const double scale_g = inv_scale[0], scale_h = inv_scale[1];   // 2^-k, from k_max_final
    const int f = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    const int node = blockIdx.y;
    if (f >= n_features) return;
    const long long* hf = hist + ((int64_t)node * n_features + f) * (int64_t)S * 2;
    LaneSlots<PER> s;
    load_lane_slots<PER>(hf, n_bins, has_missing, s);
    const WavePrefix p = wave_prefix<PER>(hf, s, n_bins);
    const double g = (double)p.G * scale_g;
    const double h = (double)p.H * scale_h;
    const double parent = g * g / (h + lam);
    const int n_dirs = has_missing ? 2 : 1;
    const int64_t n_cand = (int64_t)n_features * n_bins * n_dirs;
    double* out = terms + (int64_t)node * n_cand + (int64_t)f * n_bins * n_dirs;
    prefix_visit<PER>(hf, s, p, [&](int b, long long pg, long long ph) {
        for (int d = 0; d < n_dirs; ++d) {
            const long long GL = pg + (d ? s.miss.x : 0);
            const long long HL = ph + (d ? s.miss.y : 0);
            const long long GR = p.G - GL;
            const long long HR = p.H - HL;
            double t = -__builtin_inf();
            if (HL > 0 && HR > 0)
                t = split_gain((double)GL * scale_g, (double)HL * scale_h, (double)GR * scale_g,
                               (double)HR * scale_h, parent, lam, gamma);
            out[b * n_dirs + d] = t;
        }
    });
}

__device__ inline void block_argmax(double& score, int& code, double* s_score, int* s_code)
{
    s_score[threadIdx.x] = score;
    s_code[threadIdx.x] = code;
    __syncthreads();
    for (int w = blockDim.x / 2; w > 0; w >>= 1) {
        if (threadIdx.x < w) {
            const double os = s_score[threadIdx.x + w];
            const int oc = s_code[threadIdx.x + w];
            if (better(os, oc, s_score[threadIdx.x], s_code[threadIdx.x])) {
                s_score[threadIdx.x] = os;
                s_code[threadIdx.x] = oc;
            }
        }
        __syncthreads();
    }
    score = s_score[0];
    code = s_code[0];
}

__global__ __launch_bounds__(256) void k_level_sum(const double* __restrict__ terms, int n_nodes,
                                                   int64_t n_cand, LevelBest* __restrict__ block_best)
{
    __shared__ double s_score[256];
    __shared__ int s_code[256];
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    double score = 0.0;
    int code = -1;
    if (c < n_cand) {
        bool any = false;
        const double* t = terms + c;
#pragma unroll 8
        for (int n = 0; n < n_nodes; ++n) {
            const double v = t[(int64_t)n * n_cand];
            if (v != -__builtin_inf()) {
                score += v;
                any = true;
            }
        }
        code = any ? (int)c : -1;
    }
    block_argmax(score, code, s_score, s_code);
    if (threadIdx.x == 0) {
        LevelBest r;
        r.score = code < 0 ? -__builtin_inf() : score;
        r.code = code;
        r.pad = 0;
        block_best[blockIdx.x] = r;
    }
}


// The winner: block results scanned in order per thread, then the block
// argmax.  Writes the level record (its integer sums zeroed, for
// k_level_records to add into).
__global__ __launch_bounds__(256) void k_level_pick(const LevelBest* __restrict__ block_best, int n_blocks,
                                                    int n_bins, int n_dirs, SplitOut* __restrict__ level)
{
    __shared__ double s_score[256];
    __shared__ int s_code[256];
    double score = 0.0;
    int code = -1;
    for (int i = threadIdx.x; i < n_blocks; i += blockDim.x) {
        const LevelBest r = block_best[i];
        if (better(r.score, r.code, score, code)) {
            score = r.score;
            code = r.code;
        }
    }
    block_argmax(score, code, s_score, s_code);
    if (threadIdx.x == 0) {
        SplitOut o;
        o.feature = code < 0 ? -1 : code / (n_bins * n_dirs);
        o.bin = code < 0 ? -1 : (code / n_dirs) % n_bins;
        o.default_left = code < 0 ? 0 : code % n_dirs;
        o.pad = 0;
        o.gain = code < 0 ? -__builtin_inf() : score;
        o.g_left = 0;
        o.h_left = 0;
        o.g_total = 0;
        o.h_total = 0;
        *level = o;
    }
}

// Every node's record under the level's split (one wave per node), and the
// level record's integer sums: per block in registers and LDS, then one
// atomic add per field per block (integer sums: any order gives the same).
__global__ __launch_bounds__(256) void k_level_records(const long long* __restrict__ hist,
                                                       const double* __restrict__ terms, int n_nodes,
                                                       int n_features, int n_bins, int S, int has_missing,
                                                       SplitOut* __restrict__ out)
{
    __shared__ long long s_sum[256 / kWave][4];
    SplitOut* level = out + n_nodes;
    const int f = level->feature;
    const int b = level->bin;
    const int d = level->default_left;
    const int n_dirs = has_missing ? 2 : 1;
    const int64_t n_cand = (int64_t)n_features * n_bins * n_dirs;
    const int code = f < 0 ? -1 : (f * n_bins + b) * n_dirs + d;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int waves = (int)(blockDim.x / kWave);
    long long acc[4] = {0, 0, 0, 0};   // g_left, h_left, g_total, h_total over this wave's nodes
    for (int node = blockIdx.x * waves + wv; node < n_nodes; node += gridDim.x * waves) {
        const long long* hn = hist + (int64_t)node * n_features * S * 2;
        long long t[4] = {0, 0, 0, 0};
        for (int j = lane; j < S; j += kWave) {   // totals: feature 0's slots
            t[2] += hn[2 * j];
            t[3] += hn[2 * j + 1];
        }
        if (code >= 0) {
            const long long* hf = hn + (int64_t)f * S * 2;
            for (int j = lane; j <= b; j += kWave) {
                t[0] += hf[2 * j];
                t[1] += hf[2 * j + 1];
            }
            if (d && lane == 0) {
                t[0] += hf[2 * n_bins];
                t[1] += hf[2 * n_bins + 1];
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) t[k] = wave_sum_i64(t[k]);
        if (lane == 0) {
            SplitOut o;
            o.feature = f;
            o.bin = b;
            o.default_left = d;
            o.pad = 0;
            if (code < 0) {
                o.gain = -__builtin_inf();
            } else {
                const double v = terms[(int64_t)node * n_cand + code];
                o.gain = v == -__builtin_inf() ? 0.0 : v;
            }
            o.g_left = t[0];
            o.h_left = t[1];
            o.g_total = t[2];
            o.h_total = t[3];
            out[node] = o;
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += t[k];
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) s_sum[wv][k] = acc[k];
    }
    __syncthreads();
    if (threadIdx.x < 4) {
        long long v = 0;
        for (int w = 0; w < waves; ++w) v += s_sum[w][threadIdx.x];
        long long* dst = &level->g_left + threadIdx.x;   // g_left, h_left, g_total, h_total
        atomicAdd((unsigned long long*)dst, (unsigned long long)v);
    }
}

// ---------------------------------------------------------------------------
// partition_level: route each split node's rows to its two children, keeping
// their order (a stable partition), children 2j / 2j + 1 of the j-th node with
// a split.  Three passes over fixed-size chunks of each node's rows: count the
// rows going left per chunk; scan the counts per node and the output extents
// over nodes; scatter each row to its place.
// (kPartThreads, kPartChunk, PartItem: hgb_layout.h)
// ---------------------------------------------------------------------------

__device__ inline bool part_left(int v, int n_bins, const SplitOut& sp)
{
    return v == n_bins ? sp.default_left != 0 : v <= sp.bin;
}

// Each thread takes kPartRows positions of its chunk (kPartThreads threads x
// kPartRows = kPartChunk), position begin + j * kPartThreads + thread at its
// j-th step, so that every index load and direction store of a wave is one
// contiguous run; loads are issued independently and clamped into the chunk.
constexpr int kPartRows = 8;
static_assert(kPartChunk == kPartThreads * kPartRows, "a chunk is one pass of a block");

// Count the rows going left per chunk, and record each position's direction
// (1 = left) for the scatter.  NT reads the split features' bins with
// non-temporal loads: when the nodes split on many features those scattered
// lines are read once and would only push the next level fill's rows out of
// the caches; when they share one feature (an oblivious level) the lines are
// read again by other chunks and stay cached.
template <typename BinT, bool NT>
__global__ __launch_bounds__(kPartThreads) void k_part_count(const BinT* __restrict__ bins, int64_t n, int n_bins,
                                                     int S, const int32_t* __restrict__ rot,
                                                     const int32_t* __restrict__ row_index,
                                                     const PartItem* __restrict__ items,
                                                     const SplitOut* __restrict__ splits,
                                                     int32_t* __restrict__ cnt, uint8_t* __restrict__ flags,
                                                     uint32_t* __restrict__ err)
{
    __shared__ int s_sum[kPartThreads / kWave];
    const PartItem it = items[blockIdx.x];
    // The row indices do not depend on the split: they are loaded while the
    // split record is on its way, and nothing branches on the split (a node
    // without one reads feature 0's column and sends every row right), so the
    // compiler keeps the loads ahead of it.  Positions in 64 bits: a chunk may
    // end within kPartChunk of 2^31.
    const int64_t k0 = (int64_t)it.begin + threadIdx.x;
    const int64_t kstep = blockDim.x;
    int64_t r[kPartRows];
#pragma unroll
    for (int j = 0; j < kPartRows; ++j) {
        const int64_t kc = min(k0 + j * kstep, (int64_t)it.end - 1);
        r[j] = row_index ? (int64_t)row_index[kc] : kc;
    }
    const SplitOut sp = splits[it.node];
    const bool has = sp.feature >= 0;   // uniform
    const int fe = has ? sp.feature : 0;
    const BinT* col = bins + (int64_t)fe * n;
    const int rf = rot[fe];   // stored values are rotated per feature
    int v[kPartRows];
    bool bad = false;
#pragma unroll
    for (int j = 0; j < kPartRows; ++j) {
        const bool in = (uint64_t)r[j] < (uint64_t)n;
        bad |= has && !in && k0 + j * kstep < it.end;
        const BinT* at = col + (in ? r[j] : 0);
        v[j] = unrotate((int)(NT ? __builtin_nontemporal_load(at) : *at), rf, S);
    }
    int c = 0;
#pragma unroll
    for (int j = 0; j < kPartRows; ++j) {
        const int64_t k = k0 + j * kstep;
        // a row index outside [0, n) is routed right (and reported)
        const bool left = has && (uint64_t)r[j] < (uint64_t)n && part_left(v[j], n_bins, sp);
        if (k < it.end) {
            c += left ? 1 : 0;
            flags[k] = left ? 1 : 0;
        }
    }
    if (bad) atomicOr(err, kErrRowIndex);
    for (int off = kWave / 2; off > 0; off >>= 1) c += __shfl_xor(c, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_sum[threadIdx.x / kWave] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
        int t = 0;
        for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += s_sum[w];
        cnt[blockIdx.x] = t;
    }
}

// The block's results for the host are in pinned memory: every thread makes
// its own stores visible system-wide, then thread 0 stores the sequence
// number the host waits for.  Every thread calls.
__device__ inline void publish_seq(uint32_t* host_seq, uint32_t seq)
{
    __threadfence_system();
    __syncthreads();
    if (threadIdx.x == 0) *host_seq = seq;
}

// Block-wide exclusive scan of v (blockDim.x values, a multiple of 64 up to
// 1,024), returning this thread's prefix; *total receives the sum.  Each wave
// scans its 64 values with shuffles, wave 0 scans the waves' totals, and three
// barriers serve the whole block (a scan through LDS alone takes two per
// doubling step, twenty for 1,024 threads).  Uses s[blockDim.x / 64].
__device__ inline int block_exclusive_scan(int v, int* s, int* total)
{
    const int lane = (int)(threadIdx.x & (kWave - 1)), w = (int)(threadIdx.x / kWave);
    const int nw = (int)(blockDim.x / kWave);
    int x = v;
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(x, d, kWave);
        if (lane >= d) x += y;
    }
    if (lane == kWave - 1) s[w] = x;   // the wave's total
    __syncthreads();
    if (w == 0) {
        int t = lane < nw ? s[lane] : 0;
        for (int d = 1; d < kWave; d <<= 1) {
            const int y = __shfl_up(t, d, kWave);
            if (lane >= d) t += y;
        }
        if (lane < nw) s[lane] = t;    // the waves' inclusive prefixes
    }
    __syncthreads();
    const int before = w > 0 ? s[w - 1] : 0;
    *total = s[nw - 1];
    __syncthreads();   // s is free again for the next call
    return before + x - v;
}

// One block.  left_base[item]: rows going left in the node's earlier chunks.
// node_out[3 i + 0..2]: the node's first output position (its children's
// rows follow those of earlier split nodes), its rows going left, and 1 when
// it has a split.  The per-chunk counts are scanned across all chunks, then
// rebased to each node's first chunk.
__global__ __launch_bounds__(1024) void k_part_scan(const int32_t* __restrict__ cnt,
                                                    const PartItem* __restrict__ items, int n_items,
                                                    const int32_t* __restrict__ first_item,
                                                    const int32_t* __restrict__ offsets,
                                                    const SplitOut* __restrict__ splits, int n_nodes,
                                                    int32_t* __restrict__ left_base,
                                                    int32_t* __restrict__ node_out,
                                                    int32_t* __restrict__ host_out,
                                                    const uint32_t* __restrict__ err_dev,
                                                    uint32_t* __restrict__ err_host,
                                                    uint32_t* __restrict__ host_seq, uint32_t seq)
{
    __shared__ int s_scan[1024];
    int carry = 0, tot = 0;
    for (int base = 0; base < n_items; base += blockDim.x) {   // exclusive scan of the counts
        const int j = base + threadIdx.x;
        const int v = j < n_items ? cnt[j] : 0;
        const int ex = block_exclusive_scan(v, s_scan, &tot);
        if (j < n_items) left_base[j] = carry + ex;
        carry += tot;
    }
    const int all = carry;
    __syncthreads();
    for (int i = threadIdx.x; i < n_nodes; i += blockDim.x) {
        const int f0 = first_item[i], f1 = first_item[i + 1];
        const int e0 = f0 < n_items ? left_base[f0] : all;
        const int e1 = f1 < n_items ? left_base[f1] : all;
        node_out[3 * i] = e0;   // the node's base, for the rebase below
        node_out[3 * i + 1] = e1 - e0;
        node_out[3 * i + 2] = splits[i].feature >= 0 ? 1 : 0;
    }
    __syncthreads();
    for (int j = threadIdx.x; j < n_items; j += blockDim.x) left_base[j] -= node_out[3 * items[j].node];
    __syncthreads();
    carry = 0;
    for (int base = 0; base < n_nodes; base += blockDim.x) {   // output extents over nodes
        const int i = base + threadIdx.x;
        const int v = i < n_nodes && node_out[3 * i + 2] ? offsets[i + 1] - offsets[i] : 0;
        const int ex = block_exclusive_scan(v, s_scan, &tot);
        if (i < n_nodes) node_out[3 * i] = carry + ex;
        carry += tot;
    }
    // the node records and the count pass's error word straight into pinned
    // host memory, then the level's number once they are visible (the host
    // waits for it)
    __syncthreads();
    for (int i = threadIdx.x; i < 3 * n_nodes; i += blockDim.x) host_out[i] = node_out[i];
    if (threadIdx.x == 0) *err_host = *err_dev;
    publish_seq(host_seq, seq);
}

// k_part_scan for a level of at most MAXI chunks and MAXN nodes, by one block
// of 1,024 threads: the same outputs, from one round of loads issued together
// (each thread's counts and node records, held in registers until all are
// issued, then put in LDS), with the scans, the rebase and each chunk's node
// (a binary search of the nodes' first chunks) done in LDS.  A single block
// pays every global round trip in full; the chunk records themselves (in
// pinned host memory) are not read at all.
template <int MAXI, int MAXN>
__global__ __launch_bounds__(1024) void k_part_scan_lds(const int32_t* __restrict__ cnt, int n_items,
                                                        const int32_t* __restrict__ first_item,
                                                        const int32_t* __restrict__ offsets,
                                                        const SplitOut* __restrict__ splits, int n_nodes,
                                                        int32_t* __restrict__ left_base,
                                                        int32_t* __restrict__ node_out,
                                                        int32_t* __restrict__ host_out,
                                                        const uint32_t* __restrict__ err_dev,
                                                        uint32_t* __restrict__ err_host,
                                                        uint32_t* __restrict__ host_seq, uint32_t seq)
{
    constexpr int kT = 1024;
    constexpr int IP = MAXI / kT, NP = MAXN / kT;   // entries per thread
    static_assert(IP * kT == MAXI && NP * kT == MAXN, "whole passes of the block");
    __shared__ int s_ex[MAXI];         // the counts, then their exclusive scan
    __shared__ int s_first[MAXN + 1];  // each node's first chunk
    __shared__ int s_rows[MAXN];       // each node's rows, -1 without a split
    __shared__ int s_scan[kT];
    const int t = threadIdx.x;
    int c[IP], fi[NP], o0[NP], o1[NP], ft[NP];
#pragma unroll
    for (int u = 0; u < IP; ++u) {
        const int j = t + u * kT;
        c[u] = j < n_items ? cnt[j] : 0;
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int i = t + u * kT;
        const bool in = i < n_nodes;
        fi[u] = in ? first_item[i] : 0;
        o0[u] = in ? offsets[i] : 0;
        o1[u] = in ? offsets[i + 1] : 0;
        ft[u] = in ? splits[i].feature : -1;
    }
    const int fi_last = t == 0 ? first_item[n_nodes] : 0;
#pragma unroll
    for (int u = 0; u < IP; ++u) s_ex[t + u * kT] = c[u];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
        const int i = t + u * kT;
        if (i < n_nodes) {
            s_first[i] = fi[u];
            s_rows[i] = ft[u] >= 0 ? o1[u] - o0[u] : -1;
        }
    }
    if (t == 0) s_first[n_nodes] = fi_last;
    __syncthreads();
    int carry = 0, tot = 0;
    for (int base = 0; base < n_items; base += kT) {   // exclusive scan of the counts
        const int j = base + t;
        const int v = j < n_items ? s_ex[j] : 0;
        const int ex = block_exclusive_scan(v, s_scan, &tot);   // (its barriers order the writes below)
        if (j < n_items) s_ex[j] = carry + ex;
        carry += tot;
    }
    const int all = carry;
    __syncthreads();
    // rows going left in the node's earlier chunks; chunk j's node is the
    // last node whose first chunk is at most j (empty nodes own no chunk)
    for (int j = t; j < n_items; j += kT) {
        int lo = 0, hi = n_nodes - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_first[mid] <= j) lo = mid;
            else hi = mid - 1;
        }
        left_base[j] = s_ex[j] - s_ex[s_first[lo]];
    }
    carry = 0;
    for (int base = 0; base < n_nodes; base += kT) {   // output extents over nodes
        const int i = base + t;
        const int v = i < n_nodes && s_rows[i] > 0 ? s_rows[i] : 0;
        const int ex = block_exclusive_scan(v, s_scan, &tot);
        if (i < n_nodes) {
            const int f0 = s_first[i], f1 = s_first[i + 1];
            const int e0 = f0 < n_items ? s_ex[f0] : all;
            const int e1 = f1 < n_items ? s_ex[f1] : all;
            const int rec[3] = {carry + ex, e1 - e0, s_rows[i] >= 0 ? 1 : 0};
            for (int k = 0; k < 3; ++k) {
                node_out[3 * i + k] = rec[k];
                host_out[3 * i + k] = rec[k];   // pinned host memory: the host reads it after the stream passes
            }
        }
        carry += tot;
    }
    if (t == 0) *err_host = *err_dev;
    publish_seq(host_seq, seq);
}

// Write each row to its place: the chunk's left rows from its left base on,
// its right rows from its right base on, in position order.  Step j covers
// positions begin + j * kPartThreads .. + kPartThreads - 1: a lane's rank
// among the step's left (right) rows is its wave's ballot below it plus the
// counts of every (step, wave) before its own in position order.  Every wave
// publishes its counts of all steps at once; wave 0 turns the 64 (step,
// wave) counts into exclusive prefixes with one shuffle scan, so each lane
// reads two prefixes per step.  The stores of a wave's left (right) rows in
// one step are one contiguous run.
__global__ __launch_bounds__(kPartThreads) void k_part_scatter(const int32_t* __restrict__ row_index,
                                                       const PartItem* __restrict__ items,
                                                       const SplitOut* __restrict__ splits,
                                                       const uint8_t* __restrict__ flags,
                                                       const int32_t* __restrict__ left_base,
                                                       const int32_t* __restrict__ node_out,
                                                       int32_t* __restrict__ out_rows)
{
    constexpr int kWaves = kPartThreads / kWave;
    static_assert(kPartRows * kWaves == kWave, "one lane of wave 0 per (step, wave)");
    __shared__ int s_left[kPartRows * kWaves];   // per (step, wave): its left rows, then those before it
    __shared__ int s_all[kPartRows * kWaves];    // the same for all its rows
    const PartItem it = items[blockIdx.x];
    // Every load below depends on the chunk record alone, so all of them are
    // in flight together; a node without a split (no children) stores nothing.
    const bool has = splits[it.node].feature >= 0;   // uniform
    const int lb = left_base[blockIdx.x];
    const int base = node_out[3 * it.node];
    const int n_left = node_out[3 * it.node + 1];
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int wv = (int)(threadIdx.x / kWave);
    const int64_t k0 = (int64_t)it.begin + threadIdx.x;   // 64 bits: see k_part_count
    const int64_t kstep = blockDim.x;
    int32_t r[kPartRows];
    uint8_t f[kPartRows];
#pragma unroll
    for (int j = 0; j < kPartRows; ++j) {
        const int64_t kc = min(k0 + j * kstep, (int64_t)it.end - 1);
        r[j] = row_index ? row_index[kc] : (int32_t)kc;
        f[j] = flags[kc];
    }
    uint64_t bl[kPartRows], bi[kPartRows];   // per step: the wave's left rows, its rows
#pragma unroll
    for (int j = 0; j < kPartRows; ++j) {
        const bool in = has && k0 + j * kstep < it.end;
        bl[j] = __ballot(in && f[j] != 0);
        bi[j] = __ballot(in);
        if (lane == 0) {
            s_left[j * kWaves + wv] = __popcll(bl[j]);
            s_all[j * kWaves + wv] = __popcll(bi[j]);
        }
    }
    __syncthreads();
    if (wv == 0) {
        const int l = s_left[lane], a = s_all[lane];
        int xl = l, xa = a;
        for (int d = 1; d < kWave; d <<= 1) {
            const int yl = __shfl_up(xl, d, kWave), ya = __shfl_up(xa, d, kWave);
            if (lane >= d) {
                xl += yl;
                xa += ya;
            }
        }
        s_left[lane] = xl - l;
        s_all[lane] = xa - a;
    }
    __syncthreads();
    const int lbase = base + lb;                                   // the chunk's first left slot
    const int rbase = base + n_left + (it.begin - it.node_begin - lb);   // and its first right slot
    const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kPartRows; ++j) {
        const int pl = s_left[j * kWaves + wv], pa = s_all[j * kWaves + wv];
        if ((bi[j] >> lane) & 1ull) {
            if ((bl[j] >> lane) & 1ull)
                out_rows[lbase + pl + __popcll(bl[j] & below)] = r[j];
            else
                out_rows[rbase + (pa - pl) + __popcll(bi[j] & ~bl[j] & below)] = r[j];
        }
    }
}

}  // namespace hgb
