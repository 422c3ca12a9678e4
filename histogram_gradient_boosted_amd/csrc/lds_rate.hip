// LDS atomic-add rate microbenchmark (gfx950), and the rate of scattered
// line reads (gather_rate_measure, at the end).  The level histogram fill adds
// 64-bit integers into block-private LDS histograms at data-dependent bins, so
// its second ceiling, after HBM, is the rate at which a CU retires LDS atomic
// adds.  This measures that rate for the access patterns the fill produces:
//
//   kind 0  u64 atomic add, uniformly random bin of a 256-bin histogram held in
//           `copies` lane-interleaved copies (word = bin * copies + lane % copies,
//           the fill's layout);
//   kind 1  u64 atomic add, every lane a distinct word (no bank or address
//           conflicts: the conflict-free ceiling);
//   kind 2  u32 atomic add, random bins as kind 0.
//   kind 3  u64 atomic add in the fills' interleaved (slot-major) tile: word =
//           bin * 64 + (lane + k) mod 32 for the k-th add -- two lanes per bank
//           pair whatever the bins -- launched in the fills' shape, one block
//           of 1024 threads and a 128 KB tile per CU (`copies` unused).
//   kind 4  u32 atomic add, every lane a distinct word (the u32 conflict-free
//           ceiling, for comparison with kind 1: a cell split into 32-bit
//           halves would take four of these instead of two u64 adds).
//
// Kinds 0-2 and 4 fill the chip with 8 blocks of 256 threads per CU; each thread
// issues `iters` x 4 adds.  Indices are reduced modulo the allocated word count,
// so every access stays inside the block's LDS allocation.  The result is read
// back into a sink so the adds cannot be elided.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lds_probe {

__device__ inline uint32_t xorshift(uint32_t x)
{
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
}

template <int KIND>
__global__ __launch_bounds__(1024) void k_lds_rate(int iters, int copies, int words, unsigned long long* sink)
{
    extern __shared__ unsigned long long lds[];
    uint32_t* l32 = (uint32_t*)lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    for (int i = tid; i < words; i += blockDim.x) lds[i] = 0;
    __syncthreads();
    uint32_t s = 0x9e3779b9u * (uint32_t)(blockIdx.x * blockDim.x + tid + 1);
    const uint32_t cm = (uint32_t)copies - 1;
    const uint32_t wm = (uint32_t)words - 1;        // words is a power of two
    for (int it = 0; it < iters; ++it) {
        s = xorshift(s);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t b = (s >> (8 * k)) & 255u;
            if (KIND == 0) atomicAdd(&lds[(b * (uint32_t)copies + ((uint32_t)lane & cm)) & wm], 3ull);
            if (KIND == 1) atomicAdd(&lds[((uint32_t)lane + 64u * (uint32_t)k) & wm], 3ull);
            if (KIND == 2) atomicAdd(&l32[(b * (uint32_t)copies + ((uint32_t)lane & cm)) & (2 * wm + 1)], 3u);
            if (KIND == 3) atomicAdd(&lds[((b << 6) | (((uint32_t)lane + (uint32_t)k) & 31u)) & wm], 3ull);
            if (KIND == 4) atomicAdd(&l32[((uint32_t)lane + 64u * (uint32_t)k) & (2 * wm + 1)], 3u);
        }
    }
    __syncthreads();
    unsigned long long acc = s;
    for (int i = tid; i < words; i += blockDim.x) acc += lds[i];
    if (acc == 0x123456789abcdefull) sink[0] = acc;   // practically never: keeps the adds live
}

template <int KIND>
hipError_t launch(int iters, int copies, int words, int blocks, int threads, unsigned long long* sink,
                  hipStream_t st)
{
    const size_t bytes = (size_t)words * 8;
    hipError_t e = hipFuncSetAttribute((const void*)k_lds_rate<KIND>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    k_lds_rate<KIND><<<blocks, threads, bytes, st>>>(iters, copies, words, sink);
    return hipGetLastError();
}

// Random 128-byte line reads: every thread reads 16 bytes from each of U
// lines at pseudo-random line indices of a buffer larger than the 256 MB
// Infinity Cache (indices reduced modulo the line count: every read stays in
// the buffer), with all U loads issued before any is used.  The chip's rate
// of scattered line fetches: the ceiling of a gather that touches one line
// per row.
template <int U>
__global__ __launch_bounds__(256) void k_rand_lines(const uint4* __restrict__ buf, uint64_t n_lines, int iters,
                                                    unsigned long long* sink)
{
    uint32_t h = (blockIdx.x * 256u + threadIdx.x) * 2654435761u + 12345u;
    unsigned long long acc = 0;
    for (int it = 0; it < iters; ++it) {
        uint4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            h = h * 1664525u + 1013904223u;
            const uint64_t line = ((uint64_t)h * n_lines) >> 32;   // < n_lines
            v[u] = buf[line * 8];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc += v[u].x ^ v[u].w;
    }
    if (acc == 0x1234567ull) sink[0] = acc;   // practically never: keeps the loads live
}

}  // namespace lds_probe

using namespace lds_probe;

extern "C" {

// Measures lane-level LDS atomic adds per second on `device` for pattern
// `kind` (0 to 4 above) with `copies` in {1, 2, 4, ..., 32}.  Writes the
// rate to *lane_ops_per_s and the number of compute units to *n_cu.  Returns 0
// on success, 1 for bad arguments, 2 for a HIP error.
int lds_rate_measure(int device, int kind, int copies, double* lane_ops_per_s, int* n_cu)
{
    if (!lane_ops_per_s || !n_cu || kind < 0 || kind > 4 || copies < 1 || copies > 32 ||
        (copies & (copies - 1)) != 0)
        return 1;
    if (hipSetDevice(device) != hipSuccess) return 2;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 2;
    *n_cu = prop.multiProcessorCount;
    const bool fill_shape = kind == 3;
    const int blocks = prop.multiProcessorCount * (fill_shape ? 1 : 8);
    const int threads = fill_shape ? 1024 : 256;
    const int iters = 2000;
    // kinds 1, 2 and 4 use kind 0's allocation; kind 3 a 128 KB tile (256 slots x 2
    // planes x 32 positions)
    const int words = fill_shape ? 256 * 64 : 256 * copies;
    unsigned long long* sink = nullptr;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    int rc = 2;
    float ms = 0.0f;
    if (hipMalloc(&sink, 64) != hipSuccess) return 2;
    if (hipStreamCreate(&st) != hipSuccess) goto done;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) goto done;
    for (int rep = 0; rep < 2; ++rep) {   // the first launch warms up
        if (hipEventRecord(a, st) != hipSuccess) goto done;
        hipError_t e = kind == 0   ? launch<0>(iters, copies, words, blocks, threads, sink, st)
                       : kind == 1 ? launch<1>(iters, copies, words, blocks, threads, sink, st)
                       : kind == 2 ? launch<2>(iters, copies, words, blocks, threads, sink, st)
                       : kind == 3 ? launch<3>(iters, copies, words, blocks, threads, sink, st)
                                   : launch<4>(iters, copies, words, blocks, threads, sink, st);
        if (e != hipSuccess) goto done;
        if (hipEventRecord(b, st) != hipSuccess) goto done;
        if (hipEventSynchronize(b) != hipSuccess) goto done;
    }
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess || ms <= 0.0f) goto done;
    *lane_ops_per_s = (double)blocks * threads * (double)iters * 4.0 / (ms * 1e-3);
    rc = 0;
done:
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (st) (void)hipStreamDestroy(st);
    (void)hipFree(sink);
    return rc;
}

// Scattered 128-byte line reads per second on `device` (k_rand_lines over a
// 640 MiB buffer, 8 lines in flight per thread).  Returns 0 on success, 2 for
// a HIP error.
int gather_rate_measure(int device, double* lines_per_s)
{
    if (!lines_per_s) return 1;
    if (hipSetDevice(device) != hipSuccess) return 2;
    const uint64_t bytes = 640ull << 20;
    const uint64_t n_lines = bytes / 128;
    const int blocks = 16384, iters = 4;
    uint4* buf = nullptr;
    unsigned long long* sink = nullptr;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    int rc = 2;
    float ms = 0.0f;
    if (hipMalloc(&buf, bytes) != hipSuccess) return 2;
    if (hipMalloc(&sink, 64) != hipSuccess) goto done;
    if (hipStreamCreate(&st) != hipSuccess) goto done;
    if (hipMemsetAsync(buf, 1, bytes, st) != hipSuccess) goto done;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) goto done;
    for (int rep = 0; rep < 2; ++rep) {   // the first launch warms up
        if (hipEventRecord(a, st) != hipSuccess) goto done;
        k_rand_lines<8><<<blocks, 256, 0, st>>>(buf, n_lines, iters, sink);
        if (hipGetLastError() != hipSuccess) goto done;
        if (hipEventRecord(b, st) != hipSuccess) goto done;
        if (hipEventSynchronize(b) != hipSuccess) goto done;
    }
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess || ms <= 0.0f) goto done;
    *lines_per_s = (double)blocks * 256.0 * iters * 8.0 / (ms * 1e-3);
    rc = 0;
done:
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (st) (void)hipStreamDestroy(st);
    (void)hipFree(sink);
    (void)hipFree(buf);
    return rc;
}

}  // extern "C"
