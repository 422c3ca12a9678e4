// LDS atomic-add rate microbenchmark (gfx950).  The level histogram fill adds
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
//
// Every launch fills the chip (8 blocks of 256 threads per CU) and each thread
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
__global__ __launch_bounds__(256) void k_lds_rate(int iters, int copies, int words, unsigned long long* sink)
{
    extern __shared__ unsigned long long lds[];
    uint32_t* l32 = (uint32_t*)lds;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    for (int i = tid; i < words; i += blockDim.x) lds[i] = 0;
    __syncthreads();
    uint32_t s = 0x9e3779b9u * (uint32_t)(blockIdx.x * 256 + tid + 1);
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
        }
    }
    __syncthreads();
    unsigned long long acc = s;
    for (int i = tid; i < words; i += blockDim.x) acc += lds[i];
    if (acc == 0x123456789abcdefull) sink[0] = acc;   // practically never: keeps the adds live
}

template <int KIND>
hipError_t launch(int iters, int copies, int words, int blocks, unsigned long long* sink, hipStream_t st)
{
    const size_t bytes = (size_t)words * 8;
    hipError_t e = hipFuncSetAttribute((const void*)k_lds_rate<KIND>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return e;
    k_lds_rate<KIND><<<blocks, 256, bytes, st>>>(iters, copies, words, sink);
    return hipGetLastError();
}

}  // namespace lds_probe

using namespace lds_probe;

extern "C" {

// Measures lane-level LDS atomic adds per second on `device` for pattern
// `kind` (0, 1 or 2 above) with `copies` in {1, 2, 4, ..., 32}.  Writes the
// rate to *lane_ops_per_s and the number of compute units to *n_cu.  Returns 0
// on success, 1 for bad arguments, 2 for a HIP error.
int lds_rate_measure(int device, int kind, int copies, double* lane_ops_per_s, int* n_cu)
{
    if (!lane_ops_per_s || !n_cu || kind < 0 || kind > 2 || copies < 1 || copies > 32 ||
        (copies & (copies - 1)) != 0)
        return 1;
    if (hipSetDevice(device) != hipSuccess) return 2;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return 2;
    *n_cu = prop.multiProcessorCount;
    const int blocks = prop.multiProcessorCount * 8;
    const int iters = 2000;
    const int words = 256 * copies;   // kind 1 uses the same allocation
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
        hipError_t e = kind == 0   ? launch<0>(iters, copies, words, blocks, sink, st)
                       : kind == 1 ? launch<1>(iters, copies, words, blocks, sink, st)
                                   : launch<2>(iters, copies, words, blocks, sink, st);
        if (e != hipSuccess) goto done;
        if (hipEventRecord(b, st) != hipSuccess) goto done;
        if (hipEventSynchronize(b) != hipSuccess) goto done;
    }
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess || ms <= 0.0f) goto done;
    *lane_ops_per_s = (double)blocks * 256.0 * iters * 4.0 / (ms * 1e-3);
    rc = 0;
done:
    if (a) (void)hipEventDestroy(a);
    if (b) (void)hipEventDestroy(b);
    if (st) (void)hipStreamDestroy(st);
    (void)hipFree(sink);
    return rc;
}

}  // extern "C"
