// stream_ceiling.hip -- calibration kernels for the bandwidth rooflines that
// the benchmark reports; built into its own libkda_stream.so, not into the KDA
// library.
//
// A streaming copy (16-byte nontemporal loads and stores, one per thread) and
// a streaming read (16-byte loads summed in registers) over a buffer much
// larger than the 256 MiB Infinity Cache measure what HBM sustains on this
// part for a 1:1 read/write mix and for reads alone.  A bandwidth-bound KDA
// kernel is then reported both against the published 8 TB/s and against the
// rate a kernel with nothing to compute reaches.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
// One 16-byte element per thread: measured over 1 GiB buffers, the copy moves
// 6.5 TB/s this way against 6.1 with two per thread, 6.2 with four and 4.4
// with eight, and 5.6-5.9 as a grid-stride loop.
constexpr int kPerThread = 1;

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const f32x4* __restrict__ a, f32x4* __restrict__ b,
                                                               int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * (kThreads * kPerThread) + threadIdx.x;
    f32x4 v[kPerThread];
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
        if (i + u * kThreads < n) v[u] = __builtin_nontemporal_load(a + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
        if (i + u * kThreads < n) __builtin_nontemporal_store(v[u], b + i + u * kThreads);
}

// The sum is stored only when it equals a value no finite input sum hits by
// chance in practice, so that the loads are not removed and nothing is written.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const f32x4* __restrict__ a, float* __restrict__ sink,
                                                               int64_t n) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * (kThreads * kPerThread) + threadIdx.x;
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kPerThread; ++u)
        if (i + u * kThreads < n) {
            const f32x4 v = a[i + u * kThreads];
            s += v[0] + v[1] + v[2] + v[3];
        }
    if (s == -1.2345678e30f) sink[threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to
// dst on `stream` (a hipStream_t, null for the default stream).  Returns 0, or
// the HIP error code of the launch; 1 for a size or alignment it refuses.
int kda_stream_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16) return 1;
    const int64_t n = bytes / 16;
    const int64_t grid = (n + kThreads * kPerThread - 1) / (kThreads * kPerThread);
    if (grid == 0) return 0;
    if (grid > INT32_MAX) return 1;
    hipLaunchKernelGGL(stream_copy_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const f32x4*>(src), static_cast<f32x4*>(dst), n);
    return static_cast<int>(hipGetLastError());
}

// Read `bytes` from src; sink (256 floats) is written only in the case the
// kernel's comment describes.  Same conventions as kda_stream_copy.
int kda_stream_read(const void* src, float* sink, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 || !sink) return 1;
    const int64_t n = bytes / 16;
    const int64_t grid = (n + kThreads * kPerThread - 1) / (kThreads * kPerThread);
    if (grid == 0) return 0;
    if (grid > INT32_MAX) return 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), static_cast<const f32x4*>(src), sink, n);
    return static_cast<int>(hipGetLastError());
}

}  // extern "C"
