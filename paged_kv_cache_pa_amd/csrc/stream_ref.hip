// stream_ref.hip -- bandwidth reference kernels for the benchmark, built
// into their own library (libpa_stream.so) and not part of the attention
// library's C ABI.  A plain streaming read and a plain copy over HBM, with
// the same 16-byte non-temporal loads the decode kernels use, so a decode or
// copy launch can be read against what a kernel that only moves the bytes
// reaches on the same GPU ([Res] "Attention over scattered blocks" times a
// plain copy kernel beside its attention kernel for the same purpose).
//
// Two access orders: each workgroup streaming one contiguous chunk of the
// buffer, or a grid-stride loop (256 threads, consecutive workgroups on
// consecutive 32 KiB pieces); every thread keeps kUnroll loads in flight.
// Which order and grid size stream fastest differs between them (measured
// on MI355X: both reach ~7.0 TB/s at their best), so the benchmark times a
// set of both and reports the best.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t vec4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 512;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const vec4 *src, int64_t n16,
                                                               int64_t per_wg, uint32_t key,
                                                               vec4 *sink) {
    const int64_t b0 = (int64_t)blockIdx.x * per_wg;
    const int64_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    vec4 acc = {0u, 0u, 0u, 0u};
    int64_t i = b0 + threadIdx.x;
    for (; i + (int64_t)(kUnroll - 1) * kThreads < b1; i += (int64_t)kUnroll * kThreads) {
        vec4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
    }
    for (; i < b1; i += kThreads) acc ^= __builtin_nontemporal_load(src + i);
    // The loads stay live through a data-dependent store that a random key
    // makes practically never happen (sink holds one vector per thread of
    // the first workgroup).
    if (acc.x == key && acc.y == ~key && acc.z == key && acc.w == ~key) sink[threadIdx.x] = acc;
}

constexpr int kStrideThreads = 256;

__global__ __launch_bounds__(kStrideThreads) void stream_read_stride_kernel(const vec4 *src,
                                                                            int64_t n16,
                                                                            uint32_t key,
                                                                            vec4 *sink) {
    const int64_t stride = (int64_t)gridDim.x * kStrideThreads * kUnroll;
    vec4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i0 = (int64_t)blockIdx.x * kStrideThreads * kUnroll + threadIdx.x; i0 < n16;
         i0 += stride) {
        vec4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = i0 + u * kStrideThreads;
            x[u] = i < n16 ? __builtin_nontemporal_load(src + i) : vec4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
    }
    if (acc.x == key && acc.y == ~key && acc.z == key && acc.w == ~key) sink[threadIdx.x] = acc;
}

__global__ __launch_bounds__(kThreads) void stream_copy_kernel(vec4 *dst, const vec4 *src,
                                                               int64_t n16, int64_t per_wg) {
    const int64_t b0 = (int64_t)blockIdx.x * per_wg;
    const int64_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    int64_t i = b0 + threadIdx.x;
    for (; i + (int64_t)(kUnroll - 1) * kThreads < b1; i += (int64_t)kUnroll * kThreads) {
        vec4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(x[u], dst + i + u * kThreads);
    }
    for (; i < b1; i += kThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

int64_t chunk_of(size_t bytes, int workgroups) {
    const int64_t n16 = (int64_t)(bytes / 16);
    return (n16 + workgroups - 1) / workgroups;
}

}  // namespace

extern "C" {

// Threads per workgroup of both kernels (the sink of pa_ref_stream_read
// holds this many 16-byte vectors).
int pa_ref_threads(void) { return kThreads; }

// Reads `bytes` (a multiple of 16, buffer 16-byte aligned) of device memory
// once with `workgroups` workgroups: order 0 = one contiguous chunk per
// workgroup, 1 = grid-stride.  Writes at most pa_ref_threads() 16-byte
// vectors to `sink` (device memory), practically never.  Returns 0 or the
// hipError_t of the launch; 1 (hipErrorInvalidValue) for a bad argument.
int pa_ref_stream_read(const void *src, size_t bytes, int workgroups, int order, uint32_t key,
                       void *sink, void *stream) {
    if (!src || !sink || bytes == 0 || bytes % 16 || ((uintptr_t)src & 15) || workgroups < 1 ||
        workgroups > 65535 * 16 || (order != 0 && order != 1))
        return (int)hipErrorInvalidValue;
    (void)hipGetLastError();
    if (order == 0)
        hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                           (hipStream_t)stream, (const vec4 *)src, (int64_t)(bytes / 16),
                           chunk_of(bytes, workgroups), key, (vec4 *)sink);
    else
        hipLaunchKernelGGL(stream_read_stride_kernel, dim3((unsigned)workgroups),
                           dim3(kStrideThreads), 0, (hipStream_t)stream, (const vec4 *)src,
                           (int64_t)(bytes / 16), key, (vec4 *)sink);
    return (int)hipGetLastError();
}

// Copies `bytes` (a multiple of 16, both buffers 16-byte aligned, not
// overlapping) from src to dst, split over `workgroups` contiguous chunks.
int pa_ref_stream_copy(void *dst, const void *src, size_t bytes, int workgroups, void *stream) {
    if (!src || !dst || bytes == 0 || bytes % 16 || ((uintptr_t)src & 15) || ((uintptr_t)dst & 15) ||
        workgroups < 1 || workgroups > 65535 * 16)
        return (int)hipErrorInvalidValue;
    (void)hipGetLastError();
    hipLaunchKernelGGL(stream_copy_kernel, dim3((unsigned)workgroups), dim3(kThreads), 0,
                       (hipStream_t)stream, (vec4 *)dst, (const vec4 *)src, (int64_t)(bytes / 16),
                       chunk_of(bytes, workgroups));
    return (int)hipGetLastError();
}

}  // extern "C"
