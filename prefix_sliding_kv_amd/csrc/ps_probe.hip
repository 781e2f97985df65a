// Measurement probes for the benchmark (libps_probe.so, not part of the
// attention library): the floor a single launch of a given shape can reach
// on this GPU, to set the decode kernel's time beside.
//   * ps_probe_empty: a launch that does nothing (dispatch and completion
//     cost of one dependent launch);
//   * ps_probe_stream_read: every workgroup reads one contiguous share of a
//     byte range with 16-byte loads, eight in flight per lane, and folds
//     them into a value it stores only if it matches an impossible pattern,
//     so nothing but the reads costs time.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ void __launch_bounds__(512) probe_empty_kernel(uint32_t* sink) {
    if (sink == nullptr && threadIdx.x == 1023) sink[0] = 0;
}

__global__ void __launch_bounds__(512) probe_stream_kernel(const uint4* base, size_t n16, uint32_t* sink) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = per * blockIdx.x;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0;
    for (size_t i = lo + threadIdx.x; i < hi; i += 512 * 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = i + u * 512 < hi ? base[i + u * 512] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// One launch of n_wg workgroups of 512 threads that do nothing.  Returns a
// hipError_t (0 = success).
int ps_probe_empty(int32_t n_wg, void* stream) {
    if (n_wg < 1) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_empty_kernel, dim3((unsigned)n_wg), dim3(512), 0, (hipStream_t)stream, nullptr);
    return (int)hipGetLastError();
}

// One launch of n_wg workgroups of 512 threads reading `bytes` (a multiple
// of 16) from device memory at `base` (16-byte aligned); `sink` is a device
// buffer of at least 512 uint32 that is written only by an impossible match.
int ps_probe_stream_read(const void* base, size_t bytes, int32_t n_wg, uint32_t* sink, void* stream) {
    if (!base || !sink || n_wg < 1 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(base) % 16 != 0)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(probe_stream_kernel, dim3((unsigned)n_wg), dim3(512), 0, (hipStream_t)stream,
                       static_cast<const uint4*>(base), bytes / 16, sink);
    return (int)hipGetLastError();
}

}  // extern "C"
