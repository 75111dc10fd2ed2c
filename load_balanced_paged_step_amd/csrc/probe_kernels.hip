// Measurement helpers (declared in hpc_probe.h): HBM streaming-read probe
// and a plain 16-byte copy.  Every access is within [0, bytes) of the
// caller's buffers.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hpc_decode.h"
#include "hpc_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeUnroll = 8;   // 16-byte loads in flight per thread

// Workgroup g streams the contiguous chunk [g * per, (g + 1) * per) of 16-byte
// words (per a multiple of 256 * kProbeUnroll, so every unrolled load stays
// inside the chunk), with nontemporal loads, 4 KiB per wave in flight; the
// words past grid * per are read grid-stride.  Contiguous per-workgroup
// chunks with deep unrolling read faster than a plain grid-stride loop.
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ buf, int64_t n16,
                                                         float* __restrict__ sink) {
    constexpr int64_t step = 256 * kProbeUnroll;
    const int64_t per = n16 / gridDim.x / step * step;
    const int64_t beg = per * blockIdx.x;
    uint32_t x = 0;
    for (int64_t i = beg + threadIdx.x; i < beg + per; i += step) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) v[k] = __builtin_nontemporal_load(buf + i + k * 256);
#pragma unroll
        for (int k = 0; k < kProbeUnroll; ++k) x ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = per * gridDim.x + static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) {
        const u32x4 a = buf[i];
        x ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
    __shared__ uint32_t s[4];
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = static_cast<float>((s[0] ^ s[1] ^ s[2] ^ s[3]) & 0xffffu);
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n16) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" int hpc_probe_read(const void* buf, int64_t bytes, float* sink, int32_t n_workgroups, void* stream) {
    if (!buf || !sink) return HPC_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || n_workgroups < 1) return HPC_ERR_INVALID;
    hipLaunchKernelGGL(read_probe_kernel, dim3(n_workgroups), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? HPC_OK : HPC_ERR_HIP;
}

extern "C" int hpc_probe_read_timed(const void* buf, int64_t bytes, float* sink, int32_t n_workgroups, void* stream,
                                    float* ms) {
    if (!buf || !sink || !ms) return HPC_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0 || n_workgroups < 1) return HPC_ERR_INVALID;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess) return HPC_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return HPC_ERR_HIP;
    }
    // the events are stamped when the kernel is dispatched and when it ends,
    // as for the decode library's own kernel timings
    hipExtLaunchKernelGGL(read_probe_kernel, dim3(n_workgroups), dim3(256), 0, static_cast<hipStream_t>(stream), e0, e1,
                          0u, static_cast<const u32x4*>(buf), bytes / 16, sink);
    int status = hipGetLastError() == hipSuccess ? HPC_OK : HPC_ERR_HIP;
    if (status == HPC_OK && (hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(ms, e0, e1) != hipSuccess))
        status = HPC_ERR_HIP;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return status;
}

extern "C" int hpc_probe_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst) return HPC_ERR_NULL;
    if (bytes <= 0 || bytes % 16 != 0) return HPC_ERR_INVALID;
    const int64_t n16 = bytes / 16;
    int64_t blocks = (n16 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                       static_cast<u32x4*>(dst), n16);
    return hipGetLastError() == hipSuccess ? HPC_OK : HPC_ERR_HIP;
}
