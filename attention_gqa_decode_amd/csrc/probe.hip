// probe.hip -- streaming references of known traffic (16-byte non-temporal vector accesses).
// The copy probe calibrates the HBM byte counters (its bytes are exact); the
// read probe measures the practical streaming read rate, the ceiling the decode
// kernel chases.  Both use one workgroup of 512 threads per CU, each
// workgroup streaming its own contiguous slab; the copy keeps four 16-byte
// loads in flight per thread, the read eight (64 KiB per CU: on MI355X it
// read 4 GiB at 7.2 TB/s against 6.5 with four and 7.0 with sixteen).
#include "common.h"

namespace attn {
namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeUnroll = 4;  // copy probe
constexpr int kReadUnroll = 8;   // read probe

// Slab of workgroup `blk`: [begin, end) in 16-byte words, a near-equal split of n.
__device__ __forceinline__ void probe_slab(size_t n, size_t *begin, size_t *end) {
    *begin = n * blockIdx.x / gridDim.x;
    *end = n * (blockIdx.x + 1) / gridDim.x;
}

__global__ __launch_bounds__(kProbeThreads) void copy_probe_kernel(const u32x4 *__restrict__ src,
                                                                   u32x4 *__restrict__ dst, size_t n) {
    size_t i, end;
    probe_slab(n, &i, &end);
    constexpr size_t step = (size_t)kProbeUnroll * kProbeThreads;
    for (i += threadIdx.x; i + (kProbeUnroll - 1) * kProbeThreads < end; i += step) {
        u32x4 r[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) r[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) __builtin_nontemporal_store(r[u], dst + i + u * kProbeThreads);
    }
    for (; i < end; i += kProbeThreads) dst[i] = src[i];
}

// Every 16-byte word is loaded once; a per-thread xor is stored only if it
// matches a value the data never holds, so the kernel writes (almost) nothing.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ src, size_t n,
                                                                   uint32_t *__restrict__ sink) {
    size_t i, end;
    probe_slab(n, &i, &end);
    constexpr size_t step = (size_t)kReadUnroll * kProbeThreads;
    uint32_t acc = 0;
    for (i += threadIdx.x; i + (kReadUnroll - 1) * kProbeThreads < end; i += step) {
        u32x4 r[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) r[u] = __builtin_nontemporal_load(src + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= r[u][0] ^ r[u][1] ^ r[u][2] ^ r[u][3];
    }
    for (; i < end; i += kProbeThreads) {
        const u32x4 w = src[i];
        acc ^= w[0] ^ w[1] ^ w[2] ^ w[3];
    }
    if (acc == 0x9e3779b9u) sink[0] = acc;
}

hipError_t probe_grid(size_t n, unsigned *grid) {
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const size_t want = (n + kProbeThreads - 1) / kProbeThreads;
    *grid = (unsigned)(want < (size_t)cus ? want : (size_t)cus);
    return hipSuccess;
}

}  // namespace

hipError_t launch_read_probe(const void *src, size_t bytes, void *sink, hipStream_t stream) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    unsigned grid = 0;
    hipError_t e = probe_grid(n, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, static_cast<const u32x4 *>(src),
                       n, static_cast<uint32_t *>(sink));
    return hipGetLastError();
}

hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    unsigned grid = 0;
    hipError_t e = probe_grid(n, &grid);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(copy_probe_kernel, dim3(grid), dim3(kProbeThreads), 0, stream, static_cast<const u32x4 *>(src),
                       static_cast<u32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace attn
