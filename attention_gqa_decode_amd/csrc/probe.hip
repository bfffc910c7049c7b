// probe.hip -- plain streaming copy of known size (16-byte vector loads and stores).
// A measurement reference: its bytes are exact, so it calibrates the HBM byte
// counters and shows the practical streaming rate next to the 8 TB/s peak.
#include "common.h"

namespace attn {
namespace {

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                         size_t n) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy_probe(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    if (n == 0) return hipSuccess;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    size_t blocks = (n + 255) / 256;
    const size_t cap = (size_t)cus * 16;
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), n);
    return hipGetLastError();
}

}  // namespace attn
