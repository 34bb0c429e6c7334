// Stream-read probe: the device's sustained HBM read rate, against which the
// forward's kernels are compared beside the 8 TB/s nominal peak.  Every
// thread reads 16-byte vectors grid-stride with non-temporal loads (no reuse,
// as the forward's weight streams), so that at each step the grid reads one
// contiguous 8 MB stretch, and folds them with XOR; each thread adds
// its fold to one word with a device-scope atomic XOR, so the result is
// checkable (the XOR of every 32-bit word read) and the loads cannot be
// optimized away.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace prox {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 2048;  // 8 per CU: measured the fastest of 1024 to 8192 for a 1 GiB read

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4 *__restrict__ p, size_t n,
                                                                    uint32_t *__restrict__ sink)
{
    uint32_t acc = 0u;
    const size_t stride = (size_t)gridDim.x * kProbeThreads;
    for (size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    if (acc) __hip_atomic_fetch_xor(sink, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_read_probe(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st)
{
    const size_t n = bytes / 16;
    read_probe_kernel<<<kProbeBlocks, kProbeThreads, 0, st>>>((const u32x4 *)buf, n, sink);
    return hipGetLastError();
}

}  // namespace prox
