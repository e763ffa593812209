// hbm_read.hip -- an HBM streaming-read yardstick for the benchmark (not part
// of the layer): every 16-byte unit of a buffer is read once, each
// workgroup streaming a contiguous share with eight loads in flight per
// thread; the XOR of what was read is stored only if it
// equals a value no test buffer produces, so the loads cannot be dropped and
// almost nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(256) void hbm_read_kernel(const uint4* p, size_t n16, uint32_t* sink) {
    // workgroup b streams its own contiguous share of the buffer, 2048
    // units (32 KB) per round: eight loads of consecutive 4 KB lines per thread
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = (size_t)blockIdx.x * per;
    const size_t b1 = b0 + per < n16 ? b0 + per : n16;
    uint4 acc = {0u, 0u, 0u, 0u};
    size_t i = b0 + threadIdx.x;
    for (; i + 7 * 256 < b1; i += 8 * 256) {
        uint4 v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[i + j * 256];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            acc.x ^= v[j].x;
            acc.y ^= v[j].y;
            acc.z ^= v[j].z;
            acc.w ^= v[j].w;
        }
    }
    for (; i < b1; i += 256) {
        const uint4 v = p[i];
        acc.x ^= v.x;
        acc.y ^= v.y;
        acc.z ^= v.z;
        acc.w ^= v.w;
    }
    const uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
    if (x == 0x9E3779B9u) sink[0] = x;
}

}  // namespace

// Reads `bytes` (a multiple of 16) from device buffer `p` (16-byte aligned)
// once, on `stream`, with `blocks` workgroups of 256 threads (`blocks` <= the
// number of 16-byte units); sink: one device uint32 (almost never written).
// Returns a hipError_t.
extern "C" int hbm_read(const void* p, size_t bytes, void* sink, int blocks, void* stream) {
    if (!p || !sink || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(p) & 15) != 0 || blocks < 1 ||
        (size_t)blocks > bytes / 16)
        return (int)hipErrorInvalidValue;
    hbm_read_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(p), bytes / 16,
                                                                           static_cast<uint32_t*>(sink));
    return (int)hipGetLastError();
}
