// A plain streaming read of device memory: the achievable-bandwidth reference of the benchmark.
// Every wave reads whole 1 KiB lines (64 lanes x 16 bytes) of a contiguous share of the buffer,
// eight lines in flight, and folds them with xor; one word per workgroup is written at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_bench.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 512;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void k_stream_read(const u32x4* __restrict__ src, uint64_t n16,
                                                           uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t waves = (uint64_t)gridDim.x * (kThreads / 64);
    const uint64_t w = (uint64_t)blockIdx.x * (kThreads / 64) + wave;
    // contiguous share of whole 64-chunk lines per wave
    const uint64_t lines = (n16 + 63) / 64;
    const uint64_t l0 = lines * w / waves, l1 = lines * (w + 1) / waves;
    u32x4 acc = {0u, 0u, 0u, 0u};
    uint64_t l = l0;
    for (; l + kUnroll <= l1; l += kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint64_t i = (l + u) * 64 + lane;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
    for (; l < l1; ++l) {
        const uint64_t i = l * 64 + lane;
        if (i < n16) acc ^= __builtin_nontemporal_load(src + i);
    }
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    __shared__ uint32_t red[kThreads / 64];
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    if (lane == 0) red[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
        for (int i = 0; i < kThreads / 64; ++i) r ^= red[i];
        sink[blockIdx.x] = r;
    }
}

int blocks() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    return 2 * cus;  // two 8-wave workgroups per CU
}

}  // namespace

extern "C" int moe_bench_stream_read_blocks(void) { return blocks(); }

extern "C" int moe_bench_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
    if (!src || !sink || bytes == 0 || (bytes & 15) || ((uintptr_t)src & 15)) return -1;
    const int g = blocks();
    if (g <= 0) return -6;
    hipLaunchKernelGGL(k_stream_read, dim3(g), dim3(kThreads), 0, (hipStream_t)stream, (const u32x4*)src,
                       (uint64_t)(bytes / 16), sink);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}
