// probe.hip -- a streaming-read calibration kernel: the HBM read rate that the load form of the
// partial passes reaches on this part, measured in the same process as the decode step.
//
// Every work group streams its own contiguous region, as a split-KV work unit streams its keys:
// 16-byte nontemporal loads (each wave instruction reads whole 128-byte lines once), four loads
// per lane in flight per step, XOR-folded so that no load can be dropped, and one 32-bit word per
// wave written at the end.
#include "ad_internal.h"

namespace ad {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(kThreads) read_probe_kernel(const u32x4 *src, int64_t n16, int64_t per_group,
                                                               uint32_t *sink) {
    const int64_t begin = (int64_t)blockIdx.x * per_group;
    const int64_t end = begin + per_group < n16 ? begin + per_group : n16;
    u32x4 acc = {0, 0, 0, 0};
    int64_t i = begin + threadIdx.x;
    // whole steps: kUnroll loads per lane, all inside [begin, end)
    for (; i + (kUnroll - 1) * kThreads < end; i += kUnroll * kThreads) {
        u32x4 x[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) x[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= x[u];
    }
    for (; i < end; i += kThreads) acc ^= __builtin_nontemporal_load(src + i);
    uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
    // one word per wave, folded over its lanes
    v ^= __shfl_xor(v, 32);
    v ^= __shfl_xor(v, 16);
    v ^= __shfl_xor(v, 8);
    v ^= __shfl_xor(v, 4);
    v ^= __shfl_xor(v, 2);
    v ^= __shfl_xor(v, 1);
    if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = v;
}

}  // namespace

// `groups` work groups of 256 threads; sink holds 4 words per group.
hipError_t launch_read_probe(const void *src, int64_t bytes, uint32_t *sink, int groups, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t per = (n16 + groups - 1) / groups;
    hipLaunchKernelGGL(read_probe_kernel, dim3(groups), dim3(kThreads), 0, stream, static_cast<const u32x4 *>(src),
                       n16, per, sink);
    return hipGetLastError();
}

}  // namespace ad
