// Measurement kernels: the HBM streaming rates and the fp32 atomic-add rate in
// the backward's flush pattern. They give the benchmark measured denominators
// beside the published peaks, and the copy kernel is the known-size reference
// for scaling rocprof's FETCH_SIZE / WRITE_SIZE counters.
#include "common.hpp"
#include "launch.hpp"

namespace gs {

namespace {

__global__ __launch_bounds__(256) void k_mb_read(const float4* __restrict__ src, size_t n4, float* sink) {
    float acc = 0.f;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 v = src[i];
        acc += (v.x + v.y) + (v.z + v.w);
    }
    if (acc == -1.2345678e30f) sink[0] = acc;  // keeps the loads; never true for real data
}

__global__ __launch_bounds__(256) void k_mb_copy(float4* __restrict__ dst, const float4* __restrict__ src, size_t n4) {
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
}

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352dU;
    x ^= x >> 15;
    x *= 0x846ca68bU;
    x ^= x >> 16;
    return x;
}

__global__ __launch_bounds__(256) void k_mb_atomic(float* __restrict__ rec, uint32_t n_records, int64_t n_ops,
                                                  int lanes) {
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_ops; i += stride) {
        int64_t grp = i / lanes;
        int c = (int)(i - grp * lanes);
        uint32_t r = n_records == 1 ? 0u : mix32((uint32_t)grp) % n_records;
        atomicAdd(&rec[(size_t)r * GRAD2D_STRIDE + c], 1.0f);
    }
}

int grid_for(size_t work, int per_thread_min = 4) {
    size_t blocks = (work / per_thread_min + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 256 * 16) blocks = 256 * 16;  // 16 blocks per CU, 256 CUs
    return (int)blocks;
}

}  // namespace

hipError_t launch_mb_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
    size_t n4 = bytes / 16;
    k_mb_read<<<grid_for(n4), 256, 0, s>>>(reinterpret_cast<const float4*>(src), n4, sink);
    return hipGetLastError();
}

hipError_t launch_mb_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
    size_t n4 = bytes / 16;
    k_mb_copy<<<grid_for(n4), 256, 0, s>>>(reinterpret_cast<float4*>(dst), reinterpret_cast<const float4*>(src), n4);
    return hipGetLastError();
}

hipError_t launch_mb_atomic(float* records, int64_t n_records, int64_t n_ops, int lanes, hipStream_t s) {
    k_mb_atomic<<<grid_for((size_t)n_ops, 16), 256, 0, s>>>(records, (uint32_t)n_records, n_ops, lanes);
    return hipGetLastError();
}

}  // namespace gs
