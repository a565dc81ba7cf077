// Achievable rates of the GPU the library runs on, for reading roofline fractions.
//
// The published peaks (8 TB/s HBM3E, 2.5 PFLOP/s dense bf16 MFMA on MI355X) are the
// bounds every kernel of the library is priced against.  These two kernels measure
// what a plain kernel reaches on the same part, under sustained load:
//   calib_read    streams a buffer once with non-temporal 16-byte loads (each
//                 workgroup takes 64 KB a round, 16 loads per lane in flight), folds
//                 the words into one XOR per workgroup so no load is dead.
//   calib_mfma    every wave issues v_mfma_f32_32x32x16_bf16 back to back on eight
//                 independent accumulators whose operands live in registers (no memory
//                 traffic); each accumulator element ends at 16 * a * b * iters.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 16;
constexpr int kMfmaThreads = 256;   // one wave per SIMD
constexpr int kMfmaChains = 8;

__global__ __launch_bounds__(kReadThreads) void calib_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                  uint32_t* __restrict__ sink) {
    __shared__ uint32_t s_x[kReadThreads / kWave];
    const int tid = threadIdx.x;
    constexpr int64_t kChunk = static_cast<int64_t>(kReadThreads) * kReadUnroll;
    uint32_t x = 0;
    for (int64_t c0 = static_cast<int64_t>(blockIdx.x) * kChunk; c0 < n16; c0 += static_cast<int64_t>(gridDim.x) * kChunk) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t i = c0 + u * kReadThreads + tid;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x ^= __shfl_xor(x, off, kWave);
    if ((tid & (kWave - 1)) == 0) s_x[tid / kWave] = x;
    __syncthreads();
    if (tid == 0) {
        uint32_t t = 0;
#pragma unroll
        for (int w = 0; w < kReadThreads / kWave; ++w) t ^= s_x[w];
        sink[blockIdx.x] = t;
    }
}

__global__ __launch_bounds__(kMfmaThreads) void calib_mfma_kernel(int iters, float a_val, float b_val,
                                                                  float* __restrict__ sink) {
    bf16x8 av, bv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        av[e] = static_cast<__bf16>(a_val);
        bv[e] = static_cast<__bf16>(b_val);
    }
    f32x16 acc[kMfmaChains];
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[c], 0, 0, 0);
    }
    // every element of every chain holds 16 a b iters; lane 0 of each wave reports chain 0's
    // first element and the largest deviation of any element from it
    float ref = acc[0][0], dev = 0.0f;
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) dev = fmaxf(dev, fabsf(acc[c][i] - ref));
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) dev = fmaxf(dev, __shfl_xor(dev, off, kWave));
    const int wave = blockIdx.x * (kMfmaThreads / kWave) + threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        sink[2 * wave] = ref;
        sink[2 * wave + 1] = dev;
    }
}

}  // namespace

hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
    hipLaunchKernelGGL(calib_read_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kReadThreads), 0, stream,
                       static_cast<const u32x4*>(src), static_cast<int64_t>(bytes / 16), sink);
    return hipGetLastError();
}

hipError_t launch_calib_mfma(int workgroups, int iters, float a_val, float b_val, float* sink, hipStream_t stream) {
    hipLaunchKernelGGL(calib_mfma_kernel, dim3(static_cast<unsigned>(workgroups)), dim3(kMfmaThreads), 0, stream,
                       iters, a_val, b_val, sink);
    return hipGetLastError();
}

}  // namespace fdl
