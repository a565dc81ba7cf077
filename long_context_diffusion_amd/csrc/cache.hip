// Approximate KV cache refresh and the block means it touches.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159),
// "Prerequisites" (approximate KV cache): in a step the rows of the refresh set
// U(t) take freshly computed keys and values and every other row keeps its cached
// ones.  "Method steps" (4): a prompt block is represented by the mean of its own
// keys, so a refresh can only change the means of the blocks that hold a refreshed
// prompt row; those are recomputed from the cache, exactly as the full pass does.
//
//   kv_scatter           one workgroup per (refreshed row, sequence, KV head): copies
//                        the new K and V rows into the cache, and V's elements into
//                        the keys-contiguous copy V^T when the caller keeps one.
//   block_means_refresh  one workgroup per (refreshed row, sequence, KV head): the
//                        first row of a block in the (ascending) list recomputes that
//                        block's mean with an fp64 sum (exact for bf16 and fp32 keys,
//                        so the result has the same single rounding as the full pass).

#include "ops.cuh"

namespace fdl {

namespace {

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) {
    return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }

template <typename T>
__global__ __launch_bounds__(128) void kv_scatter_kernel(const CacheArgs a) {
    const int i = blockIdx.x;
    const int b = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
    const int n = a.n_rows ? a.n_rows[b] : a.n_max;
    if (i >= n) return;
    const int r = a.rows[static_cast<int64_t>(b) * a.n_max + i];
    if (r < 0 || r >= a.L) return;
    const T* kn = static_cast<const T*>(a.k_new) + b * a.knb + g * a.knh + static_cast<int64_t>(i) * a.knr;
    const T* vn = static_cast<const T*>(a.v_new) + b * a.vnb + g * a.vnh + static_cast<int64_t>(i) * a.vnr;
    T* k = static_cast<T*>(a.k) + b * a.ksb + g * a.ksh + static_cast<int64_t>(r) * a.ksr;
    T* v = static_cast<T*>(a.v) + b * a.vsb + g * a.vsh + static_cast<int64_t>(r) * a.vsr;
    T* vt = a.vt ? static_cast<T*>(a.vt) + b * a.vtsb + g * a.vtsh + r : nullptr;
    for (int c = threadIdx.x; c < a.d; c += blockDim.x) {
        k[c] = kn[c];
        const T x = vn[c];
        v[c] = x;
        if (vt) vt[static_cast<int64_t>(c) * a.vtsd] = x;
    }
}

constexpr int kRefreshThreads = 256;

template <typename T>
__global__ __launch_bounds__(kRefreshThreads) void block_means_refresh_kernel(const CacheArgs a) {
    __shared__ double s_part[kRefreshThreads];
    const int i = blockIdx.x;
    const int b = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
    const int n = a.n_rows ? a.n_rows[b] : a.n_max;
    if (i >= n) return;
    const int32_t* rows = a.rows + static_cast<int64_t>(b) * a.n_max;
    const int r = rows[i];
    if (r < 0 || r >= a.P) return;
    const int blk = r / a.bs;
    if (i > 0) {   // an earlier row of the list in the same block does it
        const int rp = rows[i - 1];
        if (rp >= 0 && rp < a.P && rp / a.bs == blk) return;
    }
    const int lo = blk * a.bs, hi = min(lo + a.bs, a.P);
    const int parts = kRefreshThreads / a.d;   // d divides kRefreshThreads (d = 64 or 128)
    const int c = threadIdx.x % a.d, part = threadIdx.x / a.d;
    const T* k = static_cast<const T*>(a.k) + b * a.ksb + g * a.ksh + c;
    double s = 0.0;
    if (part < parts)
        for (int j = lo + part; j < hi; j += parts) s += static_cast<double>(load_elem<T>(k + static_cast<int64_t>(j) * a.ksr));
    s_part[threadIdx.x] = s;
    __syncthreads();
    if (part == 0) {
        double tot = 0.0;
        for (int p = 0; p < parts; ++p) tot += s_part[p * a.d + c];
        a.kbar[((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + blk) * a.d + c] =
            static_cast<float>(tot / static_cast<double>(hi - lo));
    }
}

}  // namespace

hipError_t launch_kv_scatter(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream) {
    if (a.n_max == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.n_max), static_cast<unsigned>(a.B * a.Hkv));
    if (dtype == FDL_BF16) hipLaunchKernelGGL(kv_scatter_kernel<uint16_t>, grid, dim3(128), 0, stream, a);
    else hipLaunchKernelGGL(kv_scatter_kernel<float>, grid, dim3(128), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_block_means_refresh(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream) {
    if (a.n_max == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(a.n_max), static_cast<unsigned>(a.B * a.Hkv));
    if (dtype == FDL_BF16) hipLaunchKernelGGL(block_means_refresh_kernel<uint16_t>, grid, dim3(kRefreshThreads), 0, stream, a);
    else hipLaunchKernelGGL(block_means_refresh_kernel<float>, grid, dim3(kRefreshThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fdl
