// Approximate KV cache refresh and the block means it touches.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159),
// "Prerequisites" (approximate KV cache): in a step the rows of the refresh set
// U(t) take freshly computed keys and values and every other row keeps its cached
// ones.  "Method steps" (4): a prompt block is represented by the mean of its own
// keys, so a refresh can only change the means of the blocks that hold a refreshed
// prompt row; those are recomputed from the cache, exactly as the full pass does.
//
//   kv_scatter           64 list entries per workgroup: copies the new K and V rows into
//                        the cache, and V's elements into the keys-contiguous copy V^T
//                        when the caller keeps one.
//   block_means_refresh  64 list entries per workgroup: each entry that starts a block
//                        in the (ascending) list has the workgroup recompute that
//                        block's mean with an fp64 sum and one rounding, like the full
//                        pass.  Both sums are exact while the exponents of a block's keys
//                        span at most 29 - log2(bs) (fp32) or 45 - log2(bs) (bf16), and then
//                        agree bit for bit although they add the rows in different orders.

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

// One workgroup per (sequence, KV head, 64 list entries).  The K and V rows move as
// 16-byte pieces, every piece of the workgroup's share loaded before any is stored (the
// loads overlap instead of waiting one by one).  With V^T kept, the V rows are also
// staged in LDS and written out one d at a time, consecutive threads taking consecutive
// entries (consecutive keys where the refreshed rows form runs, as windows do), so the
// 2-byte writes coalesce.
constexpr int kScatterRows = 64;
constexpr int kScatterThreads = 256;

template <typename T>
__global__ __launch_bounds__(kScatterThreads) void kv_scatter_kernel(const CacheArgs a) {
    constexpr int kMaxPieces = kScatterRows * 128 * 4 / 16 / kScatterThreads;   // d <= 128, 4-byte T
    __shared__ __attribute__((aligned(16))) uint8_t tile[kScatterRows * 128 * sizeof(T)];
    __shared__ int s_row[kScatterRows];
    const int i0 = blockIdx.x * kScatterRows;
    const int b = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
    const int n = min(a.n_rows ? a.n_rows[b] : a.n_max, a.n_max);
    if (i0 >= n) return;
    const int32_t* rows = a.rows + static_cast<int64_t>(b) * a.n_max;
    if (threadIdx.x < kScatterRows) {
        const int i = i0 + threadIdx.x;
        const int r = i < n ? rows[i] : -1;
        s_row[threadIdx.x] = (r >= 0 && r < a.L) ? r : -1;
    }
    __syncthreads();
    const int ppr = a.d * static_cast<int>(sizeof(T)) / 16;   // 16-byte pieces per row
    const uint8_t* kn = static_cast<const uint8_t*>(a.k_new) + (b * a.knb + g * a.knh) * sizeof(T);
    const uint8_t* vn = static_cast<const uint8_t*>(a.v_new) + (b * a.vnb + g * a.vnh) * sizeof(T);
    uint8_t* k = static_cast<uint8_t*>(a.k) + (b * a.ksb + g * a.ksh) * sizeof(T);
    uint8_t* v = static_cast<uint8_t*>(a.v) + (b * a.vsb + g * a.vsh) * sizeof(T);
    u32x4 kx[kMaxPieces], vx[kMaxPieces];
#pragma unroll
    for (int u = 0; u < kMaxPieces; ++u) {
        const int e = threadIdx.x + u * kScatterThreads;
        const int i = e / ppr, pc = e % ppr;
        if (i < kScatterRows && s_row[i] >= 0) {
            kx[u] = *reinterpret_cast<const u32x4*>(kn + (static_cast<int64_t>(i0 + i) * a.knr) * sizeof(T) + 16 * pc);
            vx[u] = *reinterpret_cast<const u32x4*>(vn + (static_cast<int64_t>(i0 + i) * a.vnr) * sizeof(T) + 16 * pc);
        }
    }
#pragma unroll
    for (int u = 0; u < kMaxPieces; ++u) {
        const int e = threadIdx.x + u * kScatterThreads;
        const int i = e / ppr, pc = e % ppr;
        if (i < kScatterRows && s_row[i] >= 0) {
            const int64_t r = s_row[i];
            *reinterpret_cast<u32x4*>(k + (r * a.ksr) * sizeof(T) + 16 * pc) = kx[u];
            *reinterpret_cast<u32x4*>(v + (r * a.vsr) * sizeof(T) + 16 * pc) = vx[u];
            if (a.vt) *reinterpret_cast<u32x4*>(tile + (i * a.d) * sizeof(T) + 16 * pc) = vx[u];
        }
    }
    if (!a.vt) return;
    __syncthreads();
    T* vt = static_cast<T*>(a.vt) + b * a.vtsb + g * a.vtsh;
    const T* t = reinterpret_cast<const T*>(tile);
    for (int e = threadIdx.x; e < kScatterRows * a.d; e += kScatterThreads) {
        const int c = e / kScatterRows, i = e % kScatterRows;
        const int r = s_row[i];
        if (r >= 0) vt[static_cast<int64_t>(c) * a.vtsd + r] = t[i * a.d + c];
    }
}

constexpr int kRefreshThreads = 256;

template <typename T>
__global__ __launch_bounds__(kRefreshThreads) void block_means_refresh_kernel(const CacheArgs a) {
    __shared__ double s_part[kRefreshThreads];
    __shared__ int s_blk[64];
    const int i0 = blockIdx.x * 64;
    const int b = blockIdx.y / a.Hkv, g = blockIdx.y % a.Hkv;
    const int n = min(a.n_rows ? a.n_rows[b] : a.n_max, a.n_max);
    if (i0 >= n) return;
    const int32_t* rows = a.rows + static_cast<int64_t>(b) * a.n_max;
    if (threadIdx.x < 64) {
        // entry i starts a block when its row is a prompt row and the previous entry's row
        // (ascending lists) lies in another block
        const int i = i0 + threadIdx.x;
        int blk = -1;
        if (i < n) {
            const int r = rows[i];
            if (r >= 0 && r < a.P) {
                blk = r / a.bs;
                if (i > 0) {
                    const int rp = rows[i - 1];
                    if (rp >= 0 && rp < a.P && rp / a.bs == blk) blk = -1;
                }
            }
        }
        s_blk[threadIdx.x] = blk;
    }
    __syncthreads();
    const int parts = kRefreshThreads / a.d;   // d divides kRefreshThreads (d = 64 or 128)
    const int c = threadIdx.x % a.d, part = threadIdx.x / a.d;
    const T* k = static_cast<const T*>(a.k) + b * a.ksb + g * a.ksh + c;
    for (int e = 0; e < 64; ++e) {
        const int blk = s_blk[e];
        if (blk < 0) continue;
        const int lo = blk * a.bs, hi = min(lo + a.bs, a.P);
        double s = 0.0;
        for (int j0 = lo + part; j0 < hi; j0 += 16 * parts) {
            float x[16];   // 16 loads in flight, then the fp64 adds in row order
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int j = j0 + u * parts;
                x[u] = j < hi ? load_elem<T>(k + static_cast<int64_t>(j) * a.ksr) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u)
                if (j0 + u * parts < hi) s += static_cast<double>(x[u]);
        }
        s_part[threadIdx.x] = s;
        __syncthreads();
        if (part == 0) {
            double tot = 0.0;
            for (int p = 0; p < parts; ++p) tot += s_part[p * a.d + c];
            a.kbar[((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + blk) * a.d + c] =
                static_cast<float>(tot / static_cast<double>(hi - lo));
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_kv_scatter(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream) {
    if (a.n_max == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.n_max + kScatterRows - 1) / kScatterRows),
                    static_cast<unsigned>(a.B * a.Hkv));
    if (dtype == FDL_BF16) hipLaunchKernelGGL(kv_scatter_kernel<uint16_t>, grid, dim3(kScatterThreads), 0, stream, a);
    else hipLaunchKernelGGL(kv_scatter_kernel<float>, grid, dim3(kScatterThreads), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_block_means_refresh(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream) {
    if (a.n_max == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.n_max + 63) / 64), static_cast<unsigned>(a.B * a.Hkv));
    if (dtype == FDL_BF16) hipLaunchKernelGGL(block_means_refresh_kernel<uint16_t>, grid, dim3(kRefreshThreads), 0, stream, a);
    else hipLaunchKernelGGL(block_means_refresh_kernel<float>, grid, dim3(kRefreshThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fdl
