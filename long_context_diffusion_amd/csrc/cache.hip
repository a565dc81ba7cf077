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
//                        pass (16-byte loads, a block's loads in flight together).  Both sums are exact while the exponents of a block's keys
//                        span at most 29 - log2(bs) (fp32) or 45 - log2(bs) (bf16), and then
//                        agree bit for bit although they add the rows in different orders.

#include "ops.cuh"

namespace fdl {

namespace {

// One workgroup per (sequence, KV head, 64 list entries).  The K and V rows move as
// 16-byte pieces, every piece of the workgroup's share loaded before any is stored (the
// loads overlap instead of waiting one by one).  With V^T kept, the V rows are also
// staged in LDS and written out one d at a time, consecutive threads taking consecutive
// entries (consecutive keys where the refreshed rows form runs, as windows do), so the
// 2-byte writes coalesce.
constexpr int kScatterRows = 64;
constexpr int kScatterThreads = 256;

template <typename T>
__device__ __forceinline__ void kv_scatter_body(const CacheArgs& a, int chunk, int bg) {
    constexpr int kMaxPieces = kScatterRows * 128 * 4 / 16 / kScatterThreads;   // d <= 128, 4-byte T
    // staged V rows, row stride d + pad elements: the transposing reads (one d, 64 rows) then
    // fall on different banks (d = 128 bf16 rows, 256 bytes apart, would all hit one bank)
    constexpr int kPad = sizeof(T) == 2 ? 4 : 1;
    __shared__ __attribute__((aligned(16))) uint8_t tile[kScatterRows * (128 + kPad) * sizeof(T)];
    __shared__ int s_row[kScatterRows];
    const int i0 = chunk * kScatterRows;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int n = min(a.n_rows ? a.n_rows[b] : a.n_max, a.n_max);
    if (i0 >= n) return;
    const int32_t* rows = a.rows + static_cast<int64_t>(b) * a.n_max;
    const int ppr = a.d * static_cast<int>(sizeof(T)) / 16;   // 16-byte pieces per row
    const uint8_t* kn = static_cast<const uint8_t*>(a.k_new) + (b * a.knb + g * a.knh) * sizeof(T);
    const uint8_t* vn = static_cast<const uint8_t*>(a.v_new) + (b * a.vnb + g * a.vnh) * sizeof(T);
    uint8_t* k = static_cast<uint8_t*>(a.k) + (b * a.ksb + g * a.ksh) * sizeof(T);
    uint8_t* v = static_cast<uint8_t*>(a.v) + (b * a.vsb + g * a.vsh) * sizeof(T);
    // the entries' rows and their new K and V pieces are loaded together (the new rows are
    // indexed by entry, so their loads need not wait for the row indices)
    int rr[kMaxPieces];
    u32x4 kx[kMaxPieces], vx[kMaxPieces];
#pragma unroll
    for (int u = 0; u < kMaxPieces; ++u) {
        const int e = threadIdx.x + u * kScatterThreads;
        const int i = e / ppr, pc = e % ppr;
        rr[u] = -1;
        if (i < kScatterRows && i0 + i < n) {
            rr[u] = rows[i0 + i];
            kx[u] = *reinterpret_cast<const u32x4*>(kn + (static_cast<int64_t>(i0 + i) * a.knr) * sizeof(T) + 16 * pc);
            vx[u] = *reinterpret_cast<const u32x4*>(vn + (static_cast<int64_t>(i0 + i) * a.vnr) * sizeof(T) + 16 * pc);
        }
    }
    if (a.vt && threadIdx.x < kScatterRows) {
        const int i = i0 + threadIdx.x;
        const int r = i < n ? rows[i] : -1;
        s_row[threadIdx.x] = (r >= 0 && r < a.L) ? r : -1;
    }
#pragma unroll
    for (int u = 0; u < kMaxPieces; ++u) {
        const int e = threadIdx.x + u * kScatterThreads;
        const int i = e / ppr, pc = e % ppr;
        if (rr[u] >= 0 && rr[u] < a.L) {
            const int64_t r = rr[u];
            *reinterpret_cast<u32x4*>(k + (r * a.ksr) * sizeof(T) + 16 * pc) = kx[u];
            *reinterpret_cast<u32x4*>(v + (r * a.vsr) * sizeof(T) + 16 * pc) = vx[u];
            if (a.vt) {
                uint8_t* dst = tile + (i * (a.d + kPad)) * sizeof(T) + 16 * pc;
                if (sizeof(T) == 2) {   // 8-byte aligned with the padded stride
                    *reinterpret_cast<u32x2*>(dst) = u32x2{vx[u][0], vx[u][1]};
                    *reinterpret_cast<u32x2*>(dst + 8) = u32x2{vx[u][2], vx[u][3]};
                } else {                // 4-byte aligned
#pragma unroll
                    for (int q = 0; q < 4; ++q) reinterpret_cast<uint32_t*>(dst)[q] = vx[u][q];
                }
            }
        }
    }
    if (!a.vt) return;
    __syncthreads();
    T* vt = static_cast<T*>(a.vt) + b * a.vtsb + g * a.vtsh;
    const T* t = reinterpret_cast<const T*>(tile);
    for (int e = threadIdx.x; e < kScatterRows * a.d; e += kScatterThreads) {
        const int c = e / kScatterRows, i = e % kScatterRows;
        const int r = s_row[i];
        if (r >= 0) vt[static_cast<int64_t>(c) * a.vtsd + r] = t[i * (a.d + kPad) + c];
    }
}

constexpr int kRefreshThreads = 256;

template <typename T>
__device__ __forceinline__ void unpack_piece(const u32x4& x, float* out);
template <>
__device__ __forceinline__ void unpack_piece<uint16_t>(const u32x4& x, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16lo(x[i]);
        out[2 * i + 1] = bf16hi(x[i]);
    }
}
template <>
__device__ __forceinline__ void unpack_piece<float>(const u32x4& x, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(x[i]);
}

// One workgroup per (sequence, KV head, 64 list entries).  The entries that start a block
// in the ascending list name the blocks to recompute; each such block is read with 16-byte
// loads, all of a thread's loads of the block in flight together (lane l takes piece l % NP
// of rows l / NP, l / NP + RG, ...), summed in fp64, folded over the row groups with
// shuffles and over the waves through LDS, and its mean rounded once.
// FROM_NEW: the refreshed rows of a block are read from k_new (the list entry that holds
// them) and the other rows from the cache, so the means need not wait for the scatter
// (the fused refresh runs both in one launch); otherwise every row comes from the cache.
template <typename T, int D, bool FROM_NEW>
__device__ __forceinline__ void means_refresh_body(const CacheArgs& a, int chunk, int bg) {
    constexpr int EPP = 16 / sizeof(T);          // elements per 16-byte piece
    constexpr int NP = D / EPP;                  // pieces per row
    constexpr int RG = kRefreshThreads / NP;     // rows read together by the workgroup
    constexpr int kBatch = 8;                    // loads per thread in flight
    constexpr int kWaves = kRefreshThreads / kWave;
    __shared__ double s_sum[kWaves][EPP][NP];
    __shared__ int s_blk[64];
    const int i0 = chunk * 64;
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int n = min(a.n_rows ? a.n_rows[b] : a.n_max, a.n_max);
    if (i0 >= n) return;
    const int32_t* rows = a.rows + static_cast<int64_t>(b) * a.n_max;
    const int tid = threadIdx.x;
    if (tid < 64) {
        // entry i starts a block when its row is a prompt row and the previous entry's row
        // (ascending lists) lies in another block
        const int i = i0 + tid;
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
        s_blk[tid] = blk;
    }
    __syncthreads();
    const int piece = tid % NP, rg = tid / NP, wv = tid / kWave;
    const T* kbase = static_cast<const T*>(a.k) + b * a.ksb + g * a.ksh + piece * EPP;
    const T* knbase = static_cast<const T*>(a.k_new) + b * a.knb + g * a.knh + piece * EPP;
    __shared__ int s_src[FROM_NEW ? kFusedMaxBs : 1];   // row lo + j: list entry, or -1
    for (int e = 0; e < 64; ++e) {
        const int blk = s_blk[e];
        if (blk < 0) continue;   // the same for every thread
        const int lo = blk * a.bs, hi = min(lo + a.bs, a.P);
        if constexpr (FROM_NEW) {
            for (int j = tid; j < hi - lo; j += kRefreshThreads) s_src[j] = -1;
            __syncthreads();
            for (int i = tid; i < n; i += kRefreshThreads) {
                const int r = rows[i];
                if (r >= lo && r < hi) s_src[r - lo] = i;
            }
            __syncthreads();
        }
        double acc[EPP];
#pragma unroll
        for (int q = 0; q < EPP; ++q) acc[q] = 0.0;
        for (int j0 = lo + rg; j0 < hi; j0 += RG * kBatch) {
            u32x4 x[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int j = min(j0 + u * RG, hi - 1);
                const T* src = kbase + static_cast<int64_t>(j) * a.ksr;
                if constexpr (FROM_NEW) {
                    const int si = s_src[j - lo];
                    if (si >= 0) src = knbase + static_cast<int64_t>(si) * a.knr;
                }
                x[u] = *reinterpret_cast<const u32x4*>(src);
            }
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (j0 + u * RG >= hi) break;
                float v[EPP];
                unpack_piece<T>(x[u], v);
#pragma unroll
                for (int q = 0; q < EPP; ++q) acc[q] += static_cast<double>(v[q]);
            }
        }
        // within the stated exponent range the fp64 sums are exact, so the order of the
        // additions (different from the full pass) does not change them
#pragma unroll
        for (int q = 0; q < EPP; ++q)
#pragma unroll
            for (int off = NP; off < kWave; off <<= 1) acc[q] += __shfl_xor(acc[q], off, kWave);
        if ((tid % kWave) < NP) {
#pragma unroll
            for (int q = 0; q < EPP; ++q) s_sum[wv][q][piece] = acc[q];
        }
        __syncthreads();
        for (int ep = tid; ep < D; ep += kRefreshThreads) {   // ep = q * NP + piece: element piece * EPP + q
            const int q = ep / NP, pc = ep % NP;
            double t = 0.0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) t += s_sum[w][q][pc];
            a.kbar[((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + blk) * D + pc * EPP + q] =
                static_cast<float>(t / static_cast<double>(hi - lo));
        }
        __syncthreads();
    }
}

template <typename T>
__global__ __launch_bounds__(kScatterThreads) void kv_scatter_kernel(const CacheArgs a) {
    kv_scatter_body<T>(a, blockIdx.x, blockIdx.y);
}

template <typename T, int D>
__global__ __launch_bounds__(kRefreshThreads) void block_means_refresh_kernel(const CacheArgs a) {
    means_refresh_body<T, D, false>(a, blockIdx.x, blockIdx.y);
}

// Both in one launch: the first workgroups of each (sequence, KV head) scatter, the others
// recompute the touched means from the cache and the new rows.
template <typename T, int D>
__global__ __launch_bounds__(kRefreshThreads) void kv_refresh_means_kernel(const CacheArgs a) {
    static_assert(kScatterThreads == kRefreshThreads, "one workgroup size");
    const int n_scatter = (a.n_max + kScatterRows - 1) / kScatterRows;
    if (static_cast<int>(blockIdx.x) < n_scatter) kv_scatter_body<T>(a, blockIdx.x, blockIdx.y);
    else means_refresh_body<T, D, true>(a, blockIdx.x - n_scatter, blockIdx.y);
}

}  // namespace

hipError_t launch_kv_refresh_means(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream) {
    if (a.n_max == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>((a.n_max + kScatterRows - 1) / kScatterRows + (a.n_max + 63) / 64),
                    static_cast<unsigned>(a.B * a.Hkv));
#define FDL_FUSED(T, DD) hipLaunchKernelGGL((kv_refresh_means_kernel<T, DD>), grid, dim3(kRefreshThreads), 0, stream, a)
    if (dtype == FDL_BF16) { if (a.d == 128) FDL_FUSED(uint16_t, 128); else FDL_FUSED(uint16_t, 64); }
    else { if (a.d == 128) FDL_FUSED(float, 128); else FDL_FUSED(float, 64); }
#undef FDL_FUSED
    return hipGetLastError();
}

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
#define FDL_REFRESH(T, DD) \
    hipLaunchKernelGGL((block_means_refresh_kernel<T, DD>), grid, dim3(kRefreshThreads), 0, stream, a)
    if (dtype == FDL_BF16) { if (a.d == 128) FDL_REFRESH(uint16_t, 128); else FDL_REFRESH(uint16_t, 64); }
    else { if (a.d == 128) FDL_REFRESH(float, 128); else FDL_REFRESH(float, 64); }
#undef FDL_REFRESH
    return hipGetLastError();
}

}  // namespace fdl
