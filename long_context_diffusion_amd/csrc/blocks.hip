// Prompt-block pruning: block means, relevance R_b and top-C.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
// steps" (4): prompt keys are split into contiguous blocks of bs keys, each
// block is represented by the mean of its keys, the relevance R_b of the
// candidate queries to every block is scored and the C most relevant blocks
// are kept.  R_b = scale * sum_h sum_i q_{h,i} . kbar_{g(h),b}.
//
// R_b is linear in the queries and in the keys of the block, so it is
// evaluated as  R_b = scale / |b| * sum_g sum_{j in b} qsum_g . k_{g,j},  with
// qsum_g the sum of every active query row of every query head that reads KV
// head g.  The step is then one streaming read of the prompt keys:
//   block_qsum    qsum_g in fp64 (exact for bf16/fp32 inputs up to rounding of
//                 the final sum), one workgroup per (sequence, KV head).
//   block_scan    reads each prompt key once, 16 bytes per lane, fully
//                 coalesced; 8-term partial dot products in fp32, everything
//                 above them in fp64; writes one fp64 partial per (KV head,
//                 block).  Optionally also the block means (fp64 sums, one
//                 rounding to fp32).
//   block_select  sums the partials in KV-head order, scales by scale/|b|,
//                 and keeps the top-C blocks (radix select on the fp64 keys,
//                 lower block index first among equal scores), ascending.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kQsumThreads = 1024;
constexpr int kScanThreads = 256;

template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& x, float* out);
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const u32x4& x, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = bf16lo(x[i]);
        out[2 * i + 1] = bf16hi(x[i]);
    }
}
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& x, float* out) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(x[i]);
}

// qsum[b][g][e] = sum over packed rows p < Gq*nq of Q[b][g*Gq + p%Gq][row(p/Gq)][e], fp64.
template <typename T, int D>
__global__ __launch_bounds__(kQsumThreads) void block_qsum_kernel(const BlockArgs a) {
    constexpr int EPP = 16 / sizeof(T);       // elements per 16-byte piece
    constexpr int NP = D / EPP;               // pieces per row
    constexpr int RG = kQsumThreads / NP;     // row groups
    __shared__ double s_part[RG][D];
    const int tid = threadIdx.x;
    const int g = blockIdx.x % a.Hkv, b = blockIdx.x / a.Hkv;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows = a.Gq * nq;
    const int piece = tid % NP, rg = tid / NP;
    double acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
    // all row indices of a batch first, then all rows: two memory round trips per batch
    constexpr int kBatch = 16;
    for (int p0 = rg; p0 < rows; p0 += RG * kBatch) {
        int64_t off[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int p = min(p0 + u * RG, rows - 1);
            const int h = g * a.Gq + p % a.Gq, r = p / a.Gq;
            const int phys = a.q_idx ? max(a.q_idx[static_cast<int64_t>(b) * a.nq_max + r], 0) : r;
            off[u] = b * a.qsb + h * a.qsh + static_cast<int64_t>(phys) * a.qsr + piece * EPP;
        }
        u32x4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) x[u] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.q) + off[u]);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (p0 + u * RG >= rows) continue;
            float v[EPP];
            unpack16<T>(x[u], v);
#pragma unroll
            for (int e = 0; e < EPP; ++e) acc[e] += static_cast<double>(v[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < EPP; ++e) s_part[rg][piece * EPP + e] = acc[e];
    __syncthreads();
    // pairwise tree over the row groups (fixed order, so the sum is deterministic)
    for (int half = RG / 2; half >= 1; half >>= 1) {
        for (int i = tid; i < half * D; i += kQsumThreads) {
            const int r = i / D, e = i % D;
            s_part[r][e] += s_part[r + half][e];
        }
        __syncthreads();
    }
    for (int e = tid; e < D; e += kQsumThreads) a.qsum[(static_cast<int64_t>(b) * a.Hkv + g) * D + e] = s_part[0][e];
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// One workgroup per (sequence, KV head, run of blocks_per_wg blocks).
template <typename T, int D, bool KBAR>
__global__ __launch_bounds__(kScanThreads) void block_scan_kernel(const BlockArgs a) {
    constexpr int EPP = 16 / sizeof(T);
    constexpr int NP = D / EPP;                 // pieces per key row
    constexpr int RPI = kScanThreads / NP;      // key rows per block-wide load
    __shared__ double s_red[kScanThreads / 64];
    __shared__ double s_kbar[KBAR ? RPI : 1][KBAR ? D : 1];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int chunk = blockIdx.x % a.scan_chunks;
    const int bg = blockIdx.x / a.scan_chunks;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int piece = tid % NP, roff = tid / NP;
    float qg[EPP];
    {
        const double* qs = a.qsum + (static_cast<int64_t>(b) * a.Hkv + g) * D + piece * EPP;
#pragma unroll
        for (int e = 0; e < EPP; ++e) qg[e] = static_cast<float>(qs[e]);
    }
    const T* kbase = static_cast<const T*>(a.k) + b * a.ksb + g * a.ksh + piece * EPP;
    const int blk0 = chunk * a.blocks_per_wg;
    const int blk1 = min(a.nb, blk0 + a.blocks_per_wg);
    for (int blk = blk0; blk < blk1; ++blk) {
        const int lo = blk * a.bs;
        const int hi = min(lo + a.bs, a.P);
        double part = 0.0;
        double ksum[KBAR ? EPP : 1];
        if (KBAR) {
#pragma unroll
            for (int e = 0; e < EPP; ++e) ksum[e] = 0.0;
        }
        // rows lo + roff, lo + roff + RPI, ...; loads of one block are issued together
        for (int j0 = lo; j0 < hi; j0 += 4 * RPI) {
            u32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u * RPI + roff;
                x[u] = u32x4{0u, 0u, 0u, 0u};
                if (j < hi) x[u] = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * a.ksr);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float v[EPP];
                unpack16<T>(x[u], v);
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < EPP; ++e) dot = fmaf(v[e], qg[e], dot);
                part += static_cast<double>(dot);
                if (KBAR) {
#pragma unroll
                    for (int e = 0; e < EPP; ++e) ksum[e] += static_cast<double>(v[e]);
                }
            }
        }
        part = wave_sum_f64(part);
        if (lane == 0) s_red[wv] = part;
        if (KBAR) {
            // rows handled by the same piece live in threads piece + NP*roff; combine through LDS
            if (roff < RPI) {
#pragma unroll
                for (int e = 0; e < EPP; ++e) s_kbar[roff][piece * EPP + e] = ksum[e];
            }
        }
        __syncthreads();
        if (tid == 0) {
            double s = 0.0;
            for (int w = 0; w < kScanThreads / 64; ++w) s += s_red[w];
            a.rpart[(static_cast<int64_t>(b) * a.Hkv + g) * a.nb + blk] = s;
        }
        if (KBAR) {
            for (int e = tid; e < D; e += kScanThreads) {
                double s = 0.0;
                for (int i = 0; i < RPI; ++i) s += s_kbar[i][e];
                a.kbar[((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + blk) * D + e] =
                    static_cast<float>(s / static_cast<double>(hi - lo));
            }
        }
        __syncthreads();
    }
}

constexpr int kSelectLds = 2048;   // blocks ranked in LDS

__global__ __launch_bounds__(256) void block_select_kernel(const BlockArgs a, int C, int32_t* block_idx,
                                                            double* R_out) {
    __shared__ SelectSmem sm;
    __shared__ uint64_t s_key[kSelectLds];
    const int b = blockIdx.x;
    double* R = a.rfull + static_cast<int64_t>(b) * a.nb;
    for (int blk = threadIdx.x; blk < a.nb; blk += blockDim.x) {
        const double* rp = a.rpart + static_cast<int64_t>(b) * a.Hkv * a.nb + blk;
        double s = 0.0;
        int g = 0;
        for (; g + 8 <= a.Hkv; g += 8) {
            double x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = rp[static_cast<int64_t>(g + u) * a.nb];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += x[u];
        }
        for (; g < a.Hkv; ++g) s += rp[static_cast<int64_t>(g) * a.nb];
        const int cnt = min(a.bs, a.P - blk * a.bs);
        const double val = s * (static_cast<double>(a.scale) / static_cast<double>(cnt));
        if (a.nb <= kSelectLds) s_key[blk] = okey64(val);
        else R[blk] = val;
        if (R_out) R_out[static_cast<int64_t>(b) * a.nb + blk] = val;
    }
    __syncthreads();
    __threadfence_block();
    int32_t* out = block_idx + static_cast<int64_t>(b) * C;
    if (a.nb <= kSelectLds) {
        block_topk_lds<uint64_t>(a.nb, C, s_key, [](int j) { return j; }, out, C, &sm);
    } else {
        auto key_of = [&](int j, uint64_t* key) -> bool {
            *key = okey64(R[j]);
            return true;
        };
        block_emit_topk<uint64_t>(a.nb, C, key_of, [](int j) { return j; }, out, C, &sm);
    }
}

}  // namespace

size_t block_workspace_bytes(int B, int Hkv, int P, int d, int bs) {
    const int64_t nb = (static_cast<int64_t>(P) + bs - 1) / bs;
    return static_cast<size_t>(B) * Hkv * d * sizeof(double) +      // qsum
           static_cast<size_t>(B) * Hkv * nb * sizeof(double) +     // per-head partials
           static_cast<size_t>(B) * nb * sizeof(double);            // R
}

hipError_t launch_block_score_topc(fdl_dtype dtype, int d, BlockArgs a, int C, int32_t* block_idx,
                                   double* R_out, void* ws, hipStream_t stream) {
    a.qsum = static_cast<double*>(ws);
    a.rpart = a.qsum + static_cast<int64_t>(a.B) * a.Hkv * d;
    a.rfull = a.rpart + static_cast<int64_t>(a.B) * a.Hkv * a.nb;
    a.blocks_per_wg = 2;
    a.scan_chunks = (a.nb + a.blocks_per_wg - 1) / a.blocks_per_wg;
    const bool bf = dtype == FDL_BF16;
    const dim3 qgrid(a.B * a.Hkv);
#define FDL_QSUM(T, DD) hipLaunchKernelGGL((block_qsum_kernel<T, DD>), qgrid, dim3(kQsumThreads), 0, stream, a)
    if (bf) { if (d == 128) FDL_QSUM(uint16_t, 128); else FDL_QSUM(uint16_t, 64); }
    else { if (d == 128) FDL_QSUM(float, 128); else FDL_QSUM(float, 64); }
#undef FDL_QSUM
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 sgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * a.scan_chunks));
#define FDL_SCAN(T, DD, KB) hipLaunchKernelGGL((block_scan_kernel<T, DD, KB>), sgrid, dim3(kScanThreads), 0, stream, a)
    const bool kb = a.kbar != nullptr;
    if (bf) {
        if (d == 128) { if (kb) FDL_SCAN(uint16_t, 128, true); else FDL_SCAN(uint16_t, 128, false); }
        else { if (kb) FDL_SCAN(uint16_t, 64, true); else FDL_SCAN(uint16_t, 64, false); }
    } else {
        if (d == 128) { if (kb) FDL_SCAN(float, 128, true); else FDL_SCAN(float, 128, false); }
        else { if (kb) FDL_SCAN(float, 64, true); else FDL_SCAN(float, 64, false); }
    }
#undef FDL_SCAN
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(block_select_kernel, dim3(a.B), dim3(256), 0, stream, a, C, block_idx, R_out);
    return hipGetLastError();
}

}  // namespace fdl
