// Prompt-block pruning: block means, relevance R_b and top-C.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
// steps" (4): prompt keys are split into contiguous blocks of bs keys, each
// block is represented by the mean of its keys, the relevance R_b of the
// candidate queries to every block is scored and the C most relevant blocks
// are kept.  R_b = scale * sum_h sum_i q_{h,i} . kbar_{g(h),b}.
//
// The block means depend on the prompt keys only, so they are a separate pass
// (block_means) that a caller can run for every layer ahead of the layer that
// needs them, e.g. on a second stream while earlier layers attend.  Scoring is
// then three small passes; the two that read the queries and the means are spread
// over many workgroups (a single CU pulls only about 20 GB/s from memory, so a
// pass that one workgroup runs is bound by it):
//   block_means        one streaming read of the prompt keys, 16 bytes per lane,
//                      fp64 sums (exact for bf16/fp32 inputs), one rounding of the
//                      mean to fp32.
//   block_qsum         R is linear in the queries: the sum of the query rows of
//                      every 64-row chunk of one KV head's query heads (fp64).
//   block_dots         per (KV head, 32 blocks): the chunk sums added in chunk
//                      order give qsum_g, and qsum_g . kbar_gb is that head's part of R_b.
//   block_select       one workgroup per sequence adds the head parts in head order,
//                      scales by `scale`, and keeps the top-C blocks (lower block
//                      index first among equal scores), ascending.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kThreads = 256;
constexpr int kQsumRows = 64;      // packed query rows per query-sum workgroup
constexpr int kDotBlocks = 32;     // blocks per dot-product workgroup
constexpr int kMeansBlocks = 2;    // blocks per block_means workgroup

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

// kbar[b][g][blk][e] = mean of K[b][g][blk*bs .. min((blk+1)*bs, P))[e], one rounding.
// A workgroup takes kMeansBlocks consecutive blocks and keeps the loads of all of them
// in flight together.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_means_kernel(const BlockArgs a) {
    constexpr int EPP = 16 / sizeof(T);     // elements per 16-byte piece
    constexpr int NP = D / EPP;             // pieces per key row
    constexpr int RG = kThreads / NP;       // rows read together by the workgroup
    constexpr int kBatch = 8;               // loads per thread and block in flight
    __shared__ double s_sum[kMeansBlocks][RG][D];
    const int tid = threadIdx.x;
    const int chunks = (a.nb + kMeansBlocks - 1) / kMeansBlocks;
    const int chunk = blockIdx.x % chunks;
    const int bg = blockIdx.x / chunks;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int piece = tid % NP, rg = tid / NP;
    const T* kbase = static_cast<const T*>(a.k) + b * a.ksb + g * a.ksh + piece * EPP;
    float* out = a.kbar + (static_cast<int64_t>(b) * a.Hkv + g) * a.nb * D;
    const int blk0 = chunk * kMeansBlocks;
    double acc[kMeansBlocks][EPP];
#pragma unroll
    for (int c = 0; c < kMeansBlocks; ++c)
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[c][e] = 0.0;
    // rows lo + rg + RG*u of every block of the chunk; blocks past nb read nothing
    int lo[kMeansBlocks], hi[kMeansBlocks];
#pragma unroll
    for (int c = 0; c < kMeansBlocks; ++c) {
        lo[c] = min(blk0 + c, a.nb - 1) * a.bs;
        hi[c] = blk0 + c < a.nb ? min(lo[c] + a.bs, a.P) : lo[c];
    }
    for (int j0 = rg; j0 < a.bs; j0 += RG * kBatch) {
        u32x4 x[kMeansBlocks][kBatch];
#pragma unroll
        for (int c = 0; c < kMeansBlocks; ++c)
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int j = min(lo[c] + j0 + u * RG, max(hi[c] - 1, lo[c]));
                x[c][u] = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * a.ksr);
            }
#pragma unroll
        for (int c = 0; c < kMeansBlocks; ++c)
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (lo[c] + j0 + u * RG >= hi[c]) continue;
                float v[EPP];
                unpack16<T>(x[c][u], v);
#pragma unroll
                for (int e = 0; e < EPP; ++e) acc[c][e] += static_cast<double>(v[e]);
            }
    }
#pragma unroll
    for (int c = 0; c < kMeansBlocks; ++c)
#pragma unroll
        for (int e = 0; e < EPP; ++e) s_sum[c][rg][piece * EPP + e] = acc[c][e];
    __syncthreads();
    for (int i = tid; i < kMeansBlocks * D; i += kThreads) {
        const int c = i / D, e = i % D;
        if (blk0 + c >= a.nb) continue;
        double s = 0.0;
        for (int r = 0; r < RG; ++r) s += s_sum[c][r][e];
        out[static_cast<int64_t>(blk0 + c) * D + e] = static_cast<float>(s / static_cast<double>(hi[c] - lo[c]));
    }
}

// qpart[b][g][c][e] = sum over the packed rows [64c, 64c + 64) of KV head g of q[..][e] in
// fp64 (packed row p: query head g*Gq + p%Gq, active row p/Gq); zeros past the rows.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_qsum_kernel(const BlockArgs a) {
    constexpr int EPP = 16 / sizeof(T);     // elements per 16-byte piece
    constexpr int NP = D / EPP;             // pieces per row
    constexpr int RG = kThreads / NP;       // row groups
    constexpr int RPT = kQsumRows / RG;     // rows per thread
    static_assert(RPT * RG == kQsumRows, "row split");
    __shared__ double s_q[RG][D];
    const int tid = threadIdx.x;
    const int c = blockIdx.x % a.nchunks;
    const int bg = blockIdx.x / a.nchunks;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows = a.Gq * nq;
    const int piece = tid % NP, rg = tid / NP;
    u32x4 x[RPT];
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        const int p = c * kQsumRows + rg + RG * u;
        x[u] = u32x4{0u, 0u, 0u, 0u};
        if (p < rows) {
            const int r = p / a.Gq, hh = p % a.Gq;
            const int phys = a.q_idx ? max(a.q_idx[static_cast<int64_t>(b) * a.nq_max + r], 0) : r;
            x[u] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.q) + b * a.qsb + (g * a.Gq + hh) * a.qsh +
                                                   static_cast<int64_t>(phys) * a.qsr + piece * EPP);
        }
    }
    double acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
#pragma unroll
    for (int u = 0; u < RPT; ++u) {
        float v[EPP];
        unpack16<T>(x[u], v);
#pragma unroll
        for (int e = 0; e < EPP; ++e) acc[e] += static_cast<double>(v[e]);
    }
#pragma unroll
    for (int e = 0; e < EPP; ++e) s_q[rg][piece * EPP + e] = acc[e];
    __syncthreads();
    double* out = a.qpart + ((static_cast<int64_t>(b) * a.Hkv + g) * a.nchunks + c) * D;
    for (int e = tid; e < D; e += kThreads) {
        double t = 0.0;
        for (int r = 0; r < RG; ++r) t += s_q[r][e];
        out[e] = t;
    }
}

// rpart[b][g][blk] = qsum_g . kbar[b][g][blk] for the kDotBlocks blocks of this workgroup,
// qsum_g being the chunk sums added in chunk order.
template <int D>
__global__ __launch_bounds__(kThreads) void block_dots_kernel(const BlockArgs a) {
    constexpr int LPB = kThreads / kDotBlocks;   // lanes per block
    constexpr int EPL = D / LPB;                 // kbar elements per lane
    static_assert(EPL % 4 == 0, "16-byte kbar pieces");
    __shared__ double s_qsum[D];
    const int tid = threadIdx.x;
    const int nbc = (a.nb + kDotBlocks - 1) / kDotBlocks;
    const int bc = blockIdx.x % nbc;
    const int bg = blockIdx.x / nbc;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    // this workgroup's block means go out first; qsum_g meanwhile
    const int blk = bc * kDotBlocks + tid / LPB, sub = tid % LPB;
    const float* krow = a.kbar_in + ((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + min(blk, a.nb - 1)) * D + sub * EPL;
    f32x4 kx[EPL / 4];
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) kx[i] = *reinterpret_cast<const f32x4*>(krow + 4 * i);
    const double* qp = a.qpart + (static_cast<int64_t>(b) * a.Hkv + g) * a.nchunks * D;
    for (int e = tid; e < D; e += kThreads) {
        double t = 0.0;
        int c = 0;
        for (; c + 8 <= a.nchunks; c += 8) {
            double y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = qp[(c + u) * D + e];
#pragma unroll
            for (int u = 0; u < 8; ++u) t += y[u];
        }
        for (; c < a.nchunks; ++c) t += qp[c * D + e];
        s_qsum[e] = t;
    }
    __syncthreads();
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s = fma(static_cast<double>(kx[i][j]), s_qsum[sub * EPL + 4 * i + j], s);
#pragma unroll
    for (int off = 1; off < LPB; off <<= 1) s += __shfl_xor(s, off, kWave);   // every lane of the block
    if (sub == 0 && blk < a.nb) a.rpart[(static_cast<int64_t>(b) * a.Hkv + g) * a.nb + blk] = s;
}

constexpr int kSelectThreads = 1024;
constexpr int kSelectLds = 2048;   // blocks ranked in LDS
constexpr int kSlices = 4;         // threads summing the head parts of one block

// Up to kSelectThreads blocks are ranked by a distinct 64-bit key: the order-preserving
// image of R_b with its low 11 bits replaced by (2047 - b).  Scores within 2^-41 of each
// other (relative) therefore count as equal, and the lower block index wins, as it does
// for exactly equal scores.
__device__ __forceinline__ uint64_t distinct_key(double r, int blk) {
    return (okey64(r) & ~uint64_t(0x7ff)) | static_cast<uint64_t>(0x7ff - blk);
}

// R_b = scale * sum over g of rpart[b][g][blk] (KV heads in order), then the top-C blocks.
__global__ __launch_bounds__(kSelectThreads) void block_select_kernel(const BlockArgs a, int C,
                                                                       int32_t* block_idx, double* R_out) {
    __shared__ SelectSmem sm;
    __shared__ uint64_t s_key[kSelectLds];
    __shared__ double s_slice[kSlices][kSelectThreads / kSlices];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    // thread slice `slice` sums KV heads [slice*per, (slice+1)*per)
    const int per = (a.Hkv + kSlices - 1) / kSlices;
    double* R = a.rfull + static_cast<int64_t>(b) * a.nb;
    const double* rp = a.rpart + static_cast<int64_t>(b) * a.Hkv * a.nb;
    const int slice = tid / (kSelectThreads / kSlices), lb = tid % (kSelectThreads / kSlices);
    const int g0 = slice * per, g1 = min(a.Hkv, g0 + per);
    for (int blk0 = 0; blk0 < a.nb; blk0 += kSelectThreads / kSlices) {
        const int blk = blk0 + lb;
        double s = 0.0;
        if (blk < a.nb) {
            // 16 loads in flight; head g's part is nb doubles after head g-1's
            for (int g = g0; g < g1; g += 16) {
                double x[16];
#pragma unroll
                for (int u = 0; u < 16; ++u) x[u] = g + u < g1 ? rp[static_cast<int64_t>(g + u) * a.nb + blk] : 0.0;
#pragma unroll
                for (int u = 0; u < 16; ++u) s += x[u];
            }
        }
        s_slice[slice][lb] = s;
        __syncthreads();
        if (slice == 0 && blk < a.nb) {
            double tot = 0.0;
#pragma unroll
            for (int i = 0; i < kSlices; ++i) tot += s_slice[i][lb];
            const double val = tot * static_cast<double>(a.scale);
            if (a.nb <= kSelectThreads) s_key[blk] = distinct_key(val, blk);
            else if (a.nb <= kSelectLds) s_key[blk] = okey64(val);
            else R[blk] = val;
            if (R_out) R_out[static_cast<int64_t>(b) * a.nb + blk] = val;
        }
        __syncthreads();
    }
    __threadfence_block();
    int32_t* out = block_idx + static_cast<int64_t>(b) * C;
    if (a.nb <= kSelectThreads) {
        block_topk_distinct(a.nb, C, [&](int j) { return s_key[j]; }, [](int j) { return j; }, out, C, &sm);
    } else if (a.nb <= kSelectLds) {
        auto key_of = [&](int j, uint64_t* key) -> bool {
            *key = s_key[j];
            return true;
        };
        block_emit_topk<uint64_t>(a.nb, C, key_of, [](int j) { return j; }, out, C, &sm);
    } else {
        auto key_of = [&](int j, uint64_t* key) -> bool {
            *key = okey64(R[j]);
            return true;
        };
        block_emit_topk<uint64_t>(a.nb, C, key_of, [](int j) { return j; }, out, C, &sm);
    }
}

int host_chunks(int Gq, int nq_max) {
    const int64_t c = (static_cast<int64_t>(Gq) * nq_max + kQsumRows - 1) / kQsumRows;
    return static_cast<int>(c < 1 ? 1 : c);
}

}  // namespace

size_t block_workspace_bytes(int B, int Hq, int Hkv, int P, int d, int bs, int nq_max) {
    const int64_t nb = (static_cast<int64_t>(P) + bs - 1) / bs;
    const int chunks = host_chunks(Hq / Hkv, nq_max);
    return round_up(static_cast<size_t>(B) * Hkv * chunks * d * sizeof(double), 256) +   // query chunk sums
           round_up(static_cast<size_t>(B) * Hkv * nb * sizeof(double), 256) +          // per-head R parts
           round_up(static_cast<size_t>(B) * nb * sizeof(double), 256) +                // R
           static_cast<size_t>(B) * Hkv * nb * d * sizeof(float);                       // block means
}

hipError_t launch_block_means(fdl_dtype dtype, int d, const BlockArgs& a, hipStream_t stream) {
    const int chunks = (a.nb + kMeansBlocks - 1) / kMeansBlocks;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * chunks));
#define FDL_MEANS(T, DD) hipLaunchKernelGGL((block_means_kernel<T, DD>), grid, dim3(kThreads), 0, stream, a)
    if (dtype == FDL_BF16) { if (d == 128) FDL_MEANS(uint16_t, 128); else FDL_MEANS(uint16_t, 64); }
    else { if (d == 128) FDL_MEANS(float, 128); else FDL_MEANS(float, 64); }
#undef FDL_MEANS
    return hipGetLastError();
}

hipError_t launch_block_score_topc(fdl_dtype dtype, int d, BlockArgs a, int C, int32_t* block_idx,
                                   double* R_out, void* ws, hipStream_t stream) {
    a.nchunks = host_chunks(a.Gq, a.nq_max);
    uint8_t* w = static_cast<uint8_t*>(ws);
    a.qpart = reinterpret_cast<double*>(w);
    w += round_up(static_cast<size_t>(a.B) * a.Hkv * a.nchunks * d * sizeof(double), 256);
    a.rpart = reinterpret_cast<double*>(w);
    w += round_up(static_cast<size_t>(a.B) * a.Hkv * a.nb * sizeof(double), 256);
    a.rfull = reinterpret_cast<double*>(w);
    w += round_up(static_cast<size_t>(a.B) * a.nb * sizeof(double), 256);
    if (a.k) {
        // means from the keys first: into the caller's kbar when given, else the workspace
        if (!a.kbar) a.kbar = reinterpret_cast<float*>(w);
        hipError_t err = launch_block_means(dtype, d, a, stream);
        if (err != hipSuccess) return err;
    }
    a.kbar_in = a.kbar;
    const dim3 qgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * a.nchunks));
#define FDL_QSUM(T, DD) hipLaunchKernelGGL((block_qsum_kernel<T, DD>), qgrid, dim3(kThreads), 0, stream, a)
    if (dtype == FDL_BF16) { if (d == 128) FDL_QSUM(uint16_t, 128); else FDL_QSUM(uint16_t, 64); }
    else { if (d == 128) FDL_QSUM(float, 128); else FDL_QSUM(float, 64); }
#undef FDL_QSUM
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nbc = (a.nb + kDotBlocks - 1) / kDotBlocks;
    const dim3 dgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * nbc));
    if (d == 128) hipLaunchKernelGGL(block_dots_kernel<128>, dgrid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL(block_dots_kernel<64>, dgrid, dim3(kThreads), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(block_select_kernel, dim3(a.B), dim3(kSelectThreads), 0, stream, a, C, block_idx, R_out);
    return hipGetLastError();
}

}  // namespace fdl
