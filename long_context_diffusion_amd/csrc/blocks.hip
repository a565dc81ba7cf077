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
// then a small pass over the means:
//   block_means      one streaming read of the prompt keys, 16 bytes per lane,
//                    fp64 sums (exact for bf16/fp32 inputs), one rounding of the
//                    mean to fp32.
//   block_relevance  R is linear in the queries: qsum = sum of the query rows of a
//                    slice of the active rows of one KV head's query heads (fp64),
//                    then that slice's partial R_b = qsum . kbar_b for every block.
//   block_select     sums the partials in a fixed order (KV head, then slice),
//                    scales by scale, and keeps the top-C blocks (lower block index
//                    first among equal scores), ascending.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kThreads = 256;
constexpr int kPartRows = 128;     // active rows per relevance slice (at most kMaxParts slices)
constexpr int kMaxParts = 64;
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

// Relevance slices of sequence b: as many kPartRows-row slices as its active rows
// need, at most a.nparts (the grid's bound); rows are split evenly between them.
__device__ __forceinline__ int relevance_parts(const BlockArgs& a, int rows) {
    return max(1, min(a.nparts, (rows + kPartRows - 1) / kPartRows));
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

// rpart[b][g][part][blk] = qsum_part . kbar[b][g][blk], qsum_part = sum of the query rows of
// slice `part` of the Gq*nq packed rows of KV head g (packed row p: head g*Gq + p%Gq, row p/Gq).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void block_relevance_kernel(const BlockArgs a) {
    constexpr int EPP = 16 / sizeof(T);
    constexpr int NP = D / EPP;
    constexpr int RG = kThreads / NP;
    constexpr int kBatch = 8;
    constexpr int LPB = 4;                  // lanes per block in the dot products
    constexpr int EPL = D / LPB;            // kbar elements per lane
    __shared__ double s_q[RG][D];
    __shared__ double s_qsum[D];
    const int tid = threadIdx.x;
    const int part = blockIdx.x % a.nparts;
    const int bg = blockIdx.x / a.nparts;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows = a.Gq * nq;
    const int parts = relevance_parts(a, rows);
    if (part >= parts) return;
    const int rpp = (rows + parts - 1) / parts;
    const int p_lo = part * rpp, p_hi = min(rows, p_lo + rpp);

    // the block means of the first pass go out before the queries: both round trips overlap
    const float* kb = a.kbar_in + (static_cast<int64_t>(b) * a.Hkv + g) * a.nb * D;
    const int sub = tid % LPB;
    f32x4 kx[EPL / 4];
    {
        const int blk = min(tid / LPB, a.nb - 1);
        const float* row = kb + static_cast<int64_t>(blk) * D + sub * EPL;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i) kx[i] = *reinterpret_cast<const f32x4*>(row + 4 * i);
    }

    // ---- qsum of this slice (fp64)
    const int piece = tid % NP, rg = tid / NP;
    double acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
    // packed row p = r * Gq + hh (query head g*Gq + hh, row r); this thread's rows advance by RG
    const int step_r = RG / a.Gq, step_h = RG % a.Gq;
    int r_cur = (p_lo + rg) / a.Gq, h_cur = (p_lo + rg) % a.Gq;
    for (int p0 = p_lo + rg; p0 < p_hi; p0 += RG * kBatch) {
        int64_t off[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const bool in = p0 + u * RG < p_hi;
            const int r = in ? r_cur : 0, hh = in ? h_cur : 0;
            const int phys = a.q_idx ? max(a.q_idx[static_cast<int64_t>(b) * a.nq_max + r], 0) : r;
            off[u] = b * a.qsb + (g * a.Gq + hh) * a.qsh + static_cast<int64_t>(phys) * a.qsr + piece * EPP;
            r_cur += step_r;
            h_cur += step_h;
            if (h_cur >= a.Gq) { h_cur -= a.Gq; ++r_cur; }
        }
        u32x4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) x[u] = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.q) + off[u]);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (p0 + u * RG >= p_hi) continue;
            float v[EPP];
            unpack16<T>(x[u], v);
#pragma unroll
            for (int e = 0; e < EPP; ++e) acc[e] += static_cast<double>(v[e]);
        }
    }
#pragma unroll
    for (int e = 0; e < EPP; ++e) s_q[rg][piece * EPP + e] = acc[e];
    __syncthreads();
    for (int e = tid; e < D; e += kThreads) {
        double s = 0.0;
        for (int r = 0; r < RG; ++r) s += s_q[r][e];
        s_qsum[e] = s;
    }
    __syncthreads();

    // ---- partial relevance of every block: LPB consecutive lanes share a block
    double* rp = a.rpart + ((static_cast<int64_t>(b) * a.Hkv + g) * a.nparts + part) * a.nb;
    for (int blk = tid / LPB; blk < a.nb; blk += kThreads / LPB) {
        f32x4 x[EPL / 4];
        if (blk < kThreads / LPB) {
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i) x[i] = kx[i];
        } else {
            const float* row = kb + static_cast<int64_t>(blk) * D + sub * EPL;
#pragma unroll
            for (int i = 0; i < EPL / 4; ++i) x[i] = *reinterpret_cast<const f32x4*>(row + 4 * i);
        }
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < EPL / 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) s = fma(static_cast<double>(x[i][j]), s_qsum[sub * EPL + 4 * i + j], s);
        s += __shfl_xor(s, 1, 64);   // (s0 + s1) + (s2 + s3) in every lane of the four
        s += __shfl_xor(s, 2, 64);
        if (sub == 0) rp[blk] = s;
    }
}

constexpr int kSelectThreads = 1024;
constexpr int kSelectLds = 2048;   // blocks ranked in LDS
constexpr int kSlices = 4;         // threads summing the partials of one block

__global__ __launch_bounds__(kSelectThreads) void block_select_kernel(const BlockArgs a, int C,
                                                                       int32_t* block_idx, double* R_out) {
    __shared__ SelectSmem sm;
    __shared__ uint64_t s_key[kSelectLds];
    __shared__ double s_slice[kSlices][kSelectThreads / kSlices];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int parts = relevance_parts(a, a.Gq * nq);
    // thread slice `slice` sums KV heads [slice*per, (slice+1)*per) x every slice of rows
    const int per = (a.Hkv + kSlices - 1) / kSlices;
    double* R = a.rfull + static_cast<int64_t>(b) * a.nb;
    const double* rp = a.rpart + static_cast<int64_t>(b) * a.Hkv * a.nparts * a.nb;
    const int slice = tid / (kSelectThreads / kSlices), lb = tid % (kSelectThreads / kSlices);
    const int g0 = slice * per, g1 = min(a.Hkv, g0 + per);
    const int terms = max(g1 - g0, 0) * parts;
    for (int blk0 = 0; blk0 < a.nb; blk0 += kSelectThreads / kSlices) {
        const int blk = blk0 + lb;
        double s = 0.0;
        if (blk < a.nb) {
            // term t: KV head g0 + t / parts, row slice t % parts; addresses advance without a division
            int g = g0, pi = 0;
            for (int t = 0; t < terms; t += 16) {
                double x[16];
                int gg = g, pp = pi;
#pragma unroll
                for (int u = 0; u < 16; ++u) {
                    const bool in = t + u < terms;
                    const double y = rp[(static_cast<int64_t>(in ? gg : g0) * a.nparts + (in ? pp : 0)) * a.nb + blk];
                    x[u] = in ? y : 0.0;
                    if (++pp == parts) { pp = 0; ++gg; }
                }
#pragma unroll
                for (int u = 0; u < 16; ++u) s += x[u];
                g = gg;
                pi = pp;
            }
        }
        s_slice[slice][lb] = s;
        __syncthreads();
        if (slice == 0 && blk < a.nb) {
            double tot = 0.0;
#pragma unroll
            for (int i = 0; i < kSlices; ++i) tot += s_slice[i][lb];
            const double val = tot * static_cast<double>(a.scale);
            if (a.nb <= kSelectLds) s_key[blk] = okey64(val);
            else R[blk] = val;
            if (R_out) R_out[static_cast<int64_t>(b) * a.nb + blk] = val;
        }
        __syncthreads();
    }
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

int host_parts(int Gq, int nq_max) {
    const int64_t parts = (static_cast<int64_t>(Gq) * nq_max + kPartRows - 1) / kPartRows;
    return static_cast<int>(parts < 1 ? 1 : parts > kMaxParts ? kMaxParts : parts);
}

}  // namespace

size_t block_workspace_bytes(int B, int Hq, int Hkv, int P, int d, int bs, int nq_max) {
    const int64_t nb = (static_cast<int64_t>(P) + bs - 1) / bs;
    const int parts = host_parts(Hq / Hkv, nq_max);
    return round_up(static_cast<size_t>(B) * Hkv * parts * nb * sizeof(double), 256) +   // partial R
           round_up(static_cast<size_t>(B) * nb * sizeof(double), 256) +                 // R
           static_cast<size_t>(B) * Hkv * nb * d * sizeof(float);                        // block means
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
    a.nparts = host_parts(a.Gq, a.nq_max);
    uint8_t* w = static_cast<uint8_t*>(ws);
    a.rpart = reinterpret_cast<double*>(w);
    w += round_up(static_cast<size_t>(a.B) * a.Hkv * a.nparts * a.nb * sizeof(double), 256);
    a.rfull = reinterpret_cast<double*>(w);
    w += round_up(static_cast<size_t>(a.B) * a.nb * sizeof(double), 256);
    if (a.k) {
        // means from the keys first: into the caller's kbar when given, else the workspace
        if (!a.kbar) a.kbar = reinterpret_cast<float*>(w);
        hipError_t err = launch_block_means(dtype, d, a, stream);
        if (err != hipSuccess) return err;
    }
    a.kbar_in = a.kbar;
    const dim3 rgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * a.nparts));
#define FDL_REL(T, DD) hipLaunchKernelGGL((block_relevance_kernel<T, DD>), rgrid, dim3(kThreads), 0, stream, a)
    if (dtype == FDL_BF16) { if (d == 128) FDL_REL(uint16_t, 128); else FDL_REL(uint16_t, 64); }
    else { if (d == 128) FDL_REL(float, 128); else FDL_REL(float, 64); }
#undef FDL_REL
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(block_select_kernel, dim3(a.B), dim3(kSelectThreads), 0, stream, a, C, block_idx, R_out);
    return hipGetLastError();
}

}  // namespace fdl
