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
// then two small passes; the one that reads the queries and the means is spread over
// many workgroups (a single CU pulls only about 20 GB/s from memory, so a pass that
// one workgroup runs is bound by it):
//   block_means        one streaming read of the prompt keys, 16 bytes per lane,
//                      fp64 sums, one rounding of the mean to fp32.  The fp64 sum of a
//                      block is exact (so any order of the additions gives it) while the
//                      binary exponents of its nonzero keys span at most 29 - log2(bs)
//                      (fp32 keys) or 45 - log2(bs) (bf16 keys); beyond that range the
//                      result can depend on the order in the last bit.
//   block_dots         per (KV head g, 4096/d blocks): R is linear in the queries, so the
//                      workgroup first sums the query rows of g's query heads (fp64),
//                      qsum_g, and qsum_g . kbar_gb is that head's part of R_b.
//   block_select       one workgroup per sequence adds the head parts in head order,
//                      scales by `scale`, and keeps the top-C blocks (lower block
//                      index first among equal scores), ascending.
// Variants of the relevance (Summary, "Independent weaknesses"): with kScorePerHead every
// KV head keeps its own top-C from its own part of R (block_select runs per (sequence, KV
// head)); with kScoreMax a block scores by its strongest single query,
//   block_max          per (KV head g, 16 blocks): max over the query rows of g's query
//                      heads of q . kbar_gb, each dot in fp64 (the products of bf16 or
//                      fp32 queries and fp32 means are exact in fp64); the maximum does not
//                      depend on the order the rows are visited in,
// and block_select takes the max over the KV heads instead of the sum.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kThreads = 256;
constexpr int kQRows = 1024;       // packed query rows whose indices are staged in LDS at once
constexpr int kDotThreads = 512;   // threads of a dot-product workgroup
// blocks per dot-product workgroup: D / 16 lanes per block, 16 mean elements per lane (every
// workgroup of a KV head sums the same query rows, so fewer, larger workgroups read less)
__host__ __device__ constexpr int dot_blocks(int d) { return kDotThreads * 16 / d; }
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
__global__ __launch_bounds__(kThreads) void block_means_kernel(const BlockArgs a, int wg0) {
    constexpr int EPP = 16 / sizeof(T);     // elements per 16-byte piece
    constexpr int NP = D / EPP;             // pieces per key row
    constexpr int RG = kThreads / NP;       // rows read together by the workgroup
    constexpr int kBatch = 8;               // loads per thread and block in flight
    constexpr int kWaves = kThreads / kWave;
    // one row of sums per wave, element-major: s_sum[c][w][e][piece]
    __shared__ double s_sum[kMeansBlocks][kWaves][EPP][NP];
    const int tid = threadIdx.x;
    const int chunks = (a.nb + kMeansBlocks - 1) / kMeansBlocks;
    const int wg = wg0 + static_cast<int>(blockIdx.x);   // launches of one wave each: see launch_block_means
    const int chunk = wg % chunks;
    const int bg = wg / chunks;
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
                x[c][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(j) * a.ksr));
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
    // the row groups of a wave (lanes NP apart) fold with shuffles; within the exponent range
    // stated at the top the fp64 sums are exact, so the order of the additions does not change them
#pragma unroll
    for (int c = 0; c < kMeansBlocks; ++c)
#pragma unroll
        for (int e = 0; e < EPP; ++e)
#pragma unroll
            for (int off = NP; off < kWave; off <<= 1) acc[c][e] += __shfl_xor(acc[c][e], off, kWave);
    const int wv = tid / kWave;
    if ((tid % kWave) < NP) {
#pragma unroll
        for (int c = 0; c < kMeansBlocks; ++c)
#pragma unroll
            for (int e = 0; e < EPP; ++e) s_sum[c][wv][e][piece] = acc[c][e];
    }
    __syncthreads();
    for (int i = tid; i < kMeansBlocks * D; i += kThreads) {
        const int c = i / D, ep = i % D;   // ep = e * NP + piece: element piece * EPP + e
        if (blk0 + c >= a.nb) continue;
        const int e = ep / NP, pc = ep % NP;
        double s = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += s_sum[c][w][e][pc];
        out[static_cast<int64_t>(blk0 + c) * D + pc * EPP + e] = static_cast<float>(s / static_cast<double>(hi[c] - lo[c]));
    }
}

// rpart[b][g][blk] = qsum_g . kbar[b][g][blk] for the dot_blocks(D) blocks of this workgroup,
// where qsum_g is the fp64 sum of the packed query rows p < Gq * nq of KV head g (query head
// g*Gq + p%Gq, active row p/Gq).  Row group rg of the workgroup sums rows rg, rg + RG, ...
// in order; the row groups of a wave then fold with shuffles and the waves add in order.  The block means go out
// first, the query-row indices of up to kQRows rows are staged in LDS, and each thread
// loads 16 rows at once, then adds them (one round of loads covers 16 RG rows: 512 rows
// for bf16, d = 128, so the rows of a 32K step's 452 active queries arrive in one round
// trip; two rounds of 8, the second in flight during the first's additions, took 9.0
// against 8.6 us a call in a replayed 32K step).
template <typename T, int D>
__global__ __launch_bounds__(kDotThreads) void block_dots_kernel(const BlockArgs a) {
    constexpr int EPP = 16 / sizeof(T);             // elements per 16-byte piece
    constexpr int NP = D / EPP;                     // pieces per row
    constexpr int RG = kDotThreads / NP;            // row groups
    constexpr int kDotBlocks = dot_blocks(D);
    constexpr int LPB = kDotThreads / kDotBlocks;   // lanes per block
    constexpr int EPL = D / LPB;                 // kbar elements per lane
    constexpr int kBatch = 16;
    static_assert(EPL % 4 == 0, "16-byte kbar pieces");
    constexpr int kWaves = kDotThreads / kWave;
    __shared__ double s_q[kWaves][EPP][NP];      // one row of sums per wave, element-major
    __shared__ double s_qsum[D];
    __shared__ int s_phys[kQRows];
    const int tid = threadIdx.x;
    const int nbc = (a.nb + kDotBlocks - 1) / kDotBlocks;
    const int bc = blockIdx.x % nbc;
    const int bg = blockIdx.x / nbc;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int blk = bc * kDotBlocks + tid / LPB, sub = tid % LPB;
    const float* krow = a.kbar_in + ((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + min(blk, a.nb - 1)) * D + sub * EPL;
    f32x4 kx[EPL / 4];
#pragma unroll
    for (int i = 0; i < EPL / 4; ++i) kx[i] = *reinterpret_cast<const f32x4*>(krow + 4 * i);

    const int piece = tid % NP, rg = tid / NP;
    const T* qhead = static_cast<const T*>(a.q) + b * a.qsb + static_cast<int64_t>(g) * a.Gq * a.qsh + piece * EPP;
    // the row indices of a chunk are staged for up to Gq * nq_max rows, so the first chunk's
    // index loads go out together with the row count instead of after it
    const int rows_max = a.Gq * a.nq_max;
    auto stage = [&](int c0) __attribute__((always_inline)) {
        const int cn = min(kQRows, rows_max - c0);
        for (int i = tid; i < cn; i += kDotThreads) {
            const int r = (c0 + i) / a.Gq;
            s_phys[i] = a.q_idx ? max(a.q_idx[static_cast<int64_t>(b) * a.nq_max + r], 0) : r;
        }
    };
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    stage(0);
    __syncthreads();
    const int rows = min(a.Gq * nq, rows_max);
    double acc[EPP];
#pragma unroll
    for (int e = 0; e < EPP; ++e) acc[e] = 0.0;
    for (int c0 = 0; c0 < rows; c0 += kQRows) {
        if (c0 > 0) {
            __syncthreads();   // the previous chunk's indices are no longer read
            stage(c0);
            __syncthreads();
        }
        const int cn = min(kQRows, rows - c0);
        auto row_ptr = [&](int i) {   // row i of the chunk (i < cn)
            const int hh = (c0 + i) % a.Gq;
            return qhead + hh * a.qsh + static_cast<int64_t>(s_phys[i]) * a.qsr;
        };
        auto load = [&](int i0, u32x4 (&x)[kBatch]) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                const int i = i0 + RG * u;
                x[u] = i < cn ? *reinterpret_cast<const u32x4*>(row_ptr(i)) : u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto add = [&](const u32x4 (&x)[kBatch], int i0) __attribute__((always_inline)) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u) {
                if (i0 + RG * u >= cn) break;
                float v[EPP];
                unpack16<T>(x[u], v);
#pragma unroll
                for (int e = 0; e < EPP; ++e) acc[e] += static_cast<double>(v[e]);
            }
        };
        for (int i0 = rg; i0 < cn; i0 += RG * kBatch) {
            u32x4 x[kBatch];
            load(i0, x);
            add(x, i0);
        }
    }
    // the row groups of a wave (lanes NP apart) fold with shuffles, then the waves in order
#pragma unroll
    for (int e = 0; e < EPP; ++e)
#pragma unroll
        for (int off = NP; off < kWave; off <<= 1) acc[e] += __shfl_xor(acc[e], off, kWave);
    if ((tid % kWave) < NP) {
#pragma unroll
        for (int e = 0; e < EPP; ++e) s_q[tid / kWave][e][piece] = acc[e];
    }
    __syncthreads();
    for (int ep = tid; ep < D; ep += kDotThreads) {   // ep = e * NP + piece: element piece * EPP + e
        const int e = ep / NP, pc = ep % NP;
        double t = 0.0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) t += s_q[w][e][pc];
        s_qsum[pc * EPP + e] = t;
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

constexpr int kMaxThreads = 512;
constexpr int kMaxBlocks = 16;    // blocks per block_max workgroup

// rpart[b][g][blk] = max over packed rows p < Gq * nq of q_p . kbar[b][g][blk] (-inf with no
// rows).  Every wave covers all kMaxBlocks blocks of the workgroup: lanes 4j .. 4j+3 hold
// block j's mean in four slices of D/4 elements (fp64), and each row's dot is the sum of the
// four slice dots (two shuffles).  Waves take rows w, w + waves, ..., a batch of them in
// flight (32 loads of 16 bytes per lane); the per-wave maxima combine through LDS.
template <typename T, int D>
__global__ __launch_bounds__(kMaxThreads) void block_max_kernel(const BlockArgs a) {
    constexpr int SL = 4;                       // lanes per block
    constexpr int EPL = D / SL;                 // elements per lane
    constexpr int EPP = 16 / sizeof(T);         // elements per 16-byte load
    constexpr int NLD = EPL / EPP;              // loads per lane and row
    constexpr int kWaves = kMaxThreads / kWave;
    constexpr int kMaxBatch = 32 / NLD > 2 ? 32 / NLD : 2;   // query rows in flight per wave
    static_assert(kWave / SL == kMaxBlocks, "one wave covers the workgroup's blocks");
    __shared__ double s_m[kWaves][kMaxBlocks];
    __shared__ int s_phys[kQRows];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int nbc = (a.nb + kMaxBlocks - 1) / kMaxBlocks;
    const int bc = blockIdx.x % nbc;
    const int bg = blockIdx.x / nbc;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int j = lane / SL, sl = lane % SL;
    const int blk = bc * kMaxBlocks + j;
    const float* krow = a.kbar_in + ((static_cast<int64_t>(b) * a.Hkv + g) * a.nb + min(blk, a.nb - 1)) * D + sl * EPL;
    double kv[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) kv[e] = static_cast<double>(krow[e]);
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows = min(a.Gq * nq, a.Gq * a.nq_max);
    const T* qhead = static_cast<const T*>(a.q) + b * a.qsb + static_cast<int64_t>(g) * a.Gq * a.qsh + sl * EPL;
    double m = -INFINITY;
    for (int c0 = 0; c0 < rows; c0 += kQRows) {
        const int cn = min(kQRows, rows - c0);
        __syncthreads();   // the previous chunk's indices are no longer read
        for (int i = tid; i < cn; i += kMaxThreads) {
            const int r = (c0 + i) / a.Gq;
            s_phys[i] = a.q_idx ? max(a.q_idx[static_cast<int64_t>(b) * a.nq_max + r], 0) : r;
        }
        __syncthreads();
        for (int i0 = wv; i0 < cn; i0 += kWaves * kMaxBatch) {
            u32x4 x[kMaxBatch][NLD];
#pragma unroll
            for (int u = 0; u < kMaxBatch; ++u) {
                const int i = min(i0 + kWaves * u, cn - 1);
                const T* qrow = qhead + ((c0 + i) % a.Gq) * a.qsh + static_cast<int64_t>(s_phys[i]) * a.qsr;
#pragma unroll
                for (int t = 0; t < NLD; ++t) x[u][t] = *reinterpret_cast<const u32x4*>(qrow + t * EPP);
            }
#pragma unroll
            for (int u = 0; u < kMaxBatch; ++u) {
                double s = 0.0;
#pragma unroll
                for (int t = 0; t < NLD; ++t) {
                    float v[EPP];
                    unpack16<T>(x[u][t], v);
#pragma unroll
                    for (int e = 0; e < EPP; ++e) s = fma(static_cast<double>(v[e]), kv[t * EPP + e], s);
                }
                s += __shfl_xor(s, 1, kWave);
                s += __shfl_xor(s, 2, kWave);
                if (i0 + kWaves * u < cn) m = fmax(m, s);
            }
        }
    }
    if (sl == 0) s_m[wv][j] = m;
    __syncthreads();
    if (tid < kMaxBlocks) {
        double mm = s_m[0][tid];
        for (int w = 1; w < kWaves; ++w) mm = fmax(mm, s_m[w][tid]);
        const int bk = bc * kMaxBlocks + tid;
        if (bk < a.nb) a.rpart[(static_cast<int64_t>(b) * a.Hkv + g) * a.nb + bk] = mm;
    }
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

// R_b = scale * sum over g of rpart[b][g][blk] (KV heads in order; their max with
// kScoreMax), then the top-C blocks.  With kScorePerHead one workgroup per (b, g) keeps the
// top-C of scale * rpart[b][g][:] in block_idx[b][g] (R_out [b][g] likewise).
__global__ __launch_bounds__(kSelectThreads) void block_select_kernel(const BlockArgs a, int C,
                                                                       int32_t* block_idx, double* R_out) {
    __shared__ SelectSmem sm;
    __shared__ uint64_t s_key[kSelectLds];
    __shared__ double s_slice[kSlices][kSelectThreads / kSlices];
    const bool per_head = (a.mode & kScorePerHead) != 0, use_max = (a.mode & kScoreMax) != 0;
    const int li = blockIdx.x;   // list: b, or b * Hkv + g per head
    const int b = per_head ? li / a.Hkv : li;
    const int gh = per_head ? li % a.Hkv : 0;
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
        if (blk < a.nb && !per_head && !use_max) {
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
            if (per_head) {
                tot = rp[static_cast<int64_t>(gh) * a.nb + blk];
            } else if (use_max) {
                tot = -INFINITY;
                for (int g = 0; g < a.Hkv; ++g) tot = fmax(tot, rp[static_cast<int64_t>(g) * a.nb + blk]);
            } else {
#pragma unroll
                for (int i = 0; i < kSlices; ++i) tot += s_slice[i][lb];
            }
            const double val = tot * static_cast<double>(a.scale);
            if (a.nb <= kSelectThreads) s_key[blk] = distinct_key(val, blk);
            else if (a.nb <= kSelectLds) s_key[blk] = okey64(val);
            else if (!per_head) R[blk] = val;
            if (R_out) R_out[static_cast<int64_t>(li) * a.nb + blk] = val;
        }
        __syncthreads();
    }
    __threadfence_block();
    int32_t* out = block_idx + static_cast<int64_t>(li) * C;
    if (a.nb <= kSelectThreads) {
        block_topk_distinct(a.nb, C, [&](int j) { return s_key[j]; }, [](int j) { return j; }, out, C, &sm);
    } else if (a.nb <= kSelectLds) {
        auto key_of = [&](int j, uint64_t* key) -> bool {
            *key = s_key[j];
            return true;
        };
        block_emit_topk<uint64_t>(a.nb, C, key_of, [](int j) { return j; }, out, C, &sm);
    } else if (per_head) {
        const double* rg = rp + static_cast<int64_t>(gh) * a.nb;
        auto key_of = [&](int j, uint64_t* key) -> bool {
            *key = okey64(rg[j] * static_cast<double>(a.scale));
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

}  // namespace

size_t block_workspace_bytes(int B, int Hq, int Hkv, int P, int d, int bs, int nq_max) {
    (void)Hq;
    (void)nq_max;
    const int64_t nb = (static_cast<int64_t>(P) + bs - 1) / bs;
    return round_up(static_cast<size_t>(B) * Hkv * nb * sizeof(double), 256) +          // per-head R parts
           round_up(static_cast<size_t>(B) * nb * sizeof(double), 256) +                // R
           static_cast<size_t>(B) * Hkv * nb * d * sizeof(float);                       // block means
}

// Workgroups of block_means_kernel<T, D> the whole device holds at once (CUs x resident
// workgroups per CU), queried once per device; 0 when the query fails.
template <typename T, int D>
int64_t means_wave() {
    static int64_t cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0 ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, block_means_kernel<T, D>, kThreads, 0) != hipSuccess ||
            per_cu <= 0)
            cached[dev] = -1;
        else
            cached[dev] = static_cast<int64_t>(cus) * per_cu;
    }
    return cached[dev] > 0 ? cached[dev] : 0;
}

// The grid goes out as launches of at most one wave of resident workgroups each.  The means
// usually run on a second stream beside the layers' own kernels; between two launches the
// other stream's kernels are dispatched, instead of waiting behind the tail of a grid of
// several waves.  On the 32K step (4032 workgroups a layer, 1024 resident) one-wave launches
// took the replayed step from 5.15-5.17 to 4.94-5.01 ms (alternating runs on one box);
// splitting each layer's grid in two launches changed nothing and in eight (half a wave
// each) made the step slower.
template <typename T, int D>
void launch_means_waves(const BlockArgs& a, int64_t total, hipStream_t stream) {
    const int64_t wave = means_wave<T, D>();
    const int64_t step = wave > 0 ? wave : total;
    for (int64_t w0 = 0; w0 < total; w0 += step) {
        const int64_t n = total - w0 < step ? total - w0 : step;
        hipLaunchKernelGGL((block_means_kernel<T, D>), dim3(static_cast<unsigned>(n)), dim3(kThreads), 0, stream, a,
                           static_cast<int>(w0));
    }
}

hipError_t launch_block_means(fdl_dtype dtype, int d, const BlockArgs& a, hipStream_t stream) {
    const int chunks = (a.nb + kMeansBlocks - 1) / kMeansBlocks;
    const int64_t total = static_cast<int64_t>(a.B) * a.Hkv * chunks;
    if (dtype == FDL_BF16) {
        if (d == 128) launch_means_waves<uint16_t, 128>(a, total, stream);
        else launch_means_waves<uint16_t, 64>(a, total, stream);
    } else {
        if (d == 128) launch_means_waves<float, 128>(a, total, stream);
        else launch_means_waves<float, 64>(a, total, stream);
    }
    return hipGetLastError();
}

hipError_t launch_block_score_topc(fdl_dtype dtype, int d, BlockArgs a, int C, int32_t* block_idx,
                                   double* R_out, void* ws, hipStream_t stream) {
    uint8_t* w = static_cast<uint8_t*>(ws);
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
    if (a.mode & kScoreMax) {
        const int nbc = (a.nb + kMaxBlocks - 1) / kMaxBlocks;
        const dim3 mgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * nbc));
#define FDL_MAXK(T, DD) hipLaunchKernelGGL((block_max_kernel<T, DD>), mgrid, dim3(kMaxThreads), 0, stream, a)
        if (dtype == FDL_BF16) { if (d == 128) FDL_MAXK(uint16_t, 128); else FDL_MAXK(uint16_t, 64); }
        else { if (d == 128) FDL_MAXK(float, 128); else FDL_MAXK(float, 64); }
#undef FDL_MAXK
    } else {
        const int nbc = (a.nb + dot_blocks(d) - 1) / dot_blocks(d);
        const dim3 dgrid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * nbc));
#define FDL_DOTS(T, DD) hipLaunchKernelGGL((block_dots_kernel<T, DD>), dgrid, dim3(kDotThreads), 0, stream, a)
        if (dtype == FDL_BF16) { if (d == 128) FDL_DOTS(uint16_t, 128); else FDL_DOTS(uint16_t, 64); }
        else { if (d == 128) FDL_DOTS(float, 128); else FDL_DOTS(float, 64); }
#undef FDL_DOTS
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int lists = (a.mode & kScorePerHead) ? a.B * a.Hkv : a.B;
    hipLaunchKernelGGL(block_select_kernel, dim3(lists), dim3(kSelectThreads), 0, stream, a, C, block_idx, R_out);
    return hipGetLastError();
}

}  // namespace fdl
