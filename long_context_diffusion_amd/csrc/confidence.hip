// Token confidence and unmasking: the step after the sparse attention path.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Prerequisites"
// (dLLMs: every [MASK] position gets a distribution over the vocabulary and positions
// are unmasked by confidence) and "Core method" (n(t) tokens are decoded at step t; the
// confidence c_t is what PCGI reads at step t+1).  For each listed masked row the
// confidence is the largest softmax probability of its logits, c = 1 / sum_v
// exp(z_v - max z), and the predicted token is the argmax (lowest id among equal maxima).
// The n(t) rows of highest confidence whose position is still masked are unmasked.
//
// Two kernels, a single read of the logits (the work is bound by HBM bandwidth):
//   conf_partial  one workgroup per (sequence, row, chunk of kChunk logits): the
//                 chunk's max, its argmax and sum of exp(z - max), 16 bytes per lane,
//                 folded across the workgroup.
//   conf_select   one workgroup per sequence: combines the chunks of every row (in
//                 chunk order), ranks the still-masked rows by (confidence, position)
//                 and writes the mask, the tokens, c_t and the unmasked positions.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kChunk = 8192;          // logits per partial workgroup
constexpr int kPartThreads = 256;
constexpr int kSelThreadsU = 1024;
constexpr int kFoldBatch = 8;         // chunk parts loaded together per row
constexpr float kLog2eU = 1.44269504088896340736f;

struct Part {   // one chunk of one row
    float m, s;
    int arg, pad;
};

// (m, s, arg) of two disjoint pieces of a row: the larger max wins the argmax (the lower
// index between equal maxima), the sums are brought to the common max.
__device__ __forceinline__ void fold(float& m, float& s, int& arg, float m2, float s2, int a2) {
    if (m2 > m || (m2 == m && a2 < arg)) {
        const float sc = s * fast_exp2((m - m2) * kLog2eU);
        m = m2;
        s = s2 + sc;
        arg = a2;
    } else {
        s += s2 * fast_exp2((m2 - m) * kLog2eU);
    }
}

template <typename T>
__global__ __launch_bounds__(kPartThreads) void conf_partial_kernel(const T* logits, int64_t lsb, int64_t lsr,
                                                                    const int32_t* n_rows, int m_max, int V,
                                                                    int n_chunks, Part* parts) {
    constexpr int EPV = 16 / sizeof(T);                 // elements per 16-byte load
    constexpr int VPT = kChunk / EPV / kPartThreads;    // loads per thread
    __shared__ float s_m[kPartThreads / kWave], s_s[kPartThreads / kWave];
    __shared__ int s_a[kPartThreads / kWave];
    const int ch = blockIdx.x % n_chunks;
    const int row = (blockIdx.x / n_chunks) % m_max;
    const int b = blockIdx.x / (n_chunks * m_max);
    const int nr = n_rows ? n_rows[b] : m_max;
    if (row >= nr) return;
    const T* z = logits + b * lsb + static_cast<int64_t>(row) * lsr;
    const int lo = ch * kChunk, hi = min(V, lo + kChunk);
    const int tid = threadIdx.x;
    // element e = lo + EPV (tid + kPartThreads u) + j: all loads first, then the folds
    float x[VPT][EPV];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
        const int e0 = lo + EPV * (tid + kPartThreads * u);
        if (e0 + EPV <= hi) {
            const u32x4 w = *reinterpret_cast<const u32x4*>(z + e0);
            if (sizeof(T) == 2) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[u][2 * i] = bf16lo(w[i]);
                    x[u][2 * i + 1] = bf16hi(w[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) x[u][i] = __uint_as_float(w[i]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < EPV; ++j) x[u][j] = e0 + j < hi ? Elem<T>::load(z + e0 + j) : -INFINITY;
        }
    }
    float m = -INFINITY;
    int arg = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < VPT; ++u)
#pragma unroll
        for (int j = 0; j < EPV; ++j) {
            const int e = lo + EPV * (tid + kPartThreads * u) + j;
            if (x[u][j] > m) {   // elements visit in increasing index: the first max is kept
                m = x[u][j];
                arg = e;
            }
        }
    float s = 0.0f;
    if (m > -INFINITY) {
        const float mb = m * kLog2eU;
#pragma unroll
        for (int u = 0; u < VPT; ++u)
#pragma unroll
            for (int j = 0; j < EPV; ++j) s += fast_exp2(fmaf(x[u][j], kLog2eU, -mb));
    }
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const float m2 = __shfl_xor(m, off, kWave), s2 = __shfl_xor(s, off, kWave);
        const int a2 = __shfl_xor(arg, off, kWave);
        if (m2 > -INFINITY) {
            if (m == -INFINITY) {
                m = m2;
                s = s2;
                arg = a2;
            } else {
                fold(m, s, arg, m2, s2, a2);
            }
        }
    }
    const int wv = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
        s_m[wv] = m;
        s_s[wv] = s;
        s_a[wv] = arg;
    }
    __syncthreads();
    if (tid == 0) {
        float M = s_m[0], S = s_s[0];
        int A = s_a[0];
        for (int w = 1; w < kPartThreads / kWave; ++w) {
            if (s_m[w] == -INFINITY) continue;
            if (M == -INFINITY) {
                M = s_m[w];
                S = s_s[w];
                A = s_a[w];
            } else {
                fold(M, S, A, s_m[w], s_s[w], s_a[w]);
            }
        }
        parts[(static_cast<int64_t>(b) * m_max + row) * n_chunks + ch] = Part{M, S, A, 0};
    }
}

__global__ __launch_bounds__(kSelThreadsU) void conf_select_kernel(const Part* parts, int n_chunks, const int32_t* pos,
                                                                   const int32_t* n_rows, int m_max, int L, int n_t,
                                                                   uint8_t* mask, float* conf, int32_t* tokens,
                                                                   int32_t* unmasked) {
    __shared__ SelectSmem sm;
    __shared__ float s_c[kMaxConfRows];
    __shared__ int s_pos[kMaxConfRows];
    __shared__ int s_tok[kMaxConfRows];
    __shared__ int s_sel[kMaxConfRows];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int n = min(n_rows ? n_rows[b] : m_max, m_max);
    const int32_t* pb = pos + static_cast<int64_t>(b) * m_max;
    uint8_t* mb = mask + static_cast<int64_t>(b) * L;
    // combine the chunks of each row in chunk order; s_pos = -1 marks rows that are not
    // candidates (position outside [0, L) or no longer masked)
    int n_cand_local = 0;
    for (int r = tid; r < n; r += kSelThreadsU) {
        const Part* pr = parts + (static_cast<int64_t>(b) * m_max + r) * n_chunks;
        float M = -INFINITY, S = 0.0f;
        int A = 0x7fffffff;
        // the chunks' parts in batches of independent loads, folded in chunk order
        for (int c0 = 0; c0 < n_chunks; c0 += kFoldBatch) {
            Part q[kFoldBatch];
#pragma unroll
            for (int u = 0; u < kFoldBatch; ++u) q[u] = pr[min(c0 + u, n_chunks - 1)];
#pragma unroll
            for (int u = 0; u < kFoldBatch; ++u) {
                if (c0 + u >= n_chunks) break;
                if (c0 + u == 0) {
                    M = q[u].m;
                    S = q[u].s;
                    A = q[u].arg;
                } else {
                    fold(M, S, A, q[u].m, q[u].s, q[u].arg);
                }
            }
        }
        const int p = pb[r];
        const bool cand = p >= 0 && p < L && mb[p] != 0;
        s_c[r] = 1.0f / S;
        s_tok[r] = A;
        s_pos[r] = cand ? p : -1;
        n_cand_local += cand ? 1 : 0;
    }
    int n_cand;
    block_exclusive_sum(n_cand_local, sm.tmp, &n_cand);   // also orders the row writes
    // the n(t) most confident candidates; rows are ranked by (c, lower position) through
    // distinct 64-bit keys and written in row order
    auto key_of = [&](int j, uint64_t* key) -> bool {
        const int p = s_pos[j];
        *key = (static_cast<uint64_t>(okey32(s_c[j])) << 32) | static_cast<uint64_t>(0xffffffffu - static_cast<uint32_t>(p));
        return p >= 0;
    };
    const int cap = min(max(n_t, 0), kMaxConfRows);
    int nsel;
    if (n <= kSelThreadsU) {
        // up to one row per thread: rank by the distinct keys; rows that are not candidates
        // get key 0, below every candidate's, and at most n_cand rows are taken
        auto key_rank = [&](int j) -> uint64_t {
            uint64_t k;
            return key_of(j, &k) ? k : 0ull;
        };
        nsel = block_topk_distinct(n, min(cap, n_cand), key_rank, [](int j) { return j; }, s_sel, cap, &sm);
    } else {
        nsel = block_emit_topk<uint64_t>(n, cap, key_of, [](int j) { return j; }, s_sel, cap, &sm);
    }
    __syncthreads();
    for (int i = tid; i < nsel; i += kSelThreadsU) s_tok[s_sel[i]] |= static_cast<int>(0x80000000u);   // selected flag
    __syncthreads();
    for (int r = tid; r < n; r += kSelThreadsU) {
        const int p = pb[r];
        if (p < 0 || p >= L) continue;
        const bool chosen = s_tok[r] < 0;
        conf[static_cast<int64_t>(b) * L + p] = (chosen || s_pos[r] < 0) ? 0.0f : s_c[r];
        if (chosen) {
            mb[p] = 0;
            if (tokens) tokens[static_cast<int64_t>(b) * L + p] = s_tok[r] & 0x7fffffff;
        }
    }
    if (unmasked) {
        int32_t* ub = unmasked + static_cast<int64_t>(b) * max(n_t, 0);
        for (int i = tid; i < max(n_t, 0); i += kSelThreadsU) ub[i] = i < nsel ? pb[s_sel[i]] : -1;
    }
}

}  // namespace

int conf_chunks(int V) { return (V + kChunk - 1) / kChunk; }

size_t confidence_workspace_bytes(int B, int V, int m_max) {
    return static_cast<size_t>(B) * m_max * conf_chunks(V) * sizeof(Part);
}

hipError_t launch_confidence_unmask(fdl_dtype dtype, int B, int L, int V, const void* logits, int64_t lsb,
                                    int64_t lsr, const int32_t* pos, const int32_t* n_rows, int m_max, int n_t,
                                    uint8_t* mask, float* conf, int32_t* tokens, int32_t* unmasked, void* ws,
                                    hipStream_t stream) {
    const int nc = conf_chunks(V);
    Part* parts = static_cast<Part*>(ws);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * m_max * nc));
    if (dtype == FDL_BF16)
        hipLaunchKernelGGL(conf_partial_kernel<uint16_t>, grid, dim3(kPartThreads), 0, stream,
                           static_cast<const uint16_t*>(logits), lsb, lsr, n_rows, m_max, V, nc, parts);
    else
        hipLaunchKernelGGL(conf_partial_kernel<float>, grid, dim3(kPartThreads), 0, stream,
                           static_cast<const float*>(logits), lsb, lsr, n_rows, m_max, V, nc, parts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(conf_select_kernel, dim3(B), dim3(kSelThreadsU), 0, stream, parts, nc, pos, n_rows, m_max, L,
                       n_t, mask, conf, tokens, unmasked);
    return hipGetLastError();
}

}  // namespace fdl
