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
//   conf_partial  one workgroup of 1024 threads per (sequence, row): the row's max, its
//                 argmax and sum of exp(z - max), streamed in rounds of 16-byte loads per
//                 lane (the next round's loads in flight while one is folded into each
//                 thread's running state), then folded across the workgroup once.
//   conf_select   one workgroup per sequence: ranks the still-masked rows by
//                 (confidence, position) and writes the mask, the tokens, c_t and the
//                 unmasked positions.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kRowThreads = 1024;     // threads of a row's workgroup
constexpr int kRowLoads = 2;          // 16-byte loads per thread and round
constexpr int kSelThreadsU = 1024;
constexpr float kLog2eU = 1.44269504088896340736f;

struct Part {   // one row: max, sum of exp(z - max), argmax
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

// Folds the N values x (x[i] at index idx(i), increasing) into one thread's running
// (max m, sum s of exp(z - m), argmax).  The values' max is a max tree; only when it
// exceeds the running max (rare once a row's first values are in) are its first position
// found and s brought to the new max; then every value adds exp(z - m).
template <int N, typename Idx>
__device__ __forceinline__ void fold_values(const float (&x)[N], Idx idx, float& m, float& s, int& arg) {
    float rm = x[0];
#pragma unroll
    for (int i = 1; i < N; ++i) rm = fmaxf(rm, x[i]);
    if (rm > m) {
        int ra = idx(N - 1);
#pragma unroll
        for (int i = N - 2; i >= 0; --i) ra = x[i] == rm ? idx(i) : ra;   // the first one equal to rm
        s = m == -INFINITY ? 0.0f : s * fast_exp2((m - rm) * kLog2eU);
        m = rm;
        arg = ra;
    }
    if (m == -INFINITY) return;   // nothing but -inf so far
    const float mb = m * kLog2eU;
#pragma unroll
    for (int i = 0; i < N; ++i) s += fast_exp2(fmaf(x[i], kLog2eU, -mb));
}

template <typename T>
__global__ __launch_bounds__(kRowThreads) void conf_partial_kernel(const T* logits, int64_t lsb, int64_t lsr,
                                                                  const int32_t* n_rows, int m_max, int V,
                                                                  Part* parts) {
    constexpr int EPV = 16 / sizeof(T);                  // elements per 16-byte load
    constexpr int kRound = kRowThreads * kRowLoads * EPV;   // logits per round
    __shared__ float s_m[kRowThreads / kWave], s_s[kRowThreads / kWave];
    __shared__ int s_a[kRowThreads / kWave];
    const int row = blockIdx.x % m_max;
    const int b = blockIdx.x / m_max;
    const int nr = n_rows ? n_rows[b] : m_max;
    if (row >= nr) return;
    const T* z = logits + b * lsb + static_cast<int64_t>(row) * lsr;
    const int tid = threadIdx.x;
    const int n_rounds = (V + kRound - 1) / kRound;
    // round r, load u of this thread: elements r kRound + EPV (tid + kRowThreads u) + 0 .. EPV-1,
    // read as one 16-byte load when all of them exist; the loads of round r + 1 go out
    // before round r is folded
    auto load_round = [&](int r, u32x4 (&w)[kRowLoads]) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
            const int e0 = r * kRound + EPV * (tid + kRowThreads * u);
            w[u] = e0 + EPV <= V ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + e0))
                                  : u32x4{0u, 0u, 0u, 0u};
        }
    };
    float m = -INFINITY, s = 0.0f;
    int arg = 0x7fffffff;
    u32x4 cur[kRowLoads], nxt[kRowLoads];
    load_round(0, cur);
    for (int r = 0; r < n_rounds; ++r) {
        if (r + 1 < n_rounds) load_round(r + 1, nxt);
        float x[kRowLoads * EPV];
        const int base = r * kRound + EPV * tid;
#pragma unroll
        for (int u = 0; u < kRowLoads; ++u) {
            const int e0 = base + kRowThreads * EPV * u;
            if (e0 + EPV <= V) {
                if (sizeof(T) == 2) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[EPV * u + 2 * i] = bf16lo(cur[u][i]);
                        x[EPV * u + 2 * i + 1] = bf16hi(cur[u][i]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[EPV * u + i] = __uint_as_float(cur[u][i]);
                }
            } else {
                // the row's last, partial vector (or past the row): element by element
#pragma unroll
                for (int j = 0; j < EPV; ++j) x[EPV * u + j] = e0 + j < V ? Elem<T>::load(z + e0 + j) : -INFINITY;
            }
        }
        // the thread's values of this round in increasing index: value EPV u + j is element
        // base + kRowThreads EPV u + j
        fold_values(x, [&](int i) { return base + kRowThreads * EPV * (i / EPV) + i % EPV; }, m, s, arg);
        if (r + 1 < n_rounds) {
#pragma unroll
            for (int u = 0; u < kRowLoads; ++u) cur[u] = nxt[u];
        }
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
        for (int w = 1; w < kRowThreads / kWave; ++w) {
            if (s_m[w] == -INFINITY) continue;
            if (M == -INFINITY) {
                M = s_m[w];
                S = s_s[w];
                A = s_a[w];
            } else {
                fold(M, S, A, s_m[w], s_s[w], s_a[w]);
            }
        }
        parts[static_cast<int64_t>(b) * m_max + row] = Part{M, S, A, 0};
    }
}

__global__ __launch_bounds__(kSelThreadsU) void conf_select_kernel(const Part* parts, const int32_t* pos,
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
    // each row's (max, sum, argmax); s_pos = -1 marks rows that are not candidates
    // (position outside [0, L) or no longer masked)
    int n_cand_local = 0;
    for (int r = tid; r < n; r += kSelThreadsU) {
        const Part q = parts[static_cast<int64_t>(b) * m_max + r];
        const float S = q.s;
        const int A = q.arg;
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


size_t confidence_workspace_bytes(int B, int V, int m_max) {
    return V > 0 ? static_cast<size_t>(B) * m_max * sizeof(Part) : 0;   // one part per row
}

hipError_t launch_confidence_unmask(fdl_dtype dtype, int B, int L, int V, const void* logits, int64_t lsb,
                                    int64_t lsr, const int32_t* pos, const int32_t* n_rows, int m_max, int n_t,
                                    uint8_t* mask, float* conf, int32_t* tokens, int32_t* unmasked, void* ws,
                                    hipStream_t stream) {
    Part* parts = static_cast<Part*>(ws);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(B) * m_max));
    if (dtype == FDL_BF16)
        hipLaunchKernelGGL(conf_partial_kernel<uint16_t>, grid, dim3(kRowThreads), 0, stream,
                           static_cast<const uint16_t*>(logits), lsb, lsr, n_rows, m_max, V, parts);
    else
        hipLaunchKernelGGL(conf_partial_kernel<float>, grid, dim3(kRowThreads), 0, stream,
                           static_cast<const float*>(logits), lsb, lsr, n_rows, m_max, V, parts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(conf_select_kernel, dim3(B), dim3(kSelThreadsU), 0, stream, parts, pos, n_rows, m_max, L,
                       n_t, mask, conf, tokens, unmasked);
    return hipGetLastError();
}

}  // namespace fdl
