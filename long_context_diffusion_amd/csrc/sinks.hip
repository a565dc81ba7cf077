// Attention-sink identification at layer l_dense.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159),
// "Prerequisites" (attention sinks draw a disproportionate share of attention
// and keep their positions across layers) and "Method steps" (3) (layer
// l_dense's attention distribution identifies them).  The score of key j is the
// normalised attention probability it receives, summed over query heads and
// active query rows: sum_h sum_i exp(q_{h,i} . k_{g(h),j} * scale - lse_{h,i}),
// with lse from the dense attention of the same layer and rows.
//
// Three kernels:
//   sink_colsum   per (sequence, KV head, 256 keys): S = Q K^T on MFMA with keys
//                 on the N axis, so each lane owns one key column and sums the
//                 probabilities of all query rows (of every query head sharing
//                 the KV head) in a fixed order.  Q rows stream through LDS in
//                 blocks of 32.
//   sink_reduce   adds the per-KV-head partials in a fixed order (deterministic):
//                 four runs of consecutive heads, then the four run sums.
//   sink_select   top-n over the L scores of each sequence, ascending output: a
//                 threshold from the per-thread maxima, then an exact rank of the
//                 few scores above it (a radix select when there are many).

#include "ops.cuh"

namespace fdl {


namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kSinkKeysPerWg = 256;  // 4 waves x 64 keys
constexpr int kSinkRowsStaged = 1024;  // packed query rows resolved into LDS at once

template <int D>
__global__ __launch_bounds__(256, 2) void sink_colsum_bf16_kernel(const SinkArgs a) {
    constexpr int NQC = D / 16;
    constexpr int NCH = D / 8;
    constexpr int QP = D * 2 + 16;         // Q row pitch in LDS (bytes)
    constexpr int QPT = 32 * NCH / 256;    // 16-byte Q pieces staged per thread per block
    __shared__ __attribute__((aligned(16))) uint8_t s_q[2][32 * QP];
    // per packed row of the current chunk: element offset of its Q row, its lse (log2)
    __shared__ int64_t s_qoff[kSinkRowsStaged];
    __shared__ float s_lse2[kSinkRowsStaged + 32];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, hf = lane >> 5, col = lane & 31;
    const int kt = blockIdx.x % a.key_tiles;
    const int bg = blockIdx.x / a.key_tiles;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows = a.Gq * nq;
    const int key0 = kt * kSinkKeysPerWg + wv * 64;

    // K fragments (B operand): key = key0 + 32*kg + col, d = 16c + 8hf .. +7
    bf16x8 kf[2][NQC];
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + g * a.ksh;
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
        const int key = min(key0 + 32 * kg + col, a.L - 1);
#pragma unroll
        for (int c = 0; c < NQC; ++c)
            kf[kg][c] = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * a.ksr + 16 * c + 8 * hf));
    }

    // The packed rows are resolved once per chunk of kSinkRowsStaged rows (query head,
    // physical row through q_idx, lse), so a 32-row block costs each thread two table
    // reads instead of divisions by Gq and dependent loads.  Q block i of the chunk (rows
    // 32i .. 32i+31) is staged through registers into one of two LDS buffers while the
    // previous block is computed.
    const uint16_t* qb = static_cast<const uint16_t*>(a.q);
    const int pr = tid / NCH, pch = tid % NCH;   // piece x of a block: row pr + 256x/NCH, chunk pch
    float acc[2] = {0.0f, 0.0f};
    for (int c0 = 0; c0 < rows; c0 += kSinkRowsStaged) {
        const int cn = min(kSinkRowsStaged, rows - c0);
        const int nblk = (cn + 31) / 32;
        __syncthreads();   // the previous chunk's tables and blocks are no longer read
        for (int i = tid; i < 32 * nblk; i += 256) {
            const int p = c0 + min(i, cn - 1);
            const int h = g * a.Gq + p % a.Gq, r = p / a.Gq;
            const int phys = a.q_idx ? max(a.q_idx[static_cast<int64_t>(b) * a.nq_max + r], 0) : r;
            if (i < kSinkRowsStaged) s_qoff[i] = b * a.qsb + h * a.qsh + static_cast<int64_t>(phys) * a.qsr;
            s_lse2[i] = i < cn ? a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] * kLog2e : INFINITY;
        }
        __syncthreads();
        u32x4 qreg[QPT];
        auto load_block = [&](int i) __attribute__((always_inline)) {   // rows clamped to the chunk
#pragma unroll
            for (int x = 0; x < QPT; ++x) {
                const int row = min(32 * i + pr + x * (256 / NCH), cn - 1);
                qreg[x] = *reinterpret_cast<const u32x4*>(qb + s_qoff[row] + 8 * pch);
            }
        };
        auto store_block = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int x = 0; x < QPT; ++x)
                *reinterpret_cast<u32x4*>(&s_q[buf][(pr + x * (256 / NCH)) * QP + 16 * pch]) = qreg[x];
        };
        load_block(0);
        store_block(0);
        __syncthreads();
        for (int i = 0; i < nblk; ++i) {
            const int buf = i & 1;
            if (i + 1 < nblk) load_block(i + 1);
            float lrow[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) lrow[e] = s_lse2[32 * i + 8 * (e >> 2) + 4 * hf + (e & 3)];
            const uint8_t* qrow = &s_q[buf][col * QP + 16 * hf];
#pragma unroll
            for (int kg = 0; kg < 2; ++kg) {
                f32x16 sc;
#pragma unroll
                for (int e = 0; e < 16; ++e) sc[e] = 0.0f;
#pragma unroll
                for (int c = 0; c < NQC; ++c) {
                    const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qrow + 32 * c);
                    sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kg][c], sc, 0, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[kg] += fast_exp2(fmaf(sc[e], a.sl2, -lrow[e]));
            }
            if (i + 1 < nblk) store_block(buf ^ 1);
            __syncthreads();
        }
    }
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
        const float tot = acc[kg] + __shfl_xor(acc[kg], 32, 64);
        const int key = key0 + 32 * kg + col;
        if (hf == 0 && key < a.L) a.part[(static_cast<int64_t>(b) * a.Hkv + g) * a.L + key] = tot;
    }
}

template <int D>
__global__ __launch_bounds__(256) void sink_colsum_f32_kernel(const SinkArgs a) {
    __shared__ __attribute__((aligned(16))) float s_q[32][D];
    __shared__ float s_lse[32];
    const int tid = threadIdx.x;
    const int kt = blockIdx.x % a.key_tiles;
    const int bg = blockIdx.x / a.key_tiles;
    const int g = bg % a.Hkv, b = bg / a.Hkv;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows = a.Gq * nq;
    const int key = kt * kSinkKeysPerWg + tid;
    float kv[D];
    const float* krow = static_cast<const float*>(a.k) + b * a.ksb + g * a.ksh + static_cast<int64_t>(key) * a.ksr;
#pragma unroll
    for (int e = 0; e < D; ++e) kv[e] = key < a.L ? krow[e] : 0.0f;
    float acc = 0.0f;
    for (int r0 = 0; r0 < rows; r0 += 32) {
        __syncthreads();
        for (int i = tid; i < 32 * D; i += 256) {
            const int rr = i / D, e = i % D;
            const int p = r0 + rr;
            float x = 0.0f;
            if (p < rows) {
                const int h = g * a.Gq + p % a.Gq, r = p / a.Gq;
                const int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + r] : r;
                x = static_cast<const float*>(a.q)[b * a.qsb + h * a.qsh + static_cast<int64_t>(phys) * a.qsr + e];
            }
            s_q[rr][e] = x;
        }
        if (tid < 32) {
            const int p = r0 + tid;
            float l2 = INFINITY;
            if (p < rows) {
                const int h = g * a.Gq + p % a.Gq, r = p / a.Gq;
                l2 = a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] * kLog2e;
            }
            s_lse[tid] = l2;
        }
        __syncthreads();
        for (int rr = 0; rr < 32; ++rr) {
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < D; ++e) dot = fmaf(s_q[rr][e], kv[e], dot);
            acc += exp2f(fmaf(dot, a.sl2, -s_lse[rr]));
        }
    }
    if (key < a.L) a.part[(static_cast<int64_t>(b) * a.Hkv + g) * a.L + key] = acc;
}

// score[b][j] = sum over KV heads of part[b][g][j]: a workgroup takes kRedKeys keys, its
// kRedGroups thread groups each add a contiguous run of heads for every key, and the
// group sums are added in group order (a fixed order: repeated runs are bit-identical).
constexpr int kRedKeys = 64;
constexpr int kRedGroups = 4;
__global__ __launch_bounds__(kRedKeys * kRedGroups) void sink_reduce_kernel(const SinkArgs a) {
    __shared__ float s_g[kRedGroups][kRedKeys];
    const int kt = threadIdx.x % kRedKeys, grp = threadIdx.x / kRedKeys;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kRedKeys + kt;   // b * L + j
    const bool ok = i < static_cast<int64_t>(a.B) * a.L;
    const int b = ok ? static_cast<int>(i / a.L) : 0;
    const int j = ok ? static_cast<int>(i % a.L) : 0;
    const int per = (a.Hkv + kRedGroups - 1) / kRedGroups;
    const int g0 = grp * per, g1 = min(a.Hkv, g0 + per);
    const float* p = a.part + static_cast<int64_t>(b) * a.Hkv * a.L + j;
    float s = 0.0f;
    if (ok) {
        int g = g0;
        for (; g + 8 <= g1; g += 8) {
            float x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) x[u] = p[static_cast<int64_t>(g + u) * a.L];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += x[u];
        }
        for (; g < g1; ++g) s += p[static_cast<int64_t>(g) * a.L];
    }
    s_g[grp][kt] = s;
    __syncthreads();
    if (grp == 0 && ok) {
        float t = s_g[0][kt];
#pragma unroll
        for (int q = 1; q < kRedGroups; ++q) t += s_g[q][kt];
        a.scores[i] = t;
    }
}

constexpr int kSelThreads = 1024;
constexpr int kSelPerThread = 32;    // scores per thread held in registers (L <= 32768)
constexpr int kSelCand = 1024;       // candidates ranked exactly in LDS

// Unique ordered key of score x at position j: the ordered score in the high word and
// the complement of j in the low word, so the larger score wins and, among equal
// scores, the lower position.  Valid keys are never 0.
__device__ __forceinline__ uint64_t sink_key(float x, int j) {
    return (static_cast<uint64_t>(okey32(x)) << 32) | static_cast<uint32_t>(~j);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
    const uint32_t lo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), mask, kWave));
    const uint32_t hi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(v >> 32), mask, kWave));
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Top-n_sinks positions of each sequence's scores, ascending.  Every thread holds a
// contiguous run of at most 32 scores in registers.  The n-th largest of the 1024
// per-thread maxima, T, is at most the n-th largest score (the n largest maxima are n
// distinct scores), so every selected score is >= T, and at most n threads hold one.
// The scores >= T (at most 32 n of them, in position order) are ranked exactly in
// LDS.  More than 32768 scores, or more than 1024 candidates, take the radix select.
__global__ __launch_bounds__(kSelThreads) void sink_select_kernel(const float* __restrict__ scores, int L,
                                                                 int n_sinks, int32_t* __restrict__ sink_idx) {
    __shared__ SelectSmem sm;
    __shared__ uint64_t s_lm[kSelThreads];
    __shared__ uint64_t s_cand[kSelCand];
    __shared__ uint64_t s_T;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const float* s = scores + static_cast<int64_t>(b) * L;
    int32_t* out = sink_idx + static_cast<int64_t>(b) * n_sinks;
    auto radix = [&]() {
        auto key_of = [&](int j, uint32_t* key) -> bool {
            *key = okey32(s[j]);
            return true;
        };
        block_emit_topk<uint32_t>(L, n_sinks, key_of, [](int j) { return j; }, out, n_sinks, &sm);
    };
    if (n_sinks <= 0) return;
    if (L > kSelThreads * kSelPerThread) {
        radix();
        return;
    }
    const int chunk = (L + kSelThreads - 1) / kSelThreads;
    const int lo = min(L, tid * chunk);
    const int cnt = min(L, lo + chunk) - lo;
    uint64_t key[kSelPerThread];
    if (chunk == kSelPerThread && cnt == kSelPerThread && (reinterpret_cast<uintptr_t>(s) & 15) == 0) {
        f32x4 v[kSelPerThread / 4];
#pragma unroll
        for (int q = 0; q < kSelPerThread / 4; ++q) v[q] = *reinterpret_cast<const f32x4*>(s + lo + 4 * q);
#pragma unroll
        for (int u = 0; u < kSelPerThread; ++u) key[u] = sink_key(v[u / 4][u % 4], lo + u);
    } else {
        float x[kSelPerThread];
#pragma unroll
        for (int u = 0; u < kSelPerThread; ++u) x[u] = s[u < cnt ? lo + u : 0];
#pragma unroll
        for (int u = 0; u < kSelPerThread; ++u) key[u] = u < cnt ? sink_key(x[u], lo + u) : 0;
    }
    uint64_t m = 0;
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u) m = key[u] > m ? key[u] : m;
    // bitonic sort of the wave's 64 maxima, descending across the lanes
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const uint64_t p = shfl_xor_u64(m, stride);
            const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
            const bool take_max = desc == lower;
            m = take_max ? (p > m ? p : m) : (p < m ? p : m);
        }
    s_lm[tid] = m;
    if (tid == 0) s_T = 0;
    __syncthreads();
    if (m != 0) {
        // rank among all maxima = entries greater than m, by binary search in each sorted wave
        int rank = 0;
#pragma unroll
        for (int w = 0; w < kSelThreads / kWave; ++w) {
            int a0 = 0, a1 = kWave;
#pragma unroll
            for (int it = 0; it < 6; ++it) {
                const int mid = (a0 + a1) >> 1;
                if (s_lm[w * kWave + mid] > m) a0 = mid + 1;
                else a1 = mid;
            }
            rank += a0;
        }
        if (rank == n_sinks - 1) s_T = m;
    }
    __syncthreads();
    // fewer than n_sinks threads with scores leave T = 0: every score is a candidate
    const uint64_t T = s_T;
    int c = 0;
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u) c += (key[u] != 0 && key[u] >= T) ? 1 : 0;
    int total;
    int off = block_exclusive_sum(c, sm.tmp, &total);
    if (total > kSelCand) {
        radix();
        return;
    }
#pragma unroll
    for (int u = 0; u < kSelPerThread; ++u)
        if (key[u] != 0 && key[u] >= T) s_cand[off++] = key[u];
    __syncthreads();
    int sel = 0;
    uint64_t mine = 0;
    if (tid < total) {
        mine = s_cand[tid];
        int r = 0;
        int i = 0;
        for (; i + 8 <= total; i += 8) {
            uint64_t y[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) y[u] = s_cand[i + u];
#pragma unroll
            for (int u = 0; u < 8; ++u) r += y[u] > mine ? 1 : 0;
        }
        for (; i < total; ++i) r += s_cand[i] > mine ? 1 : 0;
        sel = r < n_sinks ? 1 : 0;
    }
    int nsel;
    const int pos = block_exclusive_sum(sel, sm.tmp, &nsel);
    if (sel) out[pos] = static_cast<int32_t>(~static_cast<uint32_t>(mine));
    for (int i = nsel + tid; i < n_sinks; i += blockDim.x) out[i] = -1;
}

}  // namespace

size_t sink_workspace_bytes(int B, int Hkv, int L) {
    return (static_cast<size_t>(B) * Hkv * L + static_cast<size_t>(B) * L) * sizeof(float);
}

hipError_t launch_sink_identify(fdl_dtype dtype, int d, SinkArgs a, int n_sinks, int32_t* sink_idx,
                                float* user_scores, void* ws, hipStream_t stream) {
    a.part = static_cast<float*>(ws);
    a.scores = user_scores ? user_scores : a.part + static_cast<int64_t>(a.B) * a.Hkv * a.L;
    a.key_tiles = (a.L + kSinkKeysPerWg - 1) / kSinkKeysPerWg;
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * a.key_tiles));
    if (dtype == FDL_BF16) {
        if (d == 128) hipLaunchKernelGGL(sink_colsum_bf16_kernel<128>, grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL(sink_colsum_bf16_kernel<64>, grid, dim3(256), 0, stream, a);
    } else {
        if (d == 128) hipLaunchKernelGGL(sink_colsum_f32_kernel<128>, grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL(sink_colsum_f32_kernel<64>, grid, dim3(256), 0, stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t n = static_cast<int64_t>(a.B) * a.L;
    hipLaunchKernelGGL(sink_reduce_kernel, dim3(static_cast<unsigned>((n + kRedKeys - 1) / kRedKeys)),
                       dim3(kRedKeys * kRedGroups), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(sink_select_kernel, dim3(a.B), dim3(kSelThreads), 0, stream, a.scores, a.L, n_sinks, sink_idx);
    return hipGetLastError();
}

}  // namespace fdl
