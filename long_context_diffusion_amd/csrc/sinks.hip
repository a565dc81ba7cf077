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
//   sink_reduce   adds the per-KV-head partials in head order (deterministic).
//   sink_select   radix top-n over the L scores of each sequence, ascending output.

#include "ops.cuh"

namespace fdl {


namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kSinkKeysPerWg = 256;  // 4 waves x 64 keys

template <int D>
__global__ __launch_bounds__(256) void sink_colsum_bf16_kernel(const SinkArgs a) {
    constexpr int NQC = D / 16;
    constexpr int NCH = D / 8;
    constexpr int QP = D * 2 + 16;     // Q row pitch in LDS (bytes)
    __shared__ __attribute__((aligned(16))) uint8_t s_q[32 * QP];
    __shared__ float s_lse[32];

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
        const int key = key0 + 32 * kg + col;
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (key < a.L) x = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * a.ksr + 16 * c + 8 * hf);
            kf[kg][c] = __builtin_bit_cast(bf16x8, x);
        }
    }
    float acc[2] = {0.0f, 0.0f};

    for (int r0 = 0; r0 < rows; r0 += 32) {
        __syncthreads();
        // stage 32 packed query rows (zero beyond `rows`) and their lse in log2 units
        for (int i = tid; i < 32 * NCH; i += 256) {
            const int rr = i / NCH, ch = i % NCH;
            const int p = r0 + rr;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (p < rows) {
                const int h = g * a.Gq + p % a.Gq, r = p / a.Gq;
                const int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + r] : r;
                x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + b * a.qsb + h * a.qsh +
                                                   static_cast<int64_t>(phys) * a.qsr + 8 * ch);
            }
            *reinterpret_cast<u32x4*>(s_q + rr * QP + 16 * ch) = x;
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
        float lrow[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) lrow[i] = s_lse[8 * (i >> 2) + 4 * hf + (i & 3)];
        const uint8_t* qrow = s_q + col * QP + 16 * hf;
#pragma unroll
        for (int kg = 0; kg < 2; ++kg) {
            f32x16 s;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[i] = 0.0f;
#pragma unroll
            for (int c = 0; c < NQC; ++c) {
                const bf16x8 aq = *reinterpret_cast<const bf16x8*>(qrow + 32 * c);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[kg][c], s, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[kg] += exp2f(fmaf(s[i], a.sl2, -lrow[i]));
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

__global__ __launch_bounds__(256) void sink_reduce_kernel(const SinkArgs a) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<int64_t>(a.B) * a.L) return;
    const int b = static_cast<int>(i / a.L);
    const int j = static_cast<int>(i % a.L);
    const float* p = a.part + static_cast<int64_t>(b) * a.Hkv * a.L + j;
    float s = 0.0f;
    for (int g = 0; g < a.Hkv; ++g) s += p[static_cast<int64_t>(g) * a.L];
    a.scores[i] = s;
}

__global__ __launch_bounds__(1024) void sink_select_kernel(const float* __restrict__ scores, int L,
                                                           int n_sinks, int32_t* __restrict__ sink_idx) {
    __shared__ SelectSmem sm;
    const int b = blockIdx.x;
    const float* s = scores + static_cast<int64_t>(b) * L;
    auto key_of = [&](int j, uint32_t* key) -> bool {
        *key = okey32(s[j]);
        return true;
    };
    block_emit_topk<uint32_t>(L, n_sinks, key_of, sink_idx + static_cast<int64_t>(b) * n_sinks, n_sinks, &sm);
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
    hipLaunchKernelGGL(sink_reduce_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(sink_select_kernel, dim3(a.B), dim3(1024), 0, stream, a.scores, a.L, n_sinks, sink_idx);
    return hipGetLastError();
}

}  // namespace fdl
