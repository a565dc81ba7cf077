// PCGI focus selection and window expansion.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Core
// method" and "Method steps" (1)-(2): the k = floor(rho * n(t)) still-masked
// positions with the highest previous-step confidence form I_focus; each is
// widened to the w positions [p - floor(w/2), p - floor(w/2) + w) clipped to
// [0, L), and their union is I_active.
//
// One 1024-thread workgroup per sequence.  A first pass reads the confidence
// and mask in per-thread runs of 16 positions (independent loads) and compacts
// the masked slots, in position order, into LDS as order-preserving keys.  The
// top-k is then selected among those candidates (a rank count when there are at
// most 2048 of them, a byte-wise radix select otherwise), which gives I_focus in
// ascending order with the lower index winning among equal confidences.  More
// than 8192 masked slots fall back to a radix select that reads the keys from
// global memory.  The windows of an ascending focus list have ascending ends, so
// each window adds the positions past the previous window's end; a scan over
// those counts places every active position.

#include "ops.cuh"

namespace fdl {

constexpr int kPcgiThreads = 1024;
constexpr int kPcgiRun = 16;        // positions per thread per pass
constexpr int kPcgiCap = 8192;      // masked slots kept in LDS

__global__ __launch_bounds__(kPcgiThreads) void pcgi_select_kernel(
    const float* __restrict__ conf, const uint8_t* __restrict__ mask, int L, int k, int w,
    int32_t* __restrict__ focus_idx, int32_t* __restrict__ n_focus, int k_cap,
    int32_t* __restrict__ active_idx, int32_t* __restrict__ n_active, int nq_max) {
    __shared__ SelectSmem sm;
    __shared__ int s_carry;
    __shared__ uint32_t s_key[kPcgiCap];
    __shared__ int32_t s_pos[kPcgiCap];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const float* c = conf + static_cast<int64_t>(b) * L;
    const uint8_t* m = mask + static_cast<int64_t>(b) * L;
    int32_t* focus = focus_idx + static_cast<int64_t>(b) * k_cap;
    int32_t* active = active_idx + static_cast<int64_t>(b) * nq_max;

    // compact the masked slots into LDS, in position order
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int base = 0; base < L; base += kPcgiThreads * kPcgiRun) {
        const int lo = base + tid * kPcgiRun;
        uint32_t keys[kPcgiRun];
        bool msk[kPcgiRun];
#pragma unroll
        for (int u = 0; u < kPcgiRun; ++u) {
            const int j = min(lo + u, L - 1);
            keys[u] = okey32(c[j]);
            msk[u] = m[j] != 0 && lo + u < L;
        }
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < kPcgiRun; ++u) cnt += msk[u] ? 1 : 0;
        int total;
        int off = block_exclusive_sum(cnt, sm.tmp, &total) + s_carry;
#pragma unroll
        for (int u = 0; u < kPcgiRun; ++u) {
            if (msk[u]) {
                if (off < kPcgiCap) {
                    s_key[off] = keys[u];
                    s_pos[off] = lo + u;
                }
                ++off;
            }
        }
        __syncthreads();
        if (tid == 0) s_carry += total;
        __syncthreads();
    }
    const int n_masked = s_carry;
    int nf;
    if (n_masked <= kPcgiCap) {
        nf = block_topk_lds<uint32_t>(n_masked, k, s_key, [&](int j) { return s_pos[j]; }, focus, k_cap, &sm);
    } else {
        auto key_of = [&](int j, uint32_t* key) -> bool {
            *key = okey32(c[j]);
            return m[j] != 0;
        };
        nf = block_emit_topk<uint32_t>(L, k, key_of, [](int j) { return j; }, focus, k_cap, &sm);
    }
    __syncthreads();  // focus[] written by other threads of the block is read below
    __threadfence_block();

    // Window union over the ascending focus list, processed in chunks of the block size.
    const int half = w / 2;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int f0 = 0; f0 < nf; f0 += blockDim.x) {
        const int f = f0 + tid;
        int start = 0, stop = 0, cnt = 0;
        if (f < nf) {
            const int p = focus[f];
            const int64_t s64 = static_cast<int64_t>(p) - half;
            start = static_cast<int>(s64 < 0 ? 0 : s64);
            const int64_t e64 = s64 + w;
            stop = static_cast<int>(e64 > L ? L : e64);
            int prev_stop = 0;
            if (f > 0) {
                const int64_t pe = static_cast<int64_t>(focus[f - 1]) - half + w;
                prev_stop = static_cast<int>(pe > L ? L : (pe < 0 ? 0 : pe));
            }
            start = max(start, prev_stop);
            cnt = max(0, stop - start);
        }
        int total;
        const int off = block_exclusive_sum(cnt, sm.tmp, &total) + s_carry;
        for (int i = 0; i < cnt; ++i) active[off + i] = start + i;
        __syncthreads();
        if (tid == 0) s_carry += total;
        __syncthreads();
    }
    const int na = s_carry;
    for (int i = na + tid; i < nq_max; i += blockDim.x) active[i] = -1;
    if (tid == 0) {
        n_focus[b] = nf;
        n_active[b] = na;
    }
}

hipError_t launch_pcgi_select(const float* conf, const uint8_t* mask, int B, int L, int k, int w,
                              int32_t* focus_idx, int32_t* n_focus, int k_cap,
                              int32_t* active_idx, int32_t* n_active, int nq_max,
                              hipStream_t stream) {
    hipLaunchKernelGGL(pcgi_select_kernel, dim3(B), dim3(kPcgiThreads), 0, stream, conf, mask, L, k,
                       w, focus_idx, n_focus, k_cap, active_idx, n_active, nq_max);
    return hipGetLastError();
}

}  // namespace fdl
