// PCGI focus selection and window expansion.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Core
// method" and "Method steps" (1)-(2): the k = floor(rho * n(t)) still-masked
// positions with the highest previous-step confidence form I_focus; each is
// widened to the w positions [p - floor(w/2), p - floor(w/2) + w) clipped to
// [0, L), and their union is I_active.
//
// One 1024-thread workgroup per sequence.  A first pass compacts the masked slots,
// in position order, into LDS as order-preserving keys.  Its loads are coalesced: in
// round q every thread reads 4 consecutive positions (one 16-byte confidence load and
// one 4-byte mask load), so a wave covers 256 contiguous positions.  A slot's place
// is the count of masked slots before it: ballots give the count within the wave,
// and one scan over the per-(round, wave) totals gives the rest, with two barriers
// per 32768 positions.  The top-k is then selected among those candidates (a rank
// count when there are at most 1024 of them, a byte-wise radix select otherwise),
// which gives I_focus in ascending order with the lower index winning among equal
// confidences.  More than 8192 masked slots fall back to a radix select that reads
// the keys from global memory.  The windows of an ascending focus list have
// ascending ends, so each window adds the positions past the previous window's
// end; a scan over those counts places every active position.

#include "ops.cuh"

namespace fdl {

constexpr int kPcgiThreads = 1024;
constexpr int kPcgiWaves = kPcgiThreads / kWave;
constexpr int kPcgiQuad = 4;                           // positions per thread per round
constexpr int kPcgiRounds = 8;                         // rounds per pass
constexpr int kPcgiSpan = kPcgiThreads * kPcgiQuad;    // positions per round
constexpr int kPcgiCap = 8192;                         // masked slots kept in LDS

__global__ __launch_bounds__(kPcgiThreads) void pcgi_select_kernel(
    const float* __restrict__ conf, const uint8_t* __restrict__ mask, int L, int k, int w,
    int32_t* __restrict__ focus_idx, int32_t* __restrict__ n_focus, int k_cap,
    int32_t* __restrict__ active_idx, int32_t* __restrict__ n_active, int nq_max) {
    __shared__ SelectSmem sm;
    __shared__ int s_carry;
    __shared__ int s_wcnt[kPcgiRounds * kPcgiWaves];   // masked slots per (round, wave), then their prefix
    __shared__ int s_total;
    __shared__ uint32_t s_key[kPcgiCap];
    __shared__ int32_t s_pos[kPcgiCap];
    __shared__ int32_t s_focus[kPcgiCap];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = tid / kWave;
    const float* c = conf + static_cast<int64_t>(b) * L;
    const uint8_t* m = mask + static_cast<int64_t>(b) * L;
    int32_t* focus = focus_idx + static_cast<int64_t>(b) * k_cap;
    int32_t* active = active_idx + static_cast<int64_t>(b) * nq_max;

    // ---- compact the masked slots into LDS, in position order
    const bool vec = (reinterpret_cast<uintptr_t>(c) & 15) == 0 && (reinterpret_cast<uintptr_t>(m) & 3) == 0;
    const uint64_t below = (1ull << lane) - 1ull;   // lanes before this one
    int carry = 0;                                  // masked slots of earlier passes
    for (int pass0 = 0; pass0 < L; pass0 += kPcgiRounds * kPcgiSpan) {
        uint32_t key[kPcgiRounds][kPcgiQuad];
        uint32_t bits = 0;   // bit kPcgiQuad*q + i: position pass0 + q*kPcgiSpan + 4*tid + i is masked
#pragma unroll
        for (int q = 0; q < kPcgiRounds; ++q) {
            const int p0 = pass0 + q * kPcgiSpan + kPcgiQuad * tid;
            if (vec && p0 + kPcgiQuad <= L) {
                const f32x4 cv = *reinterpret_cast<const f32x4*>(c + p0);
                const uint32_t mw = *reinterpret_cast<const uint32_t*>(m + p0);
#pragma unroll
                for (int i = 0; i < kPcgiQuad; ++i) {
                    key[q][i] = okey32(cv[i]);
                    bits |= (((mw >> (8 * i)) & 0xffu) != 0 ? 1u : 0u) << (kPcgiQuad * q + i);
                }
            } else {
#pragma unroll
                for (int i = 0; i < kPcgiQuad; ++i) {
                    const int p = p0 + i;
                    const bool in = p < L;
                    key[q][i] = okey32(c[in ? p : 0]);
                    bits |= ((in && m[in ? p : 0] != 0) ? 1u : 0u) << (kPcgiQuad * q + i);
                }
            }
        }
        // place within the wave: masked slots of earlier lanes (ballots) and earlier i
        int lane_before[kPcgiRounds];
#pragma unroll
        for (int q = 0; q < kPcgiRounds; ++q) {
            int before = 0, total = 0;
#pragma unroll
            for (int i = 0; i < kPcgiQuad; ++i) {
                const uint64_t bal = __ballot((bits >> (kPcgiQuad * q + i)) & 1u);
                before += __popcll(bal & below);
                total += __popcll(bal);
            }
            lane_before[q] = before;
            if (lane == 0) s_wcnt[q * kPcgiWaves + wv] = total;
        }
        __syncthreads();
        // exclusive scan of the (round, wave) totals, which are in position order
        if (wv == 0) {
            static_assert(kPcgiRounds * kPcgiWaves == 2 * kWave, "two totals per lane");
            const int v0 = s_wcnt[2 * lane], v1 = s_wcnt[2 * lane + 1];
            const int inc = wave_inclusive_sum(v0 + v1);
            s_wcnt[2 * lane] = inc - v0 - v1;
            s_wcnt[2 * lane + 1] = inc - v1;
            if (lane == kWave - 1) s_total = inc;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < kPcgiRounds; ++q) {
            int off = carry + s_wcnt[q * kPcgiWaves + wv] + lane_before[q];
            const int p0 = pass0 + q * kPcgiSpan + kPcgiQuad * tid;
#pragma unroll
            for (int i = 0; i < kPcgiQuad; ++i) {
                if ((bits >> (kPcgiQuad * q + i)) & 1u) {
                    if (off < kPcgiCap) {
                        s_key[off] = key[q][i];
                        s_pos[off] = p0 + i;
                    }
                    ++off;
                }
            }
        }
        carry += s_total;
        __syncthreads();   // s_wcnt and s_total are rewritten by the next pass; s_key is read below
    }
    const int n_masked = carry;
    int nf;
    const int32_t* fl;   // the focus list the windows are built from
    if (n_masked <= kPcgiCap) {
        // selected into LDS (the windows read it there), then copied out
        const int n_sel = min(max(k, 0), n_masked);
        nf = block_topk_lds(n_masked, k, s_key, [&](int j) { return s_pos[j]; }, s_focus, n_sel, &sm);
        __syncthreads();
        for (int i = tid; i < k_cap; i += blockDim.x) focus[i] = i < nf ? s_focus[i] : -1;
        fl = s_focus;
    } else {
        auto key_of = [&](int j, uint32_t* key) -> bool {
            *key = okey32(c[j]);
            return m[j] != 0;
        };
        nf = block_emit_topk<uint32_t>(L, k, key_of, [](int j) { return j; }, focus, k_cap, &sm);
        __syncthreads();  // focus[] written by other threads of the block is read below
        __threadfence_block();
        fl = focus;
    }

    // Window union over the ascending focus list, processed in chunks of the block size.
    const int half = w / 2;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int f0 = 0; f0 < nf; f0 += blockDim.x) {
        const int f = f0 + tid;
        int start = 0, stop = 0, cnt = 0;
        if (f < nf) {
            const int p = fl[f];
            const int64_t s64 = static_cast<int64_t>(p) - half;
            start = static_cast<int>(s64 < 0 ? 0 : s64);
            const int64_t e64 = s64 + w;
            stop = static_cast<int>(e64 > L ? L : e64);
            int prev_stop = 0;
            if (f > 0) {
                const int64_t pe = static_cast<int64_t>(fl[f - 1]) - half + w;
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
