// Dynamic cache update (DCU) scoring: which tokens' caches each layer refreshes.
//
// Dynamic-dLLM article, section "DCU：动态缓存更新".  The change of a token's normalised
// layer input between adjacent denoising steps is measured by the cosine distance, the
// per-token changes of a layer add up to its activity, a total update budget is split over
// the layers in proportion to activity, and each layer refreshes a mandatory window around
// the key tokens plus its budget of the most changed other tokens.
//
// Three kernels:
//   dcu_distance  one wave per token (kTokPerWave tokens in turn): the four sums
//                 |x|^2, |y|^2, |x - y|^2 and (x - y).(x + y) in one read of both inputs,
//                 then d = 1 - cos(x, y); each workgroup also leaves the fp64 sum of its
//                 kTokPerWg distances (the work is bound by HBM bandwidth).
//   dcu_activity  one workgroup per (sequence, layer): the layer's activity, the sum of
//                 its workgroup partials in a fixed order.
//   dcu_select    one workgroup per (sequence, layer): the layer's budget (every workgroup
//                 of a sequence repeats the same arithmetic on the same activities), the
//                 mandatory windows as a bitmask in LDS, a radix select of the budget over
//                 the other tokens, and the ascending update list.
//
// The distance is computed as d = (|x - y|^2 - (|x| - |y|)^2) / (2 |x| |y|) with
// |x| - |y| = (x - y).(x + y) / (|x| + |y|): the sums are of the elementwise differences
// (exact for bf16 inputs, rounded once for fp32 ones) rather than of the inputs, so d stays
// accurate relative to |x - y|^2 / (2 |x| |y|) when the two inputs are close, where
// 1 - x.y / (|x| |y|) would lose all its digits to cancellation.

#include "ops.cuh"

namespace fdl {

namespace {

constexpr int kDistThreads = 256;
constexpr int kDistWaves = kDistThreads / kWave;
constexpr int kTokPerWave = 8;
constexpr int kTokPerWg = kDistWaves * kTokPerWave;   // tokens per distance workgroup
constexpr int kLoadsPerLane = 8;   // 16-byte loads of each input per lane and iteration
constexpr int kSelThreads = 1024;

struct Sums {
    float xx, yy, dd, dq;
};

__device__ __forceinline__ void add_pair(float x, float y, Sums& s) {
    const float df = x - y, sm = x + y;
    s.xx = fmaf(x, x, s.xx);
    s.yy = fmaf(y, y, s.yy);
    s.dd = fmaf(df, df, s.dd);
    s.dq = fmaf(df, sm, s.dq);
}

template <typename T>
__device__ __forceinline__ void add_vec(const u32x4& a, const u32x4& c, Sums& s) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            add_pair(bf16lo(a[i]), bf16lo(c[i]), s);
            add_pair(bf16hi(a[i]), bf16hi(c[i]), s);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) add_pair(__uint_as_float(a[i]), __uint_as_float(c[i]), s);
    }
}

// d of one token, computed by a whole wave (the result in every lane).
template <typename T>
__device__ __forceinline__ float token_distance(const T* x, const T* y, int H, int lane) {
    constexpr int EPV = 16 / sizeof(T);
    const int nvec = H / EPV;
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    const u32x4* yv = reinterpret_cast<const u32x4*>(y);
    Sums s{0.0f, 0.0f, 0.0f, 0.0f};
    for (int v0 = 0; v0 < nvec; v0 += kWave * kLoadsPerLane) {
        u32x4 a[kLoadsPerLane], c[kLoadsPerLane];
#pragma unroll
        for (int u = 0; u < kLoadsPerLane; ++u) {
            const int v = v0 + lane + kWave * u;
            if (v < nvec) {
                a[u] = __builtin_nontemporal_load(xv + v);
                c[u] = __builtin_nontemporal_load(yv + v);
            } else {
                a[u] = u32x4{0u, 0u, 0u, 0u};
                c[u] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kLoadsPerLane; ++u) add_vec<T>(a[u], c[u], s);
    }
    for (int e = nvec * EPV + lane; e < H; e += kWave) add_pair(Elem<T>::load(x + e), Elem<T>::load(y + e), s);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        s.xx += __shfl_xor(s.xx, off, kWave);
        s.yy += __shfl_xor(s.yy, off, kWave);
        s.dd += __shfl_xor(s.dd, off, kWave);
        s.dq += __shfl_xor(s.dq, off, kWave);
    }
    const float nx = sqrtf(s.xx), ny = sqrtf(s.yy);
    if (!(nx > 0.0f && ny > 0.0f)) return 0.0f;
    const float dn = s.dq / (nx + ny);                  // |x| - |y|
    const float d = (s.dd - dn * dn) / (2.0f * nx * ny);
    return d > 0.0f ? d : 0.0f;                         // +0 for rounding below zero (and NaN)
}

template <typename T>
__global__ __launch_bounds__(kDistThreads) void dcu_distance_kernel(const T* xn, int64_t xnb, int64_t xnl,
                                                                    int64_t xnr, const T* xp, int64_t xpb,
                                                                    int64_t xpl, int64_t xpr, int NL, int L, int H,
                                                                    int n_chunks, float* dist, double* part) {
    __shared__ float s_d[kTokPerWg];
    const int ch = blockIdx.x % n_chunks;
    const int bl = blockIdx.x / n_chunks;   // b * NL + l
    const int b = bl / NL, l = bl % NL;
    const int wv = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int i0 = ch * kTokPerWg;
    for (int t = 0; t < kTokPerWave; ++t) {
        const int il = t * kDistWaves + wv;
        const int i = i0 + il;
        float d = 0.0f;
        if (i < L) {
            const T* x = xn + b * xnb + l * xnl + i * xnr;
            const T* y = xp + b * xpb + l * xpl + i * xpr;
            d = token_distance<T>(x, y, H, lane);
        }
        if (lane == 0) s_d[il] = d;
    }
    __syncthreads();
    const int nt = min(kTokPerWg, L - i0);
    if (static_cast<int>(threadIdx.x) < nt) dist[static_cast<int64_t>(bl) * L + i0 + threadIdx.x] = s_d[threadIdx.x];
    if (threadIdx.x == 0) {
        double acc = 0.0;
        for (int j = 0; j < nt; ++j) acc += static_cast<double>(s_d[j]);
        part[static_cast<int64_t>(bl) * n_chunks + ch] = acc;
    }
}

__global__ __launch_bounds__(kDistThreads) void dcu_activity_kernel(const double* part, int n_chunks,
                                                                    double* activity) {
    __shared__ double s_w[kDistWaves];
    const int bl = blockIdx.x;
    const double* p = part + static_cast<int64_t>(bl) * n_chunks;
    double acc = 0.0;
    for (int c = threadIdx.x; c < n_chunks; c += kDistThreads) acc += p[c];
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) acc += __shfl_xor(acc, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double a = 0.0;
        for (int w = 0; w < kDistWaves; ++w) a += s_w[w];
        activity[bl] = a;
    }
}

// Sum of a double over the block in a fixed order; every thread gets the total.
__device__ __forceinline__ double block_sum_f64(double x, double* s_tmp) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) x += __shfl_xor(x, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = x;
    __syncthreads();
    double tot = 0.0;
    for (int w = 0; w < static_cast<int>(blockDim.x) / kWave; ++w) tot += s_tmp[w];
    __syncthreads();
    return tot;
}

__device__ __forceinline__ bool bit_set(const uint32_t* bits, int j) { return (bits[j >> 5] >> (j & 31)) & 1u; }

constexpr int kRegKeys = 32;   // positions per thread held in registers (L up to 32768)

// Takes the mandatory positions of [lo, hi) and the `budget` other positions of largest key
// (the lower position first among equal keys; all of them when there are fewer), and
// writes them ascending to out; *count gets their number.  `key(e)` and `mand(e)` describe
// position lo + e; every thread of the block calls it.  The radix select runs over
// `for_each(body)`, which calls body(key, valid) for every position of the thread.
template <typename ForEach, typename Emit>
__device__ inline void budget_select(ForEach for_each, Emit emit, int n_mand_local, int span, int L, int budget,
                                     int32_t* out, int32_t* count, SelectSmem* sm) {
    int n_mand;
    block_exclusive_sum(n_mand_local, sm->tmp, &n_mand);
    const int n_other = L - n_mand;
    const bool take_all = budget >= n_other;
    const int nsel = take_all ? n_other : max(budget, 0);
    uint32_t thr = 0;
    const int wv = threadIdx.x / kWave;
    if (!take_all && nsel > 0) {
        // radix select of the nsel-th largest key among the valid positions, 8 bits a pass
        uint32_t prefix = 0, prefix_mask = 0;
        int remaining = nsel;
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = threadIdx.x; i < kMaxWaves * 256; i += blockDim.x) sm->hist[i / 256][i % 256] = 0;
            __syncthreads();
            for_each([&](uint32_t kj, bool ok) {
                wave_count(sm->hist[wv], static_cast<int>((kj >> shift) & 0xff), ok && (kj & prefix_mask) == prefix);
            });
            __syncthreads();
            const int dgt = radix_pick_digit(sm, &remaining);
            prefix |= static_cast<uint32_t>(dgt) << shift;
            prefix_mask |= 0xffu << shift;
        }
        thr = prefix;
    }
    int gt = 0, eq = 0;
    if (nsel > 0 && !take_all) {
        for_each([&](uint32_t kj, bool ok) {
            gt += ok && kj > thr ? 1 : 0;
            eq += ok && kj == thr ? 1 : 0;
        });
    }
    int gt_total, eq_total;
    block_exclusive_sum(gt, sm->tmp, &gt_total);
    const int eq_before = block_exclusive_sum(eq, sm->tmp, &eq_total);
    const int ties_taken = nsel - gt_total;   // ties go to the lower positions
    const int my_ties = take_all || nsel == 0 ? 0 : min(max(ties_taken - eq_before, 0), eq);
    const int my_other = take_all ? (span - n_mand_local) : (nsel == 0 ? 0 : gt + my_ties);
    int n_total;
    const int pos = block_exclusive_sum(n_mand_local + my_other, sm->tmp, &n_total);
    emit(pos, take_all, nsel, thr, eq_before, ties_taken, out);
    if (threadIdx.x == 0) *count = n_total;
}

// Positions with their keys and mandatory bits in registers (at most kRegKeys per thread).
__device__ inline void select_from_registers(const float* dl, const uint32_t* s_mand, int lo, int hi, int L,
                                             int budget, int32_t* out, int32_t* count, SelectSmem* sm) {
    uint32_t key[kRegKeys];
    uint32_t mand = 0, live = 0;   // bit e: position lo + e is mandatory / exists
    const int span = hi - lo;
    if (span == kRegKeys && (lo & 31) == 0 && (reinterpret_cast<uintptr_t>(dl + lo) & 15) == 0) {
        // a whole 32-bit word of the bitmask, 16-byte loads
        const f32x4* src = reinterpret_cast<const f32x4*>(dl + lo);
#pragma unroll
        for (int v = 0; v < kRegKeys / 4; ++v) {
            const f32x4 x = src[v];
#pragma unroll
            for (int i = 0; i < 4; ++i) key[4 * v + i] = __float_as_uint(x[i]);
        }
        mand = s_mand[lo >> 5];
        live = 0xffffffffu;
    } else {
#pragma unroll
        for (int e = 0; e < kRegKeys; ++e) {
            const bool in = e < span;
            key[e] = in ? __float_as_uint(dl[lo + e]) : 0u;
            mand |= (in && bit_set(s_mand, lo + e)) ? (1u << e) : 0u;
            live |= in ? (1u << e) : 0u;
        }
    }
    const uint32_t other = live & ~mand;
    auto for_each = [&](auto body) {
#pragma unroll
        for (int e = 0; e < kRegKeys; ++e) body(key[e], ((other >> e) & 1u) != 0);
    };
    auto emit = [&](int pos, bool take_all, int nsel, uint32_t thr, int tie_seen, int ties_taken, int32_t* dst) {
#pragma unroll
        for (int e = 0; e < kRegKeys; ++e) {
            bool take = (mand >> e) & 1u;
            if (!take && ((other >> e) & 1u) && nsel > 0) {
                if (take_all || key[e] > thr) {
                    take = true;
                } else if (key[e] == thr) {
                    take = tie_seen < ties_taken;
                    ++tie_seen;
                }
            }
            if (take) dst[pos++] = lo + e;
        }
    };
    budget_select(for_each, emit, __popc(mand), span, L, budget, out, count, sm);
}

// Positions read from the distances in memory (L2) on every pass.
__device__ inline void select_from_memory(const float* dl, const uint32_t* s_mand, int lo, int hi, int L,
                                          int budget, int32_t* out, int32_t* count, SelectSmem* sm) {
    int n_mand_local = 0;
    for (int j = lo; j < hi; ++j) n_mand_local += bit_set(s_mand, j) ? 1 : 0;
    auto for_each = [&](auto body) {
        for (int j = lo; j < hi; ++j) body(__float_as_uint(dl[j]), !bit_set(s_mand, j));
    };
    auto emit = [&](int pos, bool take_all, int nsel, uint32_t thr, int tie_seen, int ties_taken, int32_t* dst) {
        for (int j = lo; j < hi; ++j) {
            bool take = bit_set(s_mand, j);
            if (!take && nsel > 0) {
                const uint32_t kj = __float_as_uint(dl[j]);
                if (take_all || kj > thr) {
                    take = true;
                } else if (kj == thr) {
                    take = tie_seen < ties_taken;
                    ++tie_seen;
                }
            }
            if (take) dst[pos++] = j;
        }
    };
    budget_select(for_each, emit, n_mand_local, hi - lo, L, budget, out, count, sm);
}

__global__ __launch_bounds__(kSelThreads) void dcu_select_kernel(const float* dist, const double* activity, int NL,
                                                                 int L, const int32_t* keys, int n_keys, int w_m,
                                                                 int total, int32_t* budgets, int32_t* upd_idx,
                                                                 int32_t* n_upd) {
    __shared__ SelectSmem sm;
    __shared__ uint32_t s_mand[kDcuMaxTokens / 32];
    __shared__ double s_frac[kDcuMaxLayers];
    __shared__ double s_tmp[kSelThreads / kWave];
    __shared__ int s_budget;
    const int bl = blockIdx.x;
    const int b = bl / NL, l = bl % NL;
    const int tid = threadIdx.x;

    // -- the budget of layer l: floor of its proportional share, plus one for the R layers of
    //    largest fractional part (the lower layer first among equal parts)
    const double a_m = tid < NL ? activity[static_cast<int64_t>(b) * NL + tid] : 0.0;
    const double A = block_sum_f64(a_m, s_tmp);
    double q = 0.0, base = 0.0;
    if (tid < NL) {
        q = A > 0.0 ? static_cast<double>(total) * a_m / A : static_cast<double>(total) / NL;
        base = floor(q);
        s_frac[tid] = q - base;
    }
    int tmp_total;
    block_exclusive_sum(tid < NL ? static_cast<int>(base) : 0, sm.tmp, &tmp_total);   // also orders s_frac
    const int R = total - tmp_total;
    const double fl = s_frac[l];
    const bool ahead = tid < NL && (s_frac[tid] > fl || (s_frac[tid] == fl && tid < l));
    int rank;
    block_exclusive_sum(ahead ? 1 : 0, sm.tmp, &rank);
    if (tid == l) {
        const int bud = static_cast<int>(base) + (rank < R ? 1 : 0);
        s_budget = bud;
        budgets[bl] = bud;
    }

    // -- mandatory windows [c - floor(w_m/2), c - floor(w_m/2) + w_m) around the key tokens
    const int nwords = (L + 31) / 32;
    for (int i = tid; i < nwords; i += kSelThreads) s_mand[i] = 0u;
    __syncthreads();
    const int half = w_m / 2;
    for (int kk = tid; kk < n_keys; kk += kSelThreads) {
        const int c = keys[static_cast<int64_t>(b) * n_keys + kk];
        if (c < 0 || c >= L) continue;
        const int lo = max(c - half, 0), hi = min(c - half + w_m, L);   // c in [lo, hi)
        for (int wd = lo >> 5; wd <= (hi - 1) >> 5; ++wd) {
            const int a = max(lo - 32 * wd, 0), e = min(hi - 32 * wd, 32);   // bits [a, e) of this word
            const uint32_t bits = (e >= 32 ? 0xffffffffu : ((1u << e) - 1u)) & ~((1u << a) - 1u);
            atomicOr(&s_mand[wd], bits);
        }
    }
    __syncthreads();
    const int budget = s_budget;

    // -- the budget over the other tokens: keys are the distances' bits (d >= +0, so the bit
    //    patterns order like the values).  Every thread owns the contiguous positions
    //    [lo, hi); up to kRegKeys of them are held in registers for the whole selection.
    const float* dl = dist + static_cast<int64_t>(bl) * L;
    int lo, hi;
    thread_chunk(L, &lo, &hi);
    if ((L + kSelThreads - 1) / kSelThreads <= kRegKeys)
        select_from_registers(dl, s_mand, lo, hi, L, budget, upd_idx + static_cast<int64_t>(bl) * L, &n_upd[bl], &sm);
    else
        select_from_memory(dl, s_mand, lo, hi, L, budget, upd_idx + static_cast<int64_t>(bl) * L, &n_upd[bl], &sm);
}

}  // namespace

int dcu_chunks(int L) { return (L + kTokPerWg - 1) / kTokPerWg; }

size_t dcu_workspace_bytes(int B, int NL, int L) {
    return static_cast<size_t>(B) * NL * dcu_chunks(L) * sizeof(double);
}

hipError_t launch_dcu_select(fdl_dtype dtype, const DcuArgs& a, hipStream_t stream) {
    const int nc = dcu_chunks(a.L);
    double* part = static_cast<double*>(a.ws);
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.NL * nc));
    if (dtype == FDL_BF16)
        hipLaunchKernelGGL(dcu_distance_kernel<uint16_t>, grid, dim3(kDistThreads), 0, stream,
                           static_cast<const uint16_t*>(a.x_now), a.xnb, a.xnl, a.xnr,
                           static_cast<const uint16_t*>(a.x_prev), a.xpb, a.xpl, a.xpr, a.NL, a.L, a.H, nc, a.dist,
                           part);
    else
        hipLaunchKernelGGL(dcu_distance_kernel<float>, grid, dim3(kDistThreads), 0, stream,
                           static_cast<const float*>(a.x_now), a.xnb, a.xnl, a.xnr,
                           static_cast<const float*>(a.x_prev), a.xpb, a.xpl, a.xpr, a.NL, a.L, a.H, nc, a.dist,
                           part);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const dim3 grid_l(static_cast<unsigned>(a.B * a.NL));
    hipLaunchKernelGGL(dcu_activity_kernel, grid_l, dim3(kDistThreads), 0, stream, part, nc, a.activity);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(dcu_select_kernel, grid_l, dim3(kSelThreads), 0, stream, a.dist, a.activity, a.NL, a.L,
                       a.keys, a.n_keys, a.w_m, a.total, a.budgets, a.upd_idx, a.n_upd);
    return hipGetLastError();
}

}  // namespace fdl
