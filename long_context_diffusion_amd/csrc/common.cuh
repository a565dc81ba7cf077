// Device helpers shared by the Focus-dLLM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fdl.h"

namespace fdl {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// x rounded up to a multiple of m (host-side workspace layout).
inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

// ------------------------------------------------------------------ bf16 helpers

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 bits (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element loads/stores for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {  // bf16 stored as raw bits
    static __device__ __forceinline__ float load(const uint16_t* p) {
        return __uint_as_float(static_cast<uint32_t>(*p) << 16);
    }
    static __device__ __forceinline__ void store(uint16_t* p, float x) {
        *p = static_cast<uint16_t>(f32_to_bf16_bits(x));
    }
};

// 2^x on the transcendental unit (v_exp_f32).  Results below 2^-126 flush to zero,
// which is harmless for softmax weights and saves the denormal-range fix-up that
// the libm exp2f wraps around the instruction.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ ordered keys

// Monotone map of a float to uint32: a < b  <=>  okey(a) < okey(b); -0.0 maps like +0.0.
__device__ __forceinline__ uint32_t okey32(float f) {
    uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t okey64(double f) {
    uint64_t u = static_cast<uint64_t>(__double_as_longlong(f == 0.0 ? 0.0 : f));
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// ------------------------------------------------------------------ wave / block scans

__device__ __forceinline__ int wave_inclusive_sum(int x) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    return x;
}

// Exclusive prefix sum over the block (blockDim.x a multiple of 64, <= 1024).
// `s_tmp` holds >= 17 ints.  Returns the exclusive prefix; *total gets the block sum.
// Every thread reads the per-wave totals itself (broadcast LDS reads), so there is no
// serial pass over the waves.
__device__ inline int block_exclusive_sum(int x, int* s_tmp, int* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int nw = blockDim.x / kWave;
    const int inc = wave_inclusive_sum(x);
    if (lane == kWave - 1) s_tmp[wv] = inc;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = i < nw ? s_tmp[i] : 0;
        before += i < wv ? t : 0;
        tot += t;
    }
    *total = tot;
    __syncthreads();   // s_tmp is free for the next call
    return before + inc - x;
}

// Sum of a 64-bit value over the block (blockDim.x a multiple of 64, <= 512); every thread
// gets the total.  s_tmp holds at least blockDim.x / 64 values.  Two barriers.
__device__ inline uint64_t block_sum_u64(uint64_t x, uint64_t* s_tmp) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
    if ((threadIdx.x & (kWave - 1)) == 0) s_tmp[threadIdx.x / kWave] = x;
    __syncthreads();
    uint64_t tot = 0;
    for (int w = 0; w < static_cast<int>(blockDim.x) / kWave; ++w) tot += s_tmp[w];
    __syncthreads();
    return tot;
}

// Canonical form of an index list: the entries v of src[0, n) with lo <= v < hi, ascending and
// each once, written to dst[0, m); returns m (the same in every thread).  Every thread of the
// block calls it; blockDim.x is a multiple of 64.  The selections of this library write
// strictly ascending lists with -1 padding after them: those cost one compaction pass and a
// check.  Any other order, repeated entries and out-of-range entries anywhere in the list are
// sorted (bitonic, in LDS) and de-duplicated.  dst (LDS) holds at least the next power of two
// >= n ints, scratch (LDS) at least n ints; s_tmp at least 17 ints.
__device__ inline int canonical_ids(const int32_t* src, int n, int lo, int hi, int* dst, int* scratch,
                                    int* s_tmp) {
    const int tid = threadIdx.x, nt = blockDim.x;
    int m = 0;
    for (int base = 0; base < n; base += nt) {
        const int i = base + tid;
        const int v = i < n ? src[i] : lo - 1;
        const bool ok = i < n && v >= lo && v < hi;
        int tot;
        const int off = block_exclusive_sum(ok ? 1 : 0, s_tmp, &tot);
        if (ok) dst[m + off] = v;
        m += tot;
    }
    __syncthreads();
    int bad = 0;
    for (int i = tid + 1; i < m; i += nt) bad += dst[i] <= dst[i - 1] ? 1 : 0;
    int nbad;
    block_exclusive_sum(bad, s_tmp, &nbad);
    if (nbad == 0) return m;
    int p2 = 1;
    while (p2 < m) p2 <<= 1;
    for (int i = m + tid; i < p2; i += nt) dst[i] = 0x7fffffff;
    __syncthreads();
    for (int k = 2; k <= p2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int t = tid; t < p2 / 2; t += nt) {
                const int i = (t / j) * 2 * j + (t % j);   // bit j of i is clear; partner i + j
                const int x = dst[i], y = dst[i + j];
                if ((x > y) == ((i & k) == 0)) {
                    dst[i] = y;
                    dst[i + j] = x;
                }
            }
            __syncthreads();
        }
    }
    int u = 0;
    for (int base = 0; base < m; base += nt) {
        const int i = base + tid;
        const int v = i < m ? dst[i] : 0;
        const bool keep = i < m && (i == 0 || dst[i - 1] != v);
        int tot;
        const int off = block_exclusive_sum(keep ? 1 : 0, s_tmp, &tot);
        if (keep) scratch[u + off] = v;
        u += tot;
    }
    __syncthreads();
    for (int i = tid; i < u; i += nt) dst[i] = scratch[i];
    __syncthreads();
    return u;
}

// Keeps the entries of list[0, n) (LDS) for which drop(v) is false, in order; returns the new
// length.  scratch (LDS) holds at least n ints.  Every thread of the block calls it.
template <typename Drop>
__device__ inline int filter_ids(int* list, int n, int* scratch, int* s_tmp, Drop drop) {
    const int tid = threadIdx.x, nt = blockDim.x;
    int u = 0;
    for (int base = 0; base < n; base += nt) {
        const int i = base + tid;
        const int v = i < n ? list[i] : 0;
        const bool keep = i < n && !drop(v);
        int tot;
        const int off = block_exclusive_sum(keep ? 1 : 0, s_tmp, &tot);
        if (keep) scratch[u + off] = v;
        u += tot;
    }
    __syncthreads();
    for (int i = tid; i < u; i += nt) list[i] = scratch[i];
    __syncthreads();
    return u;
}

// True when sorted[0, n) (ascending, LDS or global) holds x.
__device__ __forceinline__ bool sorted_contains(const int* sorted, int n, int x) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (sorted[mid] < x) lo = mid + 1; else hi = mid;
    }
    return lo < n && sorted[lo] == x;
}

// ------------------------------------------------------------------ top-k selection
//
// Selections keep the k entries with the largest ordered keys, the lower index
// first among equal keys, and write them in ascending index order.  KeyFn(j, &key)
// loads the key of entry j and returns whether j takes part; it must be safe to call
// for every j in [0, n).  Keys are read in batches of independent loads.

// Shared scratch for the selection helpers.  Each wave counts into its own histogram
// (skewed keys would otherwise pile every atomic onto one or two LDS words).
constexpr int kMaxWaves = 16;
struct SelectSmem {
    alignas(16) int hist[kMaxWaves][256];
    int tmp[17];
    int digit;
    int remaining;
};

// Per-thread contiguous chunk [lo, hi) of [0, n).
__device__ __forceinline__ void thread_chunk(int n, int* lo, int* hi) {
    const int chunk = (n + blockDim.x - 1) / blockDim.x;
    *lo = min(n, static_cast<int>(threadIdx.x) * chunk);
    *hi = min(n, *lo + chunk);
}

// Calls body(j, key) for every valid j in [lo, hi), loading 8 keys at a time.
template <typename U, typename KeyFn, typename Body>
__device__ __forceinline__ void for_each_key(int lo, int hi, KeyFn key_of, Body body) {
    constexpr int kBatch = 8;
    for (int j0 = lo; j0 < hi; j0 += kBatch) {
        U keys[kBatch];
        bool ok[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int j = j0 + u;
            const bool in = j < hi;
            ok[u] = key_of(in ? j : lo, &keys[u]) && in;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (ok[u]) body(j0 + u, keys[u]);
    }
}

// hist[digit] += 1 for every lane of the wave with `on`.  Skewed keys put most of a
// wave on one or two digits, and same-address LDS atomics serialise, so the lanes that
// share a leader lane's digit are counted with one atomic, for up to 4 leaders; the
// lanes left over (many distinct digits, hence few conflicts) add their own.
__device__ __forceinline__ void wave_count(int* hist, int digit, bool on) {
    const int lane = threadIdx.x & (kWave - 1);
    uint64_t pending = __ballot(on);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        if (pending == 0) break;   // the same on every lane
        const int leader = __builtin_ctzll(pending);
        const int dl = __shfl(digit, leader, kWave);
        const uint64_t same = __ballot(on && digit == dl) & pending;
        if (lane == leader) atomicAdd(&hist[dl], static_cast<int>(__popcll(same)));
        pending &= ~same;
    }
    if ((pending >> lane) & 1ull) atomicAdd(&hist[digit], 1);
}

// One digit of a radix select: with every wave's histogram of the current digit in
// sm->hist (complete: the caller synchronised), finds the digit of the *remaining-th largest
// key and the rank left within it (*remaining updated), in every thread.  Three barriers;
// the histograms are free again on return.
__device__ inline int radix_pick_digit(SelectSmem* sm, int* remaining) {
    const int nw = blockDim.x / kWave;
    if (threadIdx.x < kWave) {
        // lane l owns bins 4l..4l+3; find the bin holding the remaining-th largest
        const int l = threadIdx.x;
        int h[4] = {0, 0, 0, 0};
        for (int w = 0; w < nw; ++w)
            for (int q = 0; q < 4; ++q) h[q] += sm->hist[w][4 * l + q];
        const int mine = h[0] + h[1] + h[2] + h[3];
        int suffix = mine;  // sum over lanes >= l
        for (int off = 1; off < kWave; off <<= 1) {
            const int y = __shfl_down(suffix, off, kWave);
            if (l + off < kWave) suffix += y;
        }
        int above = suffix - mine;
        for (int q = 3; q >= 0; --q) {
            if (above < *remaining && *remaining <= above + h[q]) {
                sm->digit = 4 * l + q;
                sm->remaining = *remaining - above;
            }
            above += h[q];
        }
    }
    __syncthreads();
    const int dgt = sm->digit;
    *remaining = sm->remaining;
    __syncthreads();
    return dgt;
}

// Radix select: the k-th largest ordered key among the valid entries of [0, n)
// (1 <= k <= number of valid entries).  Every thread of the block must call it.
template <typename U, typename KeyFn>
__device__ U block_kth_largest(int n, int k, KeyFn key_of, SelectSmem* sm) {
    constexpr int kBits = 8 * sizeof(U);
    U prefix = 0, prefix_mask = 0;
    int remaining = k;
    int lo, hi;
    thread_chunk(n, &lo, &hi);
    const int nw = blockDim.x / kWave;
    const int wv = threadIdx.x / kWave;
    for (int shift = kBits - 8; shift >= 0; shift -= 8) {
        for (int i = threadIdx.x; i < nw * 256; i += blockDim.x) sm->hist[i / 256][i % 256] = 0;
        __syncthreads();
        for_each_key<U>(lo, hi, key_of, [&](int, U kj) {
            wave_count(sm->hist[wv], static_cast<int>((kj >> shift) & 0xff), (kj & prefix_mask) == prefix);
        });
        __syncthreads();
        const int dgt = radix_pick_digit(sm, &remaining);
        prefix |= static_cast<U>(dgt) << shift;
        prefix_mask |= static_cast<U>(0xff) << shift;
    }
    return prefix;
}

// Writes idx_of(j) for the k valid entries with the largest keys, in ascending j,
// to out[0..), pads out[..cap) with -1 and returns the number written.
template <typename U, typename KeyFn, typename IdxFn>
__device__ int block_emit_topk(int n, int k, KeyFn key_of, IdxFn idx_of, int32_t* out, int cap,
                               SelectSmem* sm) {
    int lo, hi;
    thread_chunk(n, &lo, &hi);
    int nvalid_local = 0;
    for_each_key<U>(lo, hi, key_of, [&](int, U) { ++nvalid_local; });
    int nvalid;
    block_exclusive_sum(nvalid_local, sm->tmp, &nvalid);
    const bool take_all = nvalid <= k;
    const int nsel = take_all ? nvalid : max(k, 0);
    U thr = 0;
    if (!take_all && nsel > 0) thr = block_kth_largest<U>(n, nsel, key_of, sm);
    int gt = 0, eq = 0;
    if (nsel > 0) {
        // counted without branches: a conditional increment of one of two counters
        // makes the compiler keep them in an indexed stack array (scratch memory)
        for_each_key<U>(lo, hi, key_of, [&](int, U kj) {
            const bool above = take_all || kj > thr;
            gt += above ? 1 : 0;
            eq += (!above && kj == thr) ? 1 : 0;
        });
    }
    int gt_total, eq_total;
    int gt_before = block_exclusive_sum(gt, sm->tmp, &gt_total);
    int eq_before = block_exclusive_sum(eq, sm->tmp, &eq_total);
    const int ties_taken = nsel - gt_total;  // lowest-index ties fill the rest
    if (nsel > 0) {
        for_each_key<U>(lo, hi, key_of, [&](int j, U kj) {
            const bool above = take_all || kj > thr;
            const bool tie = !above && kj == thr;
            if (above) out[gt_before + min(eq_before, ties_taken)] = idx_of(j);
            if (tie && eq_before < ties_taken) out[gt_before + eq_before] = idx_of(j);
            gt_before += above ? 1 : 0;
            eq_before += tie ? 1 : 0;
        });
    }
    for (int i = nsel + threadIdx.x; i < cap; i += blockDim.x) out[i] = -1;
    return nsel;
}

// Top-k of n <= blockDim.x entries with distinct 64-bit keys, key_of(j) (read once per
// entry), so the order is total: rank(j) = #{i : key_i > key_j}, and j is taken when
// rank(j) < k.  A thread holds 4 consecutive entries in registers and compares them with
// one slice of the keys (S slices of `span` keys, S a power of two <= 64: one LDS read
// serves 4 comparisons, each a single 64-bit compare); the S partial counts of a group
// sit in adjacent lanes and add with shuffles.  The keys are copied into sm->hist with
// two spare slots after every slice, so the slices start on different LDS banks (slices
// starting 16 or 32 keys apart would otherwise all read the same two banks).  The taken
// entries are then written in index order from per-wave ballots.
template <typename KeyFn, typename IdxFn>
__device__ int block_topk_distinct(int n, int k, KeyFn key_of, IdxFn idx_of, int32_t* out, int cap,
                                   SelectSmem* sm) {
    const int nsel = min(max(k, 0), n);
    constexpr int kPer = 4;
    const int ngroups = (n + kPer - 1) / kPer;
    int S = 1;
    while (S < kWave && 2 * S * ngroups <= static_cast<int>(blockDim.x)) S *= 2;
    const int span = max((n + S - 1) / S, 1);
    uint64_t* pk = reinterpret_cast<uint64_t*>(&sm->hist[0][0]);        // <= 1152 keys: 9 KB
    int* s_rank = &sm->hist[10][0];                                      // <= 1024 ranks
    uint64_t* s_mask = reinterpret_cast<uint64_t*>(&sm->hist[15][0]);    // one per wave
    for (int i = threadIdx.x; i < n; i += blockDim.x) pk[i + 2 * (i / span)] = key_of(i);
    __syncthreads();
    const int jg = static_cast<int>(threadIdx.x) / S;
    const int sl = static_cast<int>(threadIdx.x) % S;
    if (jg < ngroups) {
        const int j0 = kPer * jg;
        uint64_t kj[kPer];
#pragma unroll
        for (int r = 0; r < kPer; ++r) {
            const int jj = min(j0 + r, n - 1);
            kj[r] = pk[jj + 2 * (jj / span)];
        }
        int cnt[kPer] = {0, 0, 0, 0};
        const int i0 = min(n, sl * span), i1 = min(n, i0 + span);
        const uint64_t* ps = pk + 2 * sl;   // key i of this slice at ps[i]
        constexpr int kBatch = 8;
        int ib = i0;
        for (; ib + kBatch <= i1; ib += kBatch) {
            uint64_t ki[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; ++u) ki[u] = ps[ib + u];
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
#pragma unroll
                for (int r = 0; r < kPer; ++r) cnt[r] += ki[u] > kj[r] ? 1 : 0;
        }
        for (; ib < i1; ++ib) {
            const uint64_t ki = ps[ib];
#pragma unroll
            for (int r = 0; r < kPer; ++r) cnt[r] += ki > kj[r] ? 1 : 0;
        }
        for (int off = 1; off < S; off <<= 1)
#pragma unroll
            for (int r = 0; r < kPer; ++r) cnt[r] += __shfl_xor(cnt[r], off, kWave);
        if (sl == 0) {
#pragma unroll
            for (int r = 0; r < kPer; ++r)
                if (j0 + r < n) s_rank[j0 + r] = cnt[r];
        }
    }
    __syncthreads();
    const int j = static_cast<int>(threadIdx.x);
    const int lane = j & (kWave - 1), wv = j / kWave;
    const bool take = j < n && s_rank[j] < nsel;
    const uint64_t m = __ballot(take);
    if (lane == 0) s_mask[wv] = m;
    __syncthreads();
    if (take) {
        int pos = __popcll(m & ((uint64_t(1) << lane) - 1));
        for (int w = 0; w < wv; ++w) pos += __popcll(s_mask[w]);
        out[pos] = idx_of(j);
    }
    for (int i = nsel + j; i < cap; i += blockDim.x) out[i] = -1;
    __syncthreads();   // the output (LDS or global) is complete and the scratch free
    return nsel;
}

// Selection over 32-bit keys already in LDS (every entry valid), the lower index first
// among equal keys.  Up to blockDim.x entries: ranked by the distinct 64-bit keys
// (key << 32 | ~index), same order; larger sets use the radix select.
template <typename IdxFn>
__device__ int block_topk_lds(int n, int k, const uint32_t* keys, IdxFn idx_of, int32_t* out, int cap,
                              SelectSmem* sm) {
    if (n > static_cast<int>(blockDim.x)) {
        auto key_of = [&](int j, uint32_t* key) -> bool {
            *key = keys[j];
            return true;
        };
        return block_emit_topk<uint32_t>(n, k, key_of, idx_of, out, cap, sm);
    }
    auto key_of = [&](int j) {
        return (static_cast<uint64_t>(keys[j]) << 32) | (0xffffffffu - static_cast<uint32_t>(j));
    };
    return block_topk_distinct(n, k, key_of, idx_of, out, cap, sm);
}

}  // namespace fdl
