// Tile layouts and helpers of the bf16 head-dim-128 attention kernel (attention_d128.hip):
// 64-key tiles of K (rows of 256 bytes) and of V^T (128 rows of 128 bytes) in LDS, the LDS
// map of a sparse key set, and the workgroup barrier that leaves the newest loads in flight.
#pragma once

#include "attention.cuh"

namespace fdl {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowB = 256;           // bytes per K/V row in LDS
constexpr int kTileB = 64 * kRowB;   // one 64-key tile: 16 KB
constexpr float kSlack = 8.0f;       // max growth (log2 units) tolerated before a rescale

// key sets: every key of [0, L); I_p mapped from LDS copies of its parts; I_p read
// from the list attn_prep wrote (parts too large for LDS)
enum KeyMode { kDense = 0, kSparseLds = 1, kSparseList = 2 };

__device__ __forceinline__ int swz_k(int r, int c) { return c ^ (r & 15); }
// Row r of a K tile (and of the S^T accumulator) holds key position vt_row(r) of the
// tile, where vt_row swaps bits 2 and 3.  A lane's P fragment for 16-key chunk kc holds
// S^T rows 16kc + 8(j/4) + 4hf + j%4, j = 0..7, which are then key positions
// 16kc + 8hf + j: so slot s (0..63) of a V^T row is simply key position s, and 8
// consecutive keys of one d fill one 16-byte chunk.
// V^T tile: 128 rows (d) of 128 bytes.  Chunk c of row d sits at c ^ vt_swz(d), chosen by measuring the LDS bank-conflict
// counter over candidate swizzles on gfx950: the fragment reads are conflict-free and the
// transposing stores (rows 8 apart in one instruction) 2-way; with bits 1-3 of d alone
// the stores are 8-way.
__host__ __device__ constexpr int vt_row(int s) { return (s & ~12) | ((s & 4) << 1) | ((s & 8) >> 1); }
__host__ __device__ constexpr int vt_swz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }
__host__ __device__ constexpr int vt_off(int d, int s) { return d * 128 + 16 * ((s >> 3) ^ vt_swz(d)) + 2 * (s & 7); }

// The two writers of a V^T tile compute vt_off in closed forms; both are checked here
// against it at compile time.  The V^T DMA: instruction m, lane l writes LDS bytes
// 1024 m + 16 l, the chunk of row d = 8 m + l / 8 that holds slots 8 ((l % 8) ^ vt_swz(d)) + 0..7.
// The transposing store of thread t: word e at A(t) ^ (128 e + 16 (e / 2)), d = 8 (t % 16) + e,
// slot vt_row(2 (t / 16)).
constexpr bool vt_writers_match_layout() {
    for (int m = 0; m < 16; ++m)
        for (int l = 0; l < 64; ++l) {
            const int d = 8 * m + l / 8;
            if (vt_off(d, 8 * ((l % 8) ^ vt_swz(d))) != 1024 * m + 16 * l) return false;
        }
    for (int t = 0; t < 512; ++t) {
        const int c8 = t & 15, sl = vt_row(2 * (t >> 4));
        const int A = 1024 * c8 + 2 * (sl & 7) + 16 * (((sl >> 3) ^ (4 * (c8 & 1)) ^ (c8 >> 1)) & 7);
        for (int e = 0; e < 8; ++e)
            if ((A ^ (128 * e + 16 * (e >> 1))) != vt_off(8 * c8 + e, sl)) return false;
    }
    return true;
}
static_assert(vt_writers_match_layout(), "V^T writers disagree with vt_off");


// floor(n / d) for 0 <= n < 2^30 and d >= 1, with m = ceil(2^32 / d) for d >= 2.
__device__ __forceinline__ int div_magic(int n, int d, uint32_t m) {
    if (d == 1) return n;
    uint32_t q = __umulhi(static_cast<uint32_t>(n), m);   // floor(n/d) or one more
    if (q * static_cast<uint32_t>(d) > static_cast<uint32_t>(n)) --q;
    return static_cast<int>(q);
}

// Workgroup barrier that leaves this wave's newest `keep` loads in flight: LDS reads
// have returned and every older load (LDS DMA included) has landed.  A plain
// __syncthreads() would also wait for the newest loads: its release fence drains
// every outstanding memory operation.
template <int keep>
__device__ __forceinline__ void barrier_keep() {
    static_assert(keep >= 0 && keep < 16, "vmcnt field");
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(keep | (7 << 4));   // vmcnt(keep) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The value this lane's partner (lane ^ 32) holds.
__device__ __forceinline__ float xhalf(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}


// The LDS map of the sparse key set I_p of sequence b (of its KV head g, when every KV head
// has its own block list): the selected blocks (s_blk, ascending,
// n_sel of them), then [P, L), then the sinks that no selected block holds (s_unc).  The
// key set has n_keys positions: [0, n_blk) in blocks, [n_blk, sink0) the generation
// region, [sink0, n_keys) the uncovered sinks.  The block and sink lists are taken as the
// sets of their valid ids.  Lists as the selections write them (valid ids strictly
// ascending, then padding) are recognised with one reduction and mapped as they stand; any
// other list is brought to canonical form (canonical_ids: sorted and de-duplicated in LDS,
// with `scratch`, at least 1024 ints of LDS, as the sort's scratch).  Every thread of the
// block calls it, THREADS of them; C and n_sinks are at most 1024.  PER_HEAD: the block list
// of KV head g (a.blk_per_head), else the sequence's one list.
template <int THREADS, bool PER_HEAD>
__device__ inline void build_key_map(const AttnArgs& a, int b, int g, int* s_blk, int* s_unc, int* s_tmp,
                                     uint64_t* s_tmp64, int* scratch, int& n_blk, int& sink0, int& n_keys) {
    constexpr int EPT = 1024 / THREADS;   // entries of each list per thread
    const int tid = threadIdx.x;
    const int32_t* blk_g = a.block_idx + static_cast<int64_t>(PER_HEAD ? b * a.Hkv + g : b) * a.C;
    const int32_t* snk_g = a.sink_idx + static_cast<int64_t>(b) * a.n_sinks;
    int sv[EPT];
    uint64_t packed = 0;   // bad entries << 40 | valid block ids << 20 | valid sinks
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int i = EPT * tid + e;
        const int bv = i < a.C ? blk_g[i] : -1;
        const int bp = (i < a.C && i > 0) ? blk_g[i - 1] : -1;
        sv[e] = i < a.n_sinks ? snk_g[i] : -1;
        const int sp = (i < a.n_sinks && i > 0) ? snk_g[i - 1] : -1;
        const bool bin = bv >= 0 && bv < a.nb, bpin = bp >= 0 && bp < a.nb;
        const bool sin = sv[e] >= 0 && sv[e] < a.L, spin = sp >= 0 && sp < a.L;
        const bool bad = (bin && i > 0 && !(bpin && bp < bv)) || (sin && i > 0 && !(spin && sp < sv[e]));
        packed += (static_cast<uint64_t>(bad) << 40) | (static_cast<uint64_t>(bin) << 20) | static_cast<uint64_t>(sin);
        if (bin) s_blk[i] = bv;   // in canonical lists the valid ids are the prefix
    }
    packed = block_sum_u64(packed, s_tmp64);   // also orders the s_blk writes before the reads
    int n_sel, n_unc;
    if ((packed >> 40) == 0) {
        n_sel = static_cast<int>((packed >> 20) & 0xfffff);
        const int n_snk = static_cast<int>(packed & 0xfffff);
        int take = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int i = EPT * tid + e;
            const bool t = i < n_snk && sv[e] < a.P && !sorted_contains(s_blk, n_sel, sv[e] / a.bs);
            take |= (t ? 1 : 0) << e;
        }
        int tot;
        int off = block_exclusive_sum(__builtin_popcount(take), s_tmp, &tot);
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if ((take >> e) & 1) s_unc[off++] = sv[e];
        n_unc = tot;
        __syncthreads();
    } else {
        n_sel = canonical_ids(blk_g, a.C, 0, a.nb, s_blk, scratch, s_tmp);
        n_unc = canonical_ids(snk_g, a.n_sinks, 0, a.P, s_unc, scratch, s_tmp);
        n_unc = filter_ids(s_unc, n_unc, scratch, s_tmp, [&](int j) { return sorted_contains(s_blk, n_sel, j / a.bs); });
    }
    n_blk = n_sel * a.bs;
    if (n_sel > 0 && s_blk[n_sel - 1] == a.nb - 1) n_blk -= a.nb * a.bs - a.P;
    sink0 = n_blk + (a.L - a.P);
    n_keys = sink0 + n_unc;
}

}  // namespace fdl
