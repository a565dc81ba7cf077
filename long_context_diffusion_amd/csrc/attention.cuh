// Shared description of an attention launch (dense or sparse key set).
#pragma once

#include "common.cuh"

namespace fdl {

struct AttnArgs {
    const void* q;
    int64_t qsb, qsh, qsr;
    const int32_t* q_idx;  // [B, nq_max] physical query row of each logical row, or NULL
    const int32_t* n_q;    // [B] valid logical rows, or NULL (all nq_max)
    int nq_max;
    const void* k;
    int64_t ksb, ksh, ksr;
    const void* v;
    int64_t vsb, vsh, vsr;
    const void* vt;        // V with keys contiguous, [B, Hkv, d, L] by strides (b, h, d), or NULL
    int64_t vtsb, vtsh;
    int vtsd;
    void* o;
    int64_t osb, osh, osr;
    float* lse;            // [B, Hq, nq_max] or NULL
    int B, Hq, Hkv, L, P, Gq;
    float sl2;             // softmax scale times log2(e)
    int sparse;            // 0: keys [0, L); 1: I_p from sink_idx / block_idx / [P, L)
    const int32_t* sink_idx;
    int n_sinks;
    const int32_t* block_idx;  // [B, C], or [B, Hkv, C] with blk_per_head
    int C, bs, nb;
    uint32_t bs_magic;     // ceil(2^32 / bs) for bs >= 2: division by bs as a multiply-high
    int n_splits;          // key-range splits (upper bound when dyn); > 1: partials combined by attn_merge
    int tiles_per_split;   // key tiles per split (static plans)
    int q_tiles;           // query tiles per (sequence, KV head) for nq_max rows
    int tiles_total;       // key tiles of the longest key set (upper bound)
    int slots;             // workgroups of a persistent launch
    int dyn;               // 1: the persistent kernel picks the split count from the device row counts
    int key_cap;           // row stride of kv_list (upper bound on |I_p|)
    int32_t* kv_list;      // [lists, key_cap] keys of I_p (sparse), built by attn_prep
    int32_t* n_keys;       // [lists] |I_p| (sparse)
    float* part_o;         // [B*Hq*nq_max][n_splits][d] unnormalised fp32 outputs
    float* part_ml;        // [B*Hq*nq_max][n_splits][2] running max (log2 domain) and sum
    int blk_per_head;      // 1: one block list (and key set) per KV head
};

// The key set of (sequence b, KV head g): one per sequence, or one per KV head of each
// sequence when every KV head has its own block list.
__host__ __device__ inline int list_of(const AttnArgs& a, int b, int g) { return a.blk_per_head ? b * a.Hkv + g : b; }
__host__ __device__ inline int n_lists(const AttnArgs& a) { return a.blk_per_head ? a.B * a.Hkv : a.B; }

struct AttnPlan {
    int q_tiles, n_splits, tiles_per_split, tile_keys, rows_per_tile, tiles_total;
    int64_t key_cap;
    size_t list_bytes, part_bytes, ws_bytes;
};

// Upper bound on |I_p| (keys attended by one sequence).
inline int64_t sparse_key_bound(int L, int P, int n_sinks, int C, int bs) {
    const int64_t nb = (static_cast<int64_t>(P) + bs - 1) / bs;
    const int64_t blocks = C < nb ? C : nb;
    int64_t blk_keys = blocks * bs;
    if (blk_keys > P) blk_keys = P;
    return blk_keys + (L - P) + n_sinks;
}

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 of differences never sees inf-inf

// Work units are (sequence b, KV head g, key split, query tile qt).  Only query tiles
// that hold valid rows (from the device-side row counts) get a workgroup; the rest
// of the grid exits at once.  A workgroup goes to XCD (blockIdx.x mod 8), so the
// units are laid out such that all query tiles of one (b, g, split) group run on the
// same XCD, one after another, and share that group's K/V tiles through its L2.
struct WorkUnit {
    int qt, split, g, b;
    bool valid;
};

// Query tiles with valid rows, per sequence (the same bound for every group of b).
__device__ __forceinline__ int valid_q_tiles(const AttnArgs& a, int rows_per_tile) {
    int nqt_max = 0;
    for (int b = 0; b < a.B; ++b) {
        const int nq = a.n_q ? a.n_q[b] : a.nq_max;
        nqt_max = max(nqt_max, (a.Gq * nq + rows_per_tile - 1) / rows_per_tile);
    }
    return nqt_max;
}

__device__ __forceinline__ WorkUnit decode_unit_id(const AttnArgs& a, int rows_per_tile, int id,
                                                   int n_splits, int nqt_max) {
    WorkUnit u;
    u.valid = false;
    u.qt = u.split = u.g = u.b = 0;
    if (nqt_max == 0) return u;
    const int n_groups = a.B * a.Hkv * n_splits;
    const int xcd = id & 7, slot = id >> 3;
    const int grp = (slot / nqt_max) * 8 + xcd;
    if (grp >= n_groups) return u;
    u.qt = slot % nqt_max;
    u.split = grp % n_splits;
    u.g = (grp / n_splits) % a.Hkv;
    u.b = grp / (n_splits * a.Hkv);
    const int nq = a.n_q ? a.n_q[u.b] : a.nq_max;
    u.valid = u.qt * rows_per_tile < a.Gq * nq;
    return u;
}

__device__ __forceinline__ WorkUnit decode_unit(const AttnArgs& a, int rows_per_tile) {
    return decode_unit_id(a, rows_per_tile, blockIdx.x, a.n_splits, valid_q_tiles(a, rows_per_tile));
}

// Split count of a persistent launch: as many key-range splits as it takes to give
// every workgroup of the grid one (query tile, split) item, judged from the rows that
// are valid on the device, within the bound the workspace was sized for and with at
// least kMinSplitTiles key tiles per split.  The merge kernel recomputes the same value.
constexpr int kMinSplitTiles = 8;
__device__ __forceinline__ int dyn_splits(const AttnArgs& a, int nqt_max) {
    const int units = a.B * a.Hkv * nqt_max;
    if (units == 0) return 1;
    int s = a.slots / units;
    s = min(s, a.tiles_total / kMinSplitTiles);
    s = min(s, a.n_splits);
    return max(s, 1);
}

template <typename T>
__device__ __forceinline__ void write_zero_row(const AttnArgs& a, int b, int h, int r, int d) {
    T* orow = static_cast<T*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr;
    for (int e = 0; e < d; ++e) orow[e] = T(0);
    if (a.lse) a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] = -INFINITY;
}


// Longest block and sink lists the key-list builder (attn_prep) brings to canonical form in
// LDS; longer lists are rejected on the host.
constexpr int kPrepMaxIds = 4096;

// Keys of one sparse key set that the d = 128 kernel can map in LDS by itself.
constexpr int kMapBlocks = 1024;
constexpr int kMapSinks = 1024;
__host__ __device__ inline bool sparse_map_in_lds(const AttnArgs& a) { return a.C <= kMapBlocks && a.n_sinks <= kMapSinks; }

// The bf16, head-dim-128 attention kernel (attention_d128.hip): persistent grid of
// d128_slots() workgroups, kD128Rows query rows each, split count chosen on the device.
constexpr int kD128Rows = 256;
constexpr int kD128MaxSlots = 512;    // persistent grid bound
int d128_slots();

// Split partials of the d = 128 kernel are stored per work item, at
// ((group (b, g), split), query tile, row in tile); p is the logical row among the
// Gq * nq stacked rows of KV head g.  Indices stay below
// min(kD128MaxSlots, max_splits * B * Hkv * query tiles) * kD128Rows, since more
// than one split is only taken while splits * units <= slots.
__device__ __forceinline__ int64_t d128_part_index(const AttnArgs& a, int nqt_max, int n_splits, int b,
                                                   int g, int split, int p) {
    const int64_t grp = (static_cast<int64_t>(b) * a.Hkv + g) * n_splits + split;
    return (grp * nqt_max + p / kD128Rows) * kD128Rows + p % kD128Rows;
}
hipError_t launch_attn_bf16_d128(const AttnArgs& a, hipStream_t stream);

AttnPlan plan_attention(fdl_dtype dtype, int B, int Hq, int Hkv, int d, int nq_max,
                        int64_t key_bound, bool sparse, bool per_head = false);

hipError_t launch_attention(fdl_dtype dtype, int d, const AttnArgs& args, const AttnPlan& plan,
                            hipStream_t stream);

}  // namespace fdl
