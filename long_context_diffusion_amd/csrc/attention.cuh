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
    void* o;
    int64_t osb, osh, osr;
    float* lse;            // [B, Hq, nq_max] or NULL
    int B, Hq, Hkv, L, P, Gq;
    float sl2;             // softmax scale times log2(e)
    int sparse;            // 0: keys [0, L); 1: I_p from sink_idx / block_idx / [P, L)
    const int32_t* sink_idx;
    int n_sinks;
    const int32_t* block_idx;
    int C, bs, nb;
    int n_splits;          // key-range splits; > 1: partials combined by attn_merge
    int tiles_per_split;   // key tiles per split
    int q_tiles;           // query tiles per (sequence, KV head)
    int key_cap;           // row stride of kv_list (upper bound on |I_p|)
    int32_t* kv_list;      // [B, key_cap] keys of I_p (sparse), built by attn_prep
    int32_t* n_keys;       // [B] |I_p| (sparse)
    float* part_o;         // [B*Hq*nq_max][n_splits][d] unnormalised outputs
    float* part_ml;        // [B*Hq*nq_max][n_splits][2] running max (log2 domain) and sum
};

struct AttnPlan {
    int q_tiles, n_splits, tiles_per_split, tile_keys, rows_per_tile;
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

AttnPlan plan_attention(fdl_dtype dtype, int B, int Hq, int Hkv, int d, int nq_max,
                        int64_t key_bound, bool sparse);

hipError_t launch_attention(fdl_dtype dtype, int d, const AttnArgs& args, const AttnPlan& plan,
                            hipStream_t stream);

}  // namespace fdl
