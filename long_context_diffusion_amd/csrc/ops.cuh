// Argument blocks and host launchers of the Focus-dLLM kernels.
#pragma once

#include "attention.cuh"

namespace fdl {

struct SinkArgs {
    const void* q;
    int64_t qsb, qsh, qsr;
    const int32_t* q_idx;
    const int32_t* n_q;
    int nq_max;
    const void* k;
    int64_t ksb, ksh, ksr;
    const float* lse;
    int B, Hq, Hkv, L, Gq;
    float sl2;        // scale * log2(e)
    float* part;      // [B, Hkv, L] per-KV-head partial scores
    float* scores;    // [B, L]
    int key_tiles;
};

struct BlockArgs {
    const void* q;
    int64_t qsb, qsh, qsr;
    const int32_t* q_idx;
    const int32_t* n_q;
    int nq_max;
    const void* k;
    int64_t ksb, ksh, ksr;
    int B, Hq, Hkv, P, Gq, bs, nb;
    float scale;
    float* kbar;      // [B, Hkv, nb, d] or NULL
    double* qsum;     // [B, Hkv, d]
    double* rpart;    // [B, Hkv, nb]
    double* rfull;    // [B, nb]
    int blocks_per_wg, scan_chunks;
};

hipError_t launch_pcgi_select(const float* conf, const uint8_t* mask, int B, int L, int k, int w,
                              int32_t* focus_idx, int32_t* n_focus, int k_cap,
                              int32_t* active_idx, int32_t* n_active, int nq_max,
                              hipStream_t stream);

size_t sink_workspace_bytes(int B, int Hkv, int L);
hipError_t launch_sink_identify(fdl_dtype dtype, int d, SinkArgs a, int n_sinks, int32_t* sink_idx,
                                float* user_scores, void* ws, hipStream_t stream);

size_t block_workspace_bytes(int B, int Hkv, int P, int d, int bs);
hipError_t launch_block_score_topc(fdl_dtype dtype, int d, BlockArgs a, int C, int32_t* block_idx,
                                   double* R_out, void* ws, hipStream_t stream);

}  // namespace fdl
