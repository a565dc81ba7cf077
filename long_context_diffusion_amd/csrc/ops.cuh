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
    float* kbar;            // [B, Hkv, nb, d] block means written by block_means, or NULL
    const float* kbar_in;   // [B, Hkv, nb, d] block means the relevance is scored against
    double* rpart;          // [B, Hkv, nb] each KV head's part of R (its max with kScoreMax)
    double* rfull;          // [B, nb]
    int mode;               // kScorePerHead | kScoreMax bits (0: one summed R per sequence)
};
constexpr int kScorePerHead = 1;   // one relevance and block set per KV head
constexpr int kScoreMax = 2;       // relevance = max over the queries instead of their sum

hipError_t launch_pcgi_select(const float* conf, const uint8_t* mask, int B, int L, int k, int w,
                              int32_t* focus_idx, int32_t* n_focus, int k_cap,
                              int32_t* active_idx, int32_t* n_active, int nq_max,
                              hipStream_t stream);

size_t sink_workspace_bytes(int B, int Hkv, int L);
hipError_t launch_sink_identify(fdl_dtype dtype, int d, SinkArgs a, int n_sinks, int32_t* sink_idx,
                                float* user_scores, void* ws, hipStream_t stream);

size_t block_workspace_bytes(int B, int Hq, int Hkv, int P, int d, int bs, int nq_max);
hipError_t launch_block_means(fdl_dtype dtype, int d, const BlockArgs& a, hipStream_t stream);

// approximate KV cache refresh (cache.hip)
struct CacheArgs {
    int B, Hkv, L, P, d, bs, nb, n_max;
    const int32_t* rows;     // [B, n_max] refreshed positions, -1 entries skipped
    const int32_t* n_rows;   // [B] valid entries, or NULL (all n_max)
    const void* k_new;
    int64_t knb, knh, knr;
    const void* v_new;
    int64_t vnb, vnh, vnr;
    void* k;
    int64_t ksb, ksh, ksr;
    void* v;
    int64_t vsb, vsh, vsr;
    void* vt;                // [B, Hkv, d, L] keys contiguous, or NULL
    int64_t vtsb, vtsh, vtsd;
    float* kbar;             // [B, Hkv, nb, d]
};
hipError_t launch_kv_scatter(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream);
constexpr int kFusedMaxBs = 2048;   // largest block size of the fused refresh (LDS row map)
hipError_t launch_kv_refresh_means(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream);
hipError_t launch_block_means_refresh(fdl_dtype dtype, const CacheArgs& a, hipStream_t stream);
hipError_t launch_block_score_topc(fdl_dtype dtype, int d, BlockArgs a, int C, int32_t* block_idx,
                                   double* R_out, void* ws, hipStream_t stream);

// dynamic cache update scoring (dcu.hip)
constexpr int kDcuMaxTokens = 1 << 18;   // tokens per layer (the mandatory-window bitmask sits in LDS)
constexpr int kDcuMaxLayers = 1024;
struct DcuArgs {
    int B, NL, L, H;
    const void* x_now;
    int64_t xnb, xnl, xnr;
    const void* x_prev;
    int64_t xpb, xpl, xpr;
    const int32_t* keys;     // [B, n_keys] key tokens, entries outside [0, L) ignored
    int n_keys, w_m, total;
    float* dist;             // [B, NL, L]
    double* activity;        // [B, NL]
    int32_t* budgets;        // [B, NL]
    int32_t* upd_idx;        // [B, NL, L], the first n_upd entries written
    int32_t* n_upd;          // [B, NL]
    void* ws;                // [B, NL, dcu_chunks(L)] doubles
};
int dcu_chunks(int L);
size_t dcu_workspace_bytes(int B, int NL, int L);
hipError_t launch_dcu_select(fdl_dtype dtype, const DcuArgs& a, hipStream_t stream);

// token confidence and unmasking (confidence.hip)
constexpr int kMaxConfRows = 4096;   // listed rows per sequence
size_t confidence_workspace_bytes(int B, int V, int m_max);
hipError_t launch_confidence_unmask(fdl_dtype dtype, int B, int L, int V, const void* logits, int64_t lsb,
                                    int64_t lsr, const int32_t* pos, const int32_t* n_rows, int m_max, int n_t,
                                    uint8_t* mask, float* conf, int32_t* tokens, int32_t* unmasked, void* ws,
                                    hipStream_t stream);

// calibrate.hip
hipError_t launch_calib_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream);
hipError_t launch_calib_mfma(int workgroups, int iters, float a_val, float b_val, float* sink, hipStream_t stream);

}  // namespace fdl
