// Host side of the C ABI declared in include/fdl.h: argument validation,
// workspace sizing and kernel launches.  No allocation, no synchronisation.

#include <cmath>
#include <cstdint>

#include "ops.cuh"

using namespace fdl;

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline size_t elem_size(fdl_dtype dt) { return dt == FDL_BF16 ? 2 : 4; }

fdl_status check_dtype_dims(fdl_dtype dt, int B, int Hq, int Hkv, int L, int d) {
    if (dt != FDL_F32 && dt != FDL_BF16) return FDL_ERR_DTYPE;
    if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || d < 1) return FDL_ERR_SHAPE;
    if (Hq % Hkv != 0) return FDL_ERR_SHAPE;
    if (d != 64 && d != 128) return FDL_ERR_UNSUPPORTED;
    return FDL_OK;
}

// Row starts base + b*s.b + h*s.h + r*s.r must be 16-byte aligned, d contiguous elements
// must fit between rows (|s.r| >= d) and the row stride must be below 2^31 elements.
fdl_status check_tensor(const void* p, fdl_strides s, fdl_dtype dt, int d) {
    if (!p) return FDL_ERR_NULL;
    if (!aligned16(p)) return FDL_ERR_ALIGN;
    const int64_t e = static_cast<int64_t>(elem_size(dt));
    if ((s.b * e) % 16 || (s.h * e) % 16 || (s.r * e) % 16) return FDL_ERR_ALIGN;
    if (s.r < d && s.r > -d) return FDL_ERR_SHAPE;
    if (s.r >= (1ll << 31) || s.r <= -(1ll << 31)) return FDL_ERR_SHAPE;
    return FDL_OK;
}

// V^T (keys contiguous, rows indexed by d): read only by the bf16 d = 128 kernel, so it
// is checked (and used) only there.
fdl_status check_vt(const void* vt, fdl_strides s, fdl_dtype dt, int d, int L) {
    if (!vt || dt != FDL_BF16 || d != 128) return FDL_OK;
    if (!aligned16(vt) || s.b % 8 || s.h % 8 || s.r % 8) return FDL_ERR_ALIGN;
    if (s.r < L || s.r >= (1ll << 24)) return FDL_ERR_SHAPE;
    return FDL_OK;
}

fdl_status check_rows(int nq_max, int Gq) {
    if (nq_max < 0) return FDL_ERR_SHAPE;
    if (static_cast<int64_t>(nq_max) * Gq > (1ll << 30)) return FDL_ERR_SHAPE;
    return FDL_OK;
}

fdl_status check_ws(const void* ws, size_t have, size_t need) {
    if (need == 0) return FDL_OK;
    if (!ws || have < need) return FDL_ERR_WORKSPACE;
    if (!aligned16(ws)) return FDL_ERR_ALIGN;
    return FDL_OK;
}

inline float resolve_scale(float scale, int d) {
    return scale > 0.0f ? scale : static_cast<float>(1.0 / std::sqrt(static_cast<double>(d)));
}

inline fdl_status hip_status(hipError_t e) { return e == hipSuccess ? FDL_OK : FDL_ERR_HIP; }

constexpr float kLog2eF = 1.44269504088896340736f;

AttnArgs attn_args(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, const void* q, fdl_strides qs,
                   const int32_t* q_idx, const int32_t* n_q, int nq_max, const void* k, fdl_strides ks,
                   const void* v, fdl_strides vs, const void* vt, fdl_strides vts, float scale, int d,
                   void* o, fdl_strides os, float* lse, void* ws) {
    AttnArgs a{};
    a.q = q; a.qsb = qs.b; a.qsh = qs.h; a.qsr = qs.r;
    a.q_idx = q_idx; a.n_q = n_q; a.nq_max = nq_max;
    a.k = k; a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.v = v; a.vsb = vs.b; a.vsh = vs.h; a.vsr = vs.r;
    a.vt = dt == FDL_BF16 && d == 128 ? vt : nullptr;
    a.vtsb = vts.b; a.vtsh = vts.h; a.vtsd = static_cast<int>(vts.r);
    a.o = o; a.osb = os.b; a.osh = os.h; a.osr = os.r;
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L; a.P = P; a.Gq = Hq / Hkv;
    a.sl2 = resolve_scale(scale, d) * kLog2eF;
    a.part_o = static_cast<float*>(ws);
    (void)dt;
    return a;
}

// Workspace of fdl_sink_identify: the sink partial scores, then (used only when the caller
// passes no lse) the lse and output rows of a dense attention pass and that pass's workspace.
struct SinkWs {
    size_t sink, lse, out, attn, total;
};

SinkWs sink_ws_layout(fdl_dtype dt, int B, int Hq, int Hkv, int L, int d, int nq_max) {
    SinkWs w{};
    w.sink = round_up(sink_workspace_bytes(B, Hkv, L), 256);
    const size_t rows = static_cast<size_t>(B) * Hq * (nq_max > 0 ? nq_max : 0);
    w.lse = round_up(rows * sizeof(float), 256);
    w.out = round_up(rows * d * elem_size(dt), 256);
    w.attn = nq_max > 0 ? round_up(plan_attention(dt, B, Hq, Hkv, d, nq_max, L, false).ws_bytes, 256) : 0;
    w.total = w.sink + w.lse + w.out + w.attn;
    return w;
}

}  // namespace

extern "C" {

const char* fdl_status_string(fdl_status s) {
    switch (s) {
        case FDL_OK: return "ok";
        case FDL_ERR_NULL: return "a required pointer is NULL";
        case FDL_ERR_SHAPE: return "a size is out of range or inconsistent";
        case FDL_ERR_DTYPE: return "unsupported dtype";
        case FDL_ERR_ALIGN: return "a pointer or row stride is not 16-byte aligned";
        case FDL_ERR_WORKSPACE: return "workspace missing or too small";
        case FDL_ERR_HIP: return "a HIP kernel launch failed";
        case FDL_ERR_UNSUPPORTED: return "unsupported configuration";
    }
    return "unknown status";
}

int fdl_focus_count(int n_t, double rho) {
    if (!(rho >= 0.0) || n_t < 0) return 0;
    const double k = std::floor(rho * static_cast<double>(n_t));
    return k > 2147483647.0 ? 2147483647 : static_cast<int>(k);
}

fdl_status fdl_pcgi_select(const float* conf, const uint8_t* mask, int B, int L, int n_t, double rho,
                           int w, int32_t* focus_idx, int32_t* n_focus, int k_cap, int32_t* active_idx,
                           int32_t* n_active, int nq_max, hipStream_t stream) {
    if (!conf || !mask || !focus_idx || !n_focus || !active_idx || !n_active) return FDL_ERR_NULL;
    if (B < 1 || L < 1 || w < 1 || n_t < 0 || !(rho >= 0.0) || !std::isfinite(rho)) return FDL_ERR_SHAPE;
    const int k = fdl_focus_count(n_t, rho);
    if (k_cap < k || k_cap < 0) return FDL_ERR_SHAPE;
    const int64_t need = static_cast<int64_t>(k) * w < L ? static_cast<int64_t>(k) * w : L;
    if (nq_max < need) return FDL_ERR_SHAPE;
    return hip_status(launch_pcgi_select(conf, mask, B, L, k, w, focus_idx, n_focus, k_cap, active_idx,
                                         n_active, nq_max, stream));
}

size_t fdl_dense_attention_workspace_bytes(fdl_dtype dt, int B, int Hq, int Hkv, int L, int d,
                                           int nq_max) {
    if (check_dtype_dims(dt, B, Hq, Hkv, L, d) != FDL_OK || nq_max < 1) return 0;
    return plan_attention(dt, B, Hq, Hkv, d, nq_max, L, false).ws_bytes;
}

fdl_status fdl_dense_attention(fdl_dtype dt, int B, int Hq, int Hkv, int L, int d, const void* q,
                               fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                               const void* k, fdl_strides ks, const void* v, fdl_strides vs,
                               const void* vt, fdl_strides vts, float scale, void* o, fdl_strides os,
                               float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hq, Hkv, L, d);
    if (st != FDL_OK) return st;
    if ((st = check_rows(nq_max, Hq / Hkv)) != FDL_OK) return st;
    if ((st = check_tensor(q, qs, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(v, vs, dt, d)) != FDL_OK) return st;
    if ((st = check_vt(vt, vts, dt, d, L)) != FDL_OK) return st;
    if ((st = check_tensor(o, os, dt, d)) != FDL_OK) return st;
    if (nq_max == 0) return FDL_OK;
    const AttnPlan pl = plan_attention(dt, B, Hq, Hkv, d, nq_max, L, false);
    if ((st = check_ws(ws, ws_bytes, pl.ws_bytes)) != FDL_OK) return st;
    AttnArgs a = attn_args(dt, B, Hq, Hkv, L, L, q, qs, q_idx, n_q, nq_max, k, ks, v, vs, vt, vts, scale, d,
                           o, os, lse, ws);
    a.sparse = 0;
    return hip_status(launch_attention(dt, d, a, pl, stream));
}

size_t fdl_sink_identify_workspace_bytes(fdl_dtype dt, int B, int Hq, int Hkv, int L, int d, int nq_max) {
    if (check_dtype_dims(dt, B, Hq, Hkv, L, d) != FDL_OK || nq_max < 0) return 0;
    return sink_ws_layout(dt, B, Hq, Hkv, L, d, nq_max).total;
}

fdl_status fdl_sink_identify(fdl_dtype dt, int B, int Hq, int Hkv, int L, int d, const void* q,
                             fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                             const void* k, fdl_strides ks, float scale, const float* lse, int n_sinks,
                             int32_t* sink_idx, float* scores, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hq, Hkv, L, d);
    if (st != FDL_OK) return st;
    if ((st = check_rows(nq_max, Hq / Hkv)) != FDL_OK) return st;
    if ((st = check_tensor(q, qs, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if (!sink_idx) return FDL_ERR_NULL;
    if (n_sinks < 0 || n_sinks > L) return FDL_ERR_SHAPE;
    const SinkWs w = sink_ws_layout(dt, B, Hq, Hkv, L, d, nq_max);
    if ((st = check_ws(ws, ws_bytes, lse ? w.sink : w.total)) != FDL_OK) return st;
    if (!lse && nq_max > 0) {
        // the log-sum-exp of the same rows over all L keys, from a dense pass whose outputs are
        // discarded (the values do not enter the lse, so the keys serve as values)
        uint8_t* base = static_cast<uint8_t*>(ws);
        float* lse_ws = reinterpret_cast<float*>(base + w.sink);
        void* o_ws = base + w.sink + w.lse;
        const fdl_strides os = {static_cast<int64_t>(Hq) * nq_max * d, static_cast<int64_t>(nq_max) * d, d};
        const fdl_strides none = {0, 0, 0};
        AttnArgs a = attn_args(dt, B, Hq, Hkv, L, L, q, qs, q_idx, n_q, nq_max, k, ks, k, ks, nullptr, none, scale,
                               d, o_ws, os, lse_ws, base + w.sink + w.lse + w.out);
        a.sparse = 0;
        const AttnPlan pl = plan_attention(dt, B, Hq, Hkv, d, nq_max, L, false);
        if ((st = hip_status(launch_attention(dt, d, a, pl, stream))) != FDL_OK) return st;
        lse = lse_ws;
    }
    SinkArgs a{};
    a.q = q; a.qsb = qs.b; a.qsh = qs.h; a.qsr = qs.r;
    a.q_idx = q_idx; a.n_q = n_q; a.nq_max = nq_max;
    a.k = k; a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.lse = lse;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.L = L; a.Gq = Hq / Hkv;
    a.sl2 = resolve_scale(scale, d) * kLog2eF;
    return hip_status(launch_sink_identify(dt, d, a, n_sinks, sink_idx, scores, ws, stream));
}

fdl_status fdl_block_means(fdl_dtype dt, int B, int Hkv, int L, int P, int d, const void* k, fdl_strides ks,
                           int bs, float* kbar, hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hkv, Hkv, L, d);
    if (st != FDL_OK) return st;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if (!kbar) return FDL_ERR_NULL;
    if (!aligned16(kbar)) return FDL_ERR_ALIGN;
    if (P < 1 || P > L || bs < 1) return FDL_ERR_SHAPE;
    BlockArgs a{};
    a.k = k; a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.B = B; a.Hq = Hkv; a.Hkv = Hkv; a.P = P; a.Gq = 1; a.bs = bs;
    a.nb = static_cast<int>((static_cast<int64_t>(P) + bs - 1) / bs);
    a.kbar = kbar;
    return hip_status(launch_block_means(dt, d, a, stream));
}

size_t fdl_block_score_topc_workspace_bytes(fdl_dtype dt, int B, int Hq, int Hkv, int P, int d, int bs,
                                            int nq_max) {
    if (check_dtype_dims(dt, B, Hq, Hkv, P < 1 ? 1 : P, d) != FDL_OK || P < 1 || bs < 1 || nq_max < 0)
        return 0;
    return block_workspace_bytes(B, Hq, Hkv, P, d, bs, nq_max);
}

fdl_status fdl_block_score_topc_ex(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d, const void* q,
                                   fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                                   const void* k, fdl_strides ks, float scale, int bs, int C, int mode,
                                   int32_t* block_idx, double* R, float* kbar, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hq, Hkv, L, d);
    if (st != FDL_OK) return st;
    if ((st = check_rows(nq_max, Hq / Hkv)) != FDL_OK) return st;
    if ((st = check_tensor(q, qs, dt, d)) != FDL_OK) return st;
    if (k && (st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if (!k && !kbar) return FDL_ERR_NULL;
    if (!block_idx) return FDL_ERR_NULL;
    if (kbar && !aligned16(kbar)) return FDL_ERR_ALIGN;
    if (P < 1 || P > L || bs < 1 || C < 0) return FDL_ERR_SHAPE;
    if (mode < 0 || mode > (FDL_SCORE_PER_HEAD | FDL_SCORE_MAX)) return FDL_ERR_SHAPE;
    if ((st = check_ws(ws, ws_bytes, block_workspace_bytes(B, Hq, Hkv, P, d, bs, nq_max))) != FDL_OK) return st;
    BlockArgs a{};
    a.q = q; a.qsb = qs.b; a.qsh = qs.h; a.qsr = qs.r;
    a.q_idx = q_idx; a.n_q = n_q; a.nq_max = nq_max;
    a.k = k; a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.P = P; a.Gq = Hq / Hkv; a.bs = bs;
    a.nb = static_cast<int>((static_cast<int64_t>(P) + bs - 1) / bs);
    a.scale = resolve_scale(scale, d);
    a.kbar = kbar;
    a.mode = (mode & FDL_SCORE_PER_HEAD ? kScorePerHead : 0) | (mode & FDL_SCORE_MAX ? kScoreMax : 0);
    return hip_status(launch_block_score_topc(dt, d, a, C, block_idx, R, ws, stream));
}

fdl_status fdl_block_score_topc(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d, const void* q,
                                fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                                const void* k, fdl_strides ks, float scale, int bs, int C,
                                int32_t* block_idx, double* R, float* kbar, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
    return fdl_block_score_topc_ex(dt, B, Hq, Hkv, L, P, d, q, qs, q_idx, n_q, nq_max, k, ks, scale, bs, C,
                                   FDL_SCORE_SUM, block_idx, R, kbar, ws, ws_bytes, stream);
}

size_t fdl_sparse_attention_ex_workspace_bytes(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d,
                                               int nq_max, int n_sinks, int C, int bs, int blocks_per_head) {
    if (check_dtype_dims(dt, B, Hq, Hkv, L, d) != FDL_OK || nq_max < 1 || bs < 1 || P < 0 || P > L ||
        C < 0 || n_sinks < 0 || (blocks_per_head != 0 && blocks_per_head != 1))
        return 0;
    return plan_attention(dt, B, Hq, Hkv, d, nq_max, sparse_key_bound(L, P, n_sinks, C, bs), true,
                          blocks_per_head != 0).ws_bytes;
}

size_t fdl_sparse_attention_workspace_bytes(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d,
                                            int nq_max, int n_sinks, int C, int bs) {
    return fdl_sparse_attention_ex_workspace_bytes(dt, B, Hq, Hkv, L, P, d, nq_max, n_sinks, C, bs, 0);
}

fdl_status fdl_sparse_attention_ex(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d, const void* q,
                                   fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                                   const void* k, fdl_strides ks, const void* v, fdl_strides vs,
                                   const void* vt, fdl_strides vts,
                                   const int32_t* sink_idx, int n_sinks, const int32_t* block_idx, int C,
                                   int blocks_per_head, int bs, float scale, void* o, fdl_strides os, float* lse,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hq, Hkv, L, d);
    if (st != FDL_OK) return st;
    if ((st = check_rows(nq_max, Hq / Hkv)) != FDL_OK) return st;
    if ((st = check_tensor(q, qs, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(v, vs, dt, d)) != FDL_OK) return st;
    if ((st = check_vt(vt, vts, dt, d, L)) != FDL_OK) return st;
    if ((st = check_tensor(o, os, dt, d)) != FDL_OK) return st;
    if (P < 0 || P > L || bs < 1 || C < 0 || n_sinks < 0) return FDL_ERR_SHAPE;
    if (blocks_per_head != 0 && blocks_per_head != 1) return FDL_ERR_SHAPE;
    if ((n_sinks > 0 && !sink_idx) || (C > 0 && !block_idx)) return FDL_ERR_NULL;
    if (C > kPrepMaxIds || n_sinks > kPrepMaxIds) return FDL_ERR_UNSUPPORTED;
    const int64_t bound = sparse_key_bound(L, P, n_sinks, C, bs);
    if (bound > (1ll << 30)) return FDL_ERR_SHAPE;
    if (nq_max == 0) return FDL_OK;
    const AttnPlan pl = plan_attention(dt, B, Hq, Hkv, d, nq_max, bound, true, blocks_per_head != 0);
    if ((st = check_ws(ws, ws_bytes, pl.ws_bytes)) != FDL_OK) return st;
    AttnArgs a = attn_args(dt, B, Hq, Hkv, L, P, q, qs, q_idx, n_q, nq_max, k, ks, v, vs, vt, vts, scale, d,
                           o, os, lse, ws);
    a.sparse = 1;
    a.sink_idx = sink_idx;
    a.n_sinks = n_sinks;
    a.block_idx = block_idx;
    a.C = C;
    a.blk_per_head = blocks_per_head;
    a.bs = bs;
    a.nb = static_cast<int>((static_cast<int64_t>(P) + bs - 1) / bs);
    return hip_status(launch_attention(dt, d, a, pl, stream));
}

fdl_status fdl_sparse_attention(fdl_dtype dt, int B, int Hq, int Hkv, int L, int P, int d, const void* q,
                                fdl_strides qs, const int32_t* q_idx, const int32_t* n_q, int nq_max,
                                const void* k, fdl_strides ks, const void* v, fdl_strides vs,
                                const void* vt, fdl_strides vts,
                                const int32_t* sink_idx, int n_sinks, const int32_t* block_idx, int C,
                                int bs, float scale, void* o, fdl_strides os, float* lse, void* ws,
                                size_t ws_bytes, hipStream_t stream) {
    return fdl_sparse_attention_ex(dt, B, Hq, Hkv, L, P, d, q, qs, q_idx, n_q, nq_max, k, ks, v, vs, vt, vts,
                                   sink_idx, n_sinks, block_idx, C, 0, bs, scale, o, os, lse, ws, ws_bytes, stream);
}

fdl_status fdl_kv_refresh(fdl_dtype dt, int B, int Hkv, int L, int d, const int32_t* rows,
                          const int32_t* n_rows, int n_max, const void* k_new, fdl_strides kns,
                          const void* v_new, fdl_strides vns, void* k, fdl_strides ks, void* v,
                          fdl_strides vs, void* vt, fdl_strides vts, hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hkv, Hkv, L, d);
    if (st != FDL_OK) return st;
    if (n_max < 0) return FDL_ERR_SHAPE;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(v, vs, dt, d)) != FDL_OK) return st;
    if ((st = check_vt(vt, vts, dt, d, L)) != FDL_OK) return st;
    if (vt && (vts.r < L || vts.r >= (1ll << 31))) return FDL_ERR_SHAPE;
    if (n_max == 0) return FDL_OK;
    if (!rows) return FDL_ERR_NULL;
    if ((st = check_tensor(k_new, kns, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(v_new, vns, dt, d)) != FDL_OK) return st;
    CacheArgs a{};
    a.B = B; a.Hkv = Hkv; a.L = L; a.P = L; a.d = d; a.n_max = n_max;
    a.rows = rows; a.n_rows = n_rows;
    a.k_new = k_new; a.knb = kns.b; a.knh = kns.h; a.knr = kns.r;
    a.v_new = v_new; a.vnb = vns.b; a.vnh = vns.h; a.vnr = vns.r;
    a.k = k; a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.v = v; a.vsb = vs.b; a.vsh = vs.h; a.vsr = vs.r;
    a.vt = vt; a.vtsb = vts.b; a.vtsh = vts.h; a.vtsd = vts.r;
    return hip_status(launch_kv_scatter(dt, a, stream));
}

fdl_status fdl_block_means_refresh(fdl_dtype dt, int B, int Hkv, int L, int P, int d, const void* k,
                                   fdl_strides ks, int bs, const int32_t* rows, const int32_t* n_rows,
                                   int n_max, float* kbar, hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hkv, Hkv, L, d);
    if (st != FDL_OK) return st;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if (P < 1 || P > L || bs < 1 || n_max < 0) return FDL_ERR_SHAPE;
    if (!kbar) return FDL_ERR_NULL;
    if (!aligned16(kbar)) return FDL_ERR_ALIGN;
    if (n_max == 0) return FDL_OK;
    if (!rows) return FDL_ERR_NULL;
    CacheArgs a{};
    a.B = B; a.Hkv = Hkv; a.L = L; a.P = P; a.d = d; a.bs = bs; a.n_max = n_max;
    a.nb = static_cast<int>((static_cast<int64_t>(P) + bs - 1) / bs);
    a.rows = rows; a.n_rows = n_rows;
    a.k = const_cast<void*>(k); a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.kbar = kbar;
    return hip_status(launch_block_means_refresh(dt, a, stream));
}

fdl_status fdl_kv_refresh_means(fdl_dtype dt, int B, int Hkv, int L, int P, int d, int bs, const int32_t* rows,
                                const int32_t* n_rows, int n_max, const void* k_new, fdl_strides kns,
                                const void* v_new, fdl_strides vns, void* k, fdl_strides ks, void* v,
                                fdl_strides vs, void* vt, fdl_strides vts, float* kbar, hipStream_t stream) {
    fdl_status st = check_dtype_dims(dt, B, Hkv, Hkv, L, d);
    if (st != FDL_OK) return st;
    if (n_max < 0 || P < 1 || P > L || bs < 1) return FDL_ERR_SHAPE;
    if (bs > kFusedMaxBs) return FDL_ERR_UNSUPPORTED;
    if ((st = check_tensor(k, ks, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(v, vs, dt, d)) != FDL_OK) return st;
    if ((st = check_vt(vt, vts, dt, d, L)) != FDL_OK) return st;
    if (vt && (vts.r < L || vts.r >= (1ll << 31))) return FDL_ERR_SHAPE;
    if (!kbar) return FDL_ERR_NULL;
    if (!aligned16(kbar)) return FDL_ERR_ALIGN;
    if (n_max == 0) return FDL_OK;
    if (!rows) return FDL_ERR_NULL;
    if ((st = check_tensor(k_new, kns, dt, d)) != FDL_OK) return st;
    if ((st = check_tensor(v_new, vns, dt, d)) != FDL_OK) return st;
    CacheArgs a{};
    a.B = B; a.Hkv = Hkv; a.L = L; a.P = P; a.d = d; a.bs = bs; a.n_max = n_max;
    a.nb = static_cast<int>((static_cast<int64_t>(P) + bs - 1) / bs);
    a.rows = rows; a.n_rows = n_rows;
    a.k_new = k_new; a.knb = kns.b; a.knh = kns.h; a.knr = kns.r;
    a.v_new = v_new; a.vnb = vns.b; a.vnh = vns.h; a.vnr = vns.r;
    a.k = k; a.ksb = ks.b; a.ksh = ks.h; a.ksr = ks.r;
    a.v = v; a.vsb = vs.b; a.vsh = vs.h; a.vsr = vs.r;
    a.vt = vt; a.vtsb = vts.b; a.vtsh = vts.h; a.vtsd = vts.r;
    a.kbar = kbar;
    return hip_status(launch_kv_refresh_means(dt, a, stream));
}

size_t fdl_confidence_unmask_workspace_bytes(int B, int V, int m_max) {
    if (B < 1 || V < 1 || m_max < 0 || m_max > kMaxConfRows) return 0;
    return confidence_workspace_bytes(B, V, m_max);
}

fdl_status fdl_confidence_unmask(fdl_dtype dt, int B, int L, int V, const void* logits, fdl_strides ls,
                                 const int32_t* pos, const int32_t* n_rows, int m_max, int n_t, uint8_t* mask,
                                 float* conf, int32_t* tokens, int32_t* unmasked, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
    if (dt != FDL_F32 && dt != FDL_BF16) return FDL_ERR_DTYPE;
    if (B < 1 || L < 1 || V < 1 || m_max < 0 || n_t < 0) return FDL_ERR_SHAPE;
    if (m_max > kMaxConfRows) return FDL_ERR_UNSUPPORTED;
    if (!mask || !conf) return FDL_ERR_NULL;
    if (m_max == 0) return FDL_OK;
    if (!logits || !pos) return FDL_ERR_NULL;
    const int64_t e = static_cast<int64_t>(elem_size(dt));
    if (!aligned16(logits) || (ls.b * e) % 16 || (ls.r * e) % 16) return FDL_ERR_ALIGN;
    if (ls.r < V || ls.r >= (1ll << 40)) return FDL_ERR_SHAPE;
    fdl_status st;
    if ((st = check_ws(ws, ws_bytes, confidence_workspace_bytes(B, V, m_max))) != FDL_OK) return st;
    return hip_status(launch_confidence_unmask(dt, B, L, V, logits, ls.b, ls.r, pos, n_rows, m_max, n_t, mask, conf,
                                               tokens, unmasked, ws, stream));
}

size_t fdl_dcu_select_workspace_bytes(int B, int NL, int L) {
    if (B < 1 || NL < 1 || L < 1) return 0;
    return dcu_workspace_bytes(B, NL, L);
}

fdl_status fdl_dcu_select(fdl_dtype dt, int B, int NL, int L, int H, const void* x_now, fdl_strides xns,
                          const void* x_prev, fdl_strides xps, const int32_t* key_tokens, int n_keys, int w_m,
                          int total, float* dist, double* activity, int32_t* budgets, int32_t* upd_idx,
                          int32_t* n_upd, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (dt != FDL_F32 && dt != FDL_BF16) return FDL_ERR_DTYPE;
    if (B < 1 || NL < 1 || L < 1 || H < 1 || n_keys < 0 || total < 0) return FDL_ERR_SHAPE;
    if (n_keys > 0 && w_m < 1) return FDL_ERR_SHAPE;
    if (L > kDcuMaxTokens || NL > kDcuMaxLayers) return FDL_ERR_UNSUPPORTED;
    if (static_cast<int64_t>(B) * NL * dcu_chunks(L) >= (1ll << 31)) return FDL_ERR_SHAPE;
    if (!x_now || !x_prev || !dist || !activity || !budgets || !upd_idx || !n_upd) return FDL_ERR_NULL;
    if (n_keys > 0 && !key_tokens) return FDL_ERR_NULL;
    const int64_t e = static_cast<int64_t>(elem_size(dt));
    for (const fdl_strides& s : {xns, xps}) {
        if ((s.b * e) % 16 || (s.h * e) % 16 || (s.r * e) % 16) return FDL_ERR_ALIGN;
        for (int64_t v : {s.b, s.h, s.r})
            if (v <= -(1ll << 40) || v >= (1ll << 40)) return FDL_ERR_SHAPE;
    }
    if (!aligned16(x_now) || !aligned16(x_prev)) return FDL_ERR_ALIGN;
    fdl_status st;
    if ((st = check_ws(ws, ws_bytes, dcu_workspace_bytes(B, NL, L))) != FDL_OK) return st;
    DcuArgs a{};
    a.B = B; a.NL = NL; a.L = L; a.H = H;
    a.x_now = x_now; a.xnb = xns.b; a.xnl = xns.h; a.xnr = xns.r;
    a.x_prev = x_prev; a.xpb = xps.b; a.xpl = xps.h; a.xpr = xps.r;
    a.keys = key_tokens; a.n_keys = n_keys; a.w_m = w_m; a.total = total;
    a.dist = dist; a.activity = activity; a.budgets = budgets; a.upd_idx = upd_idx; a.n_upd = n_upd;
    a.ws = ws;
    return hip_status(launch_dcu_select(dt, a, stream));
}

fdl_status fdl_calibrate_read(const void* src, size_t bytes, uint32_t* sink, int workgroups, hipStream_t stream) {
    if (bytes == 0 || bytes % 16 || workgroups < 1) return FDL_ERR_SHAPE;
    if (!src || !sink) return FDL_ERR_NULL;
    if (!aligned16(src)) return FDL_ERR_ALIGN;
    return hip_status(launch_calib_read(src, bytes, sink, workgroups, stream));
}

fdl_status fdl_calibrate_mfma(int workgroups, int iters, float a_val, float b_val, float* sink, hipStream_t stream) {
    if (workgroups < 1 || iters < 1) return FDL_ERR_SHAPE;
    if (!sink) return FDL_ERR_NULL;
    return hip_status(launch_calib_mfma(workgroups, iters, a_val, b_val, sink, stream));
}

}  // extern "C"
