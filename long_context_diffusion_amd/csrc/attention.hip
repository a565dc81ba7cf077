// Bidirectional attention of selected query rows over a dense or sparse key set.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
// steps": dense attention at the block-entry refresh and in layers 1..l_dense
// (step (3)); sparse attention over I_p = sinks U selected prompt blocks U the
// generation region (step (5)).  softmax(q k^T * scale) v with no mask.
//
// bf16 path (gfx950 MFMA, v_mfma_f32_32x32x16_bf16), per workgroup of 4 waves:
//   * 128 query rows of one KV head.  Query heads sharing the KV head are
//     interleaved into the rows (packed row p -> head g*Gq + p % Gq, logical
//     row p / Gq), so grouped-query heads reuse every K/V tile.
//   * Each wave owns 32 rows and computes S^T = K Q^T (keys on the MFMA M
//     axis), so a lane holds one query's scores: the running max/sum and the
//     rescale of the output are per-lane scalars, with one cross-half swap per
//     tile for the max.
//   * O^T = V^T P^T: V is transposed while it is staged into LDS so the MFMA
//     A operand is two 8-byte LDS reads; the key order inside a 16-key MFMA
//     chunk follows the accumulator layout of S^T, so P needs no shuffle.
//   * 64-key tiles of K and V^T are double-buffered in LDS (68 KB), with one
//     barrier per tile; global loads for tile t+1 are in flight while tile t
//     is computed.  Rows of LDS are padded so MFMA operand reads are
//     bank-conflict free.
//   * Small query sets (the active rows of a sparse step) split the key range
//     over several workgroups; attn_merge combines the partial results with
//     their running max and sum.
// Sparse key sets are never materialised: key position t of I_p maps to the
// (t / bs)-th selected block, the generation region or the sink list, and a
// sink already covered by a selected block or by [P, L) is masked out, so each
// key is attended once.
//
// fp32 path: the same decomposition on the vector ALU (one wave, one row per
// lane, 32-key tiles in LDS), for fp32 inputs.

#include "attention.cuh"

namespace fdl {

namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegBig = -1.0e30f;   // running-max start: finite, so exp2 of differences never sees inf-inf
constexpr int kMaxSinkWords = 128;    // n_sinks <= 4096

// Positions of I_p for one sequence: [0, n_blk) selected blocks, [n_blk, sink0)
// the generation region, [sink0, n_keys) the sink list (some entries masked).
struct KeyMap {
    int n_blk, sink0, n_keys;
};

// Builds the key map of sequence b and the per-sink "attend" bits in LDS.
__device__ KeyMap build_key_map(const AttnArgs& a, int b, uint32_t* s_sink_ok, int* s_tmp) {
    KeyMap km;
    if (!a.sparse) {
        km.n_blk = 0;
        km.sink0 = a.L;
        km.n_keys = a.L;
        return km;
    }
    const int32_t* blk = a.block_idx + static_cast<int64_t>(b) * a.C;
    int cnt = 0;
    for (int c = threadIdx.x; c < a.C; c += blockDim.x) cnt += blk[c] >= 0 ? 1 : 0;
    int n_sel;
    block_exclusive_sum(cnt, s_tmp, &n_sel);
    int n_blk = n_sel * a.bs;
    if (n_sel > 0 && blk[n_sel - 1] == a.nb - 1) n_blk -= a.nb * a.bs - a.P;  // short last block
    for (int i = threadIdx.x; i < kMaxSinkWords; i += blockDim.x) s_sink_ok[i] = 0;
    __syncthreads();
    const int32_t* snk = a.sink_idx + static_cast<int64_t>(b) * a.n_sinks;
    for (int s = threadIdx.x; s < a.n_sinks; s += blockDim.x) {
        const int j = snk[s];
        bool attend = j >= 0 && j < a.P;
        if (attend) {  // covered by a selected block?  (blocks ascending)
            const int target = j / a.bs;
            int lo = 0, hi = n_sel;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (blk[mid] < target) lo = mid + 1; else hi = mid;
            }
            if (lo < n_sel && blk[lo] == target) attend = false;
        }
        if (attend) atomicOr(&s_sink_ok[s >> 5], 1u << (s & 31));
    }
    __syncthreads();
    km.n_blk = n_blk;
    km.sink0 = n_blk + (a.L - a.P);
    km.n_keys = km.sink0 + a.n_sinks;
    return km;
}

// Key index of position t of the key set; *ok is false for masked or out-of-range positions.
__device__ __forceinline__ int key_at(const AttnArgs& a, const KeyMap& km, int b, int t,
                                      const uint32_t* s_sink_ok, bool* ok) {
    if (!a.sparse) {
        *ok = t < a.L;
        return *ok ? t : 0;
    }
    if (t < km.n_blk) {
        const int c = t / a.bs;
        *ok = true;
        return a.block_idx[static_cast<int64_t>(b) * a.C + c] * a.bs + (t - c * a.bs);
    }
    if (t < km.sink0) {
        *ok = true;
        return a.P + (t - km.n_blk);
    }
    if (t < km.n_keys) {
        const int s = t - km.sink0;
        *ok = (s_sink_ok[s >> 5] >> (s & 31)) & 1u;
        return *ok ? a.sink_idx[static_cast<int64_t>(b) * a.n_sinks + s] : 0;
    }
    *ok = false;
    return 0;
}

__device__ __forceinline__ bool key_attended(const AttnArgs& a, const KeyMap& km, int t,
                                             const uint32_t* s_sink_ok) {
    if (t >= km.n_keys) return false;
    if (!a.sparse || t < km.sink0) return true;
    const int s = t - km.sink0;
    return (s_sink_ok[s >> 5] >> (s & 31)) & 1u;
}

// Decodes the 1-D grid: q-tile fastest, then split, then KV head, then sequence.
struct WorkUnit {
    int qt, split, g, b;
};
__device__ __forceinline__ WorkUnit decode_unit(const AttnArgs& a) {
    WorkUnit u;
    int id = blockIdx.x;
    u.qt = id % a.q_tiles;
    id /= a.q_tiles;
    u.split = id % a.n_splits;
    id /= a.n_splits;
    u.g = id % a.Hkv;
    u.b = id / a.Hkv;
    return u;
}

template <typename T>
__device__ __forceinline__ void write_zero_row(const AttnArgs& a, int b, int h, int r, int d) {
    T* orow = static_cast<T*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr;
    for (int e = 0; e < d; ++e) orow[e] = T(0);
    if (a.lse) a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] = -INFINITY;
}

// ------------------------------------------------------------------ bf16 MFMA kernel

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(const AttnArgs a) {
    constexpr int NCH = D / 8;               // 16-byte chunks per row
    constexpr int KP = D * 2 + 16;           // K row pitch in LDS (bytes)
    constexpr int VP = 64 * 2 + 8;           // V^T row pitch in LDS (bytes)
    constexpr int KBUF = 64 * KP;
    constexpr int VBUF = D * VP;
    constexpr int STAGE = KBUF + VBUF;
    constexpr int KPT = 64 * NCH / 256;      // K chunks staged per thread
    constexpr int VPT = 32 * NCH / 256;      // V (key pair, chunk) items per thread
    constexpr int KROWS = 256 / NCH;         // K rows covered by one pass of the block
    constexpr int NDB = D / 32;              // 32-wide d blocks of the output
    constexpr int NQC = D / 16;              // 16-wide d chunks of Q . K
    static_assert(KPT >= 1 && VPT >= 1, "head dim");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];
    __shared__ uint32_t s_sink_ok[kMaxSinkWords];
    __shared__ int s_tmp[17];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int hf = lane >> 5;
    const int col = lane & 31;
    const WorkUnit u = decode_unit(a);
    const int b = u.b, g = u.g;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows_valid = a.Gq * nq;
    const int rows_all = a.Gq * a.nq_max;
    const int p0 = u.qt * 128;
    const int p = p0 + wv * 32 + col;       // this lane's packed query row
    const bool row_ok = p < rows_valid;
    const int h = g * a.Gq + p % a.Gq;
    const int r = p / a.Gq;

    if (p0 >= rows_valid) {  // whole tile is padding
        if (a.n_splits == 1 && hf == 0 && p < rows_all) write_zero_row<uint16_t>(a, b, h, r, D);
        return;
    }

    const KeyMap km = build_key_map(a, b, s_sink_ok, s_tmp);
    const int n_tiles = (km.n_keys + 63) / 64;
    const int t_begin = u.split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);

    // Q fragments (B operand of S^T = K Q^T): lane holds row p, d = 16c + 8hf .. +7
    bf16x8 qf[NQC];
    {
        const uint16_t* qrow = nullptr;
        if (row_ok) {
            const int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + r] : r;
            qrow = static_cast<const uint16_t*>(a.q) + b * a.qsb + h * a.qsh +
                   static_cast<int64_t>(phys) * a.qsr;
        }
#pragma unroll
        for (int c = 0; c < NQC; ++c) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (row_ok) x = *reinterpret_cast<const u32x4*>(qrow + 16 * c + 8 * hf);
            qf[c] = __builtin_bit_cast(bf16x8, x);
        }
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + g * a.ksh;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.vsb + g * a.vsh;

    u32x4 kreg[KPT];
    u32x4 vreg[VPT][2];
    auto load_tile = [&](int t) {
        const int base = t * 64;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int row = i * KROWS + tid / NCH;
            const int ch = tid % NCH;
            bool ok;
            const int key = key_at(a, km, b, base + row, s_sink_ok, &ok);
            u32x4 x = {0u, 0u, 0u, 0u};
            if (ok) x = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * a.ksr + ch * 8);
            kreg[i] = x;
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int pr = tid & 31;
            const int ch = (tid >> 5) + 8 * i;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                bool ok;
                const int key = key_at(a, km, b, base + 2 * pr + e, s_sink_ok, &ok);
                u32x4 x = {0u, 0u, 0u, 0u};
                if (ok) x = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(key) * a.vsr + ch * 8);
                vreg[i][e] = x;
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint8_t* kb = smem + buf * STAGE;
        uint8_t* vb = kb + KBUF;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int row = i * KROWS + tid / NCH;
            const int ch = tid % NCH;
            *reinterpret_cast<u32x4*>(kb + row * KP + ch * 16) = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int pr = tid & 31;
            const int ch = (tid >> 5) + 8 * i;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                const uint32_t w0 = vreg[i][0][e2];   // key 2pr:   d = 8ch + 2e2, +1
                const uint32_t w1 = vreg[i][1][e2];   // key 2pr+1: d = 8ch + 2e2, +1
                const uint32_t even = (w0 & 0xffffu) | (w1 << 16);
                const uint32_t odd = (w0 >> 16) | (w1 & 0xffff0000u);
                *reinterpret_cast<uint32_t*>(vb + (8 * ch + 2 * e2) * VP + pr * 4) = even;
                *reinterpret_cast<uint32_t*>(vb + (8 * ch + 2 * e2 + 1) * VP + pr * 4) = odd;
            }
        }
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
    float m_run = kNegBig;
    float l_run = 0.0f;

    if (t_begin < t_end) {
        load_tile(t_begin);
        store_tile(0);
    }
    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        __syncthreads();
        if (t + 1 < t_end) load_tile(t + 1);
        const uint8_t* kb = smem + buf * STAGE;
        const uint8_t* vb = kb + KBUF;

        // S^T = K Q^T for two 32-key blocks
        f32x16 st[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int i = 0; i < 16; ++i) st[kb2][i] = 0.0f;
            const uint8_t* krow = kb + (kb2 * 32 + col) * KP + 16 * hf;
#pragma unroll
            for (int c = 0; c < NQC; ++c) {
                const bf16x8 ak = *reinterpret_cast<const bf16x8*>(krow + 32 * c);
                st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[c], st[kb2], 0, 0, 0);
            }
        }
        const int base = t * 64;
        const bool full = base + 64 <= km.sink0 && base + 64 <= km.n_keys;
        if (!full) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kl = kb2 * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (!key_attended(a, km, base + kl, s_sink_ok)) st[kb2][i] = -INFINITY;
                }
        }
        // online softmax (log2 domain), one query per lane pair
        float mx = st[0][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, st[0][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[1][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float m_new = fmaxf(m_run, mx * a.sl2);
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.0f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = exp2f(fmaf(st[kb2][i], a.sl2, -m_new));
                st[kb2][i] = pv;
                psum += pv;
            }
        l_run = fmaf(l_run, alpha, psum);
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;

        // O^T += V^T P^T, four 16-key chunks
        bf16x8 pf[4];
#pragma unroll
        for (int kc = 0; kc < 4; ++kc)
#pragma unroll
            for (int j = 0; j < 8; ++j) pf[kc][j] = static_cast<__bf16>(st[kc >> 1][8 * (kc & 1) + j]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const uint8_t* vrow = vb + (db * 32 + col) * VP + 8 * hf;
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                const u32x2 x0 = *reinterpret_cast<const u32x2*>(vrow + 32 * kc);
                const u32x2 x1 = *reinterpret_cast<const u32x2*>(vrow + 32 * kc + 16);
                const u32x4 x = {x0[0], x0[1], x1[0], x1[1]};
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, x),
                                                                  pf[kc], acc[db], 0, 0, 0);
            }
        }
        if (t + 1 < t_end) store_tile(buf ^ 1);
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (a.n_splits == 1) {
        if (row_ok) {
            uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.osb + h * a.osh +
                             static_cast<int64_t>(r) * a.osr;
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    const int d0 = db * 32 + 8 * qd + 4 * hf;
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[db][4 * qd + 0] * inv, acc[db][4 * qd + 1] * inv);
                    w[1] = pack_bf16x2(acc[db][4 * qd + 2] * inv, acc[db][4 * qd + 3] * inv);
                    *reinterpret_cast<u32x2*>(orow + d0) = w;
                }
            if (a.lse && hf == 0)
                a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] =
                    l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
        } else if (hf == 0 && p < rows_all) {
            write_zero_row<uint16_t>(a, b, h, r, D);
        }
    } else if (row_ok) {
        const int64_t idx = ((static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r) * a.n_splits + u.split;
        float* po = a.part_o + idx * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const int d0 = db * 32 + 8 * qd + 4 * hf;
                f32x4 w = {acc[db][4 * qd + 0], acc[db][4 * qd + 1], acc[db][4 * qd + 2], acc[db][4 * qd + 3]};
                *reinterpret_cast<f32x4*>(po + d0) = w;
            }
        if (hf == 0) {
            a.part_ml[idx * 2 + 0] = m_run;
            a.part_ml[idx * 2 + 1] = l_tot;
        }
    }
}

// ------------------------------------------------------------------ fp32 kernel

constexpr int kF32Rows = 64;   // one wave, one query row per lane
constexpr int kF32Keys = 32;   // keys per LDS tile

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(16))) float s_k[kF32Keys][D];
    __shared__ __attribute__((aligned(16))) float s_v[kF32Keys][D];
    __shared__ uint32_t s_sink_ok[kMaxSinkWords];
    __shared__ int s_tmp[17];
    __shared__ int s_ok[kF32Keys];

    const int lane = threadIdx.x;
    const WorkUnit u = decode_unit(a);
    const int b = u.b, g = u.g;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows_valid = a.Gq * nq;
    const int rows_all = a.Gq * a.nq_max;
    const int p0 = u.qt * kF32Rows;
    const int p = p0 + lane;
    const bool row_ok = p < rows_valid;
    const int h = g * a.Gq + p % a.Gq;
    const int r = p / a.Gq;
    if (p0 >= rows_valid) {
        if (a.n_splits == 1 && p < rows_all) write_zero_row<float>(a, b, h, r, D);
        return;
    }
    const KeyMap km = build_key_map(a, b, s_sink_ok, s_tmp);
    const int n_tiles = (km.n_keys + kF32Keys - 1) / kF32Keys;
    const int t_begin = u.split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);

    float qv[D];
    float acc[D];
    {
        const float* qrow = nullptr;
        if (row_ok) {
            const int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + r] : r;
            qrow = static_cast<const float*>(a.q) + b * a.qsb + h * a.qsh + static_cast<int64_t>(phys) * a.qsr;
        }
#pragma unroll
        for (int e = 0; e < D; ++e) {
            qv[e] = row_ok ? qrow[e] : 0.0f;
            acc[e] = 0.0f;
        }
    }
    const float* kbase = static_cast<const float*>(a.k) + b * a.ksb + g * a.ksh;
    const float* vbase = static_cast<const float*>(a.v) + b * a.vsb + g * a.vsh;
    float m_run = kNegBig, l_run = 0.0f;

    for (int t = t_begin; t < t_end; ++t) {
        __syncthreads();
        if (lane < kF32Keys) {
            bool ok;
            key_at(a, km, b, t * kF32Keys + lane, s_sink_ok, &ok);
            s_ok[lane] = ok ? 1 : 0;
        }
        for (int i = lane; i < kF32Keys * D / 4; i += 64) {
            const int row = i / (D / 4);
            const int c4 = i % (D / 4);
            bool ok;
            const int key = key_at(a, km, b, t * kF32Keys + row, s_sink_ok, &ok);
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (ok) {
                kx = *reinterpret_cast<const f32x4*>(kbase + static_cast<int64_t>(key) * a.ksr + 4 * c4);
                vx = *reinterpret_cast<const f32x4*>(vbase + static_cast<int64_t>(key) * a.vsr + 4 * c4);
            }
            *reinterpret_cast<f32x4*>(&s_k[row][4 * c4]) = kx;
            *reinterpret_cast<f32x4*>(&s_v[row][4 * c4]) = vx;
        }
        __syncthreads();
#pragma unroll
        for (int j0 = 0; j0 < kF32Keys; j0 += 16) {
            float s[16];
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float dot = 0.0f;
#pragma unroll
                for (int e = 0; e < D; ++e) dot = fmaf(qv[e], s_k[j0 + j][e], dot);
                s[j] = s_ok[j0 + j] ? dot * a.sl2 : -INFINITY;
                mx = fmaxf(mx, s[j]);
            }
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const float pv = exp2f(s[j] - m_new);
                l_run += pv;
#pragma unroll
                for (int e = 0; e < D; ++e) acc[e] = fmaf(pv, s_v[j0 + j][e], acc[e]);
            }
            m_run = m_new;
        }
    }

    if (a.n_splits == 1) {
        if (row_ok) {
            float* orow = static_cast<float*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr;
            const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
#pragma unroll
            for (int e = 0; e < D; ++e) orow[e] = acc[e] * inv;
            if (a.lse)
                a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] =
                    l_run > 0.0f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
        } else if (p < rows_all) {
            write_zero_row<float>(a, b, h, r, D);
        }
    } else if (row_ok) {
        const int64_t idx = ((static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r) * a.n_splits + u.split;
#pragma unroll
        for (int e = 0; e < D; ++e) a.part_o[idx * D + e] = acc[e];
        a.part_ml[idx * 2 + 0] = m_run;
        a.part_ml[idx * 2 + 1] = l_run;
    }
}

// ------------------------------------------------------------------ split merge

// One workgroup per output row (b, h, r): O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <typename T>
__global__ __launch_bounds__(128) void attn_merge_kernel(const AttnArgs a, int d) {
    const int64_t row = blockIdx.x;
    const int r = static_cast<int>(row % a.nq_max);
    const int h = static_cast<int>((row / a.nq_max) % a.Hq);
    const int b = static_cast<int>(row / (static_cast<int64_t>(a.nq_max) * a.Hq));
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    T* orow = static_cast<T*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr;
    if (r >= nq) {
        for (int e = threadIdx.x; e < d; e += blockDim.x) orow[e] = T(0);
        if (a.lse && threadIdx.x == 0) a.lse[row] = -INFINITY;
        return;
    }
    const float* ml = a.part_ml + row * a.n_splits * 2;
    float M = kNegBig;
    for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, ml[2 * s]);
    float Lsum = 0.0f;
    for (int s = 0; s < a.n_splits; ++s) Lsum += ml[2 * s + 1] * exp2f(ml[2 * s] - M);
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    const float* po = a.part_o + row * a.n_splits * d;
    for (int e = threadIdx.x; e < d; e += blockDim.x) {
        float x = 0.0f;
        for (int s = 0; s < a.n_splits; ++s) x = fmaf(po[static_cast<int64_t>(s) * d + e], exp2f(ml[2 * s] - M), x);
        Elem<T>::store(orow + e, x * inv);
    }
    if (a.lse && threadIdx.x == 0) a.lse[row] = Lsum > 0.0f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

}  // namespace

AttnPlan plan_attention(fdl_dtype dtype, int B, int Hq, int Hkv, int d, int nq_max,
                        int64_t key_bound) {
    AttnPlan pl;
    const bool bf16 = dtype == FDL_BF16;
    pl.rows_per_tile = bf16 ? 128 : kF32Rows;
    pl.tile_keys = bf16 ? 64 : kF32Keys;
    const int64_t rows = static_cast<int64_t>(Hq / Hkv) * nq_max;
    pl.q_tiles = static_cast<int>((rows + pl.rows_per_tile - 1) / pl.rows_per_tile);
    const int64_t tiles = (key_bound + pl.tile_keys - 1) / pl.tile_keys;
    const int64_t units = static_cast<int64_t>(B) * Hkv * pl.q_tiles;
    const int64_t target = 1024;  // workgroups that keep 256 CUs busy
    const int64_t min_tiles = 8;  // keep each split long enough to amortise its merge
    int64_t splits = (target + units - 1) / units;
    const int64_t max_splits = tiles / min_tiles > 1 ? tiles / min_tiles : 1;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    pl.n_splits = static_cast<int>(splits);
    pl.tiles_per_split = static_cast<int>((tiles + splits - 1) / splits);
    if (pl.tiles_per_split < 1) pl.tiles_per_split = 1;
    pl.ws_bytes = 0;
    if (pl.n_splits > 1) {
        const int64_t nrows = static_cast<int64_t>(B) * Hq * nq_max * pl.n_splits;
        pl.ws_bytes = static_cast<size_t>(nrows) * (d + 2) * sizeof(float);
    }
    return pl;
}

hipError_t launch_attention(fdl_dtype dtype, int d, const AttnArgs& args_in, const AttnPlan& pl,
                            hipStream_t stream) {
    AttnArgs a = args_in;
    a.q_tiles = pl.q_tiles;
    a.n_splits = pl.n_splits;
    a.tiles_per_split = pl.tiles_per_split;
    const int64_t nrows = static_cast<int64_t>(a.B) * a.Hq * a.nq_max;
    if (pl.n_splits > 1) {
        a.part_o = static_cast<float*>(a.part_o);
        a.part_ml = a.part_o + nrows * pl.n_splits * d;
    }
    const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * pl.n_splits * pl.q_tiles));
    if (dtype == FDL_BF16) {
        if (d == 128) hipLaunchKernelGGL(attn_bf16_kernel<128>, grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL(attn_bf16_kernel<64>, grid, dim3(256), 0, stream, a);
    } else {
        if (d == 128) hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, a);
        else hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, a);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || pl.n_splits == 1) return err;
    const dim3 mgrid(static_cast<unsigned>(nrows));
    if (dtype == FDL_BF16) hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, mgrid, dim3(128), 0, stream, a, d);
    else hipLaunchKernelGGL(attn_merge_kernel<float>, mgrid, dim3(128), 0, stream, a, d);
    return hipGetLastError();
}

}  // namespace fdl
