// Bidirectional attention of selected query rows over a dense or sparse key set.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
// steps": dense attention at the block-entry refresh and in layers 1..l_dense
// (step (3)); sparse attention over I_p = sinks U selected prompt blocks U the
// generation region (step (5)).  softmax(q k^T * scale) v with no mask.
//
// attn_prep (one workgroup per sequence) writes the keys of I_p as a compact
// list (selected blocks, then [P, L), then the sinks that neither a selected
// block nor the generation region already holds).
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
//   * 64-key tiles of K and V^T are double-buffered in LDS (68 KB), one barrier
//     per tile; global loads of tile t+1 are in flight while tile t is
//     computed.  Sparse key indices come from the list two tiles ahead, through
//     LDS, so no load waits on another inside the loop.  LDS rows are padded so
//     MFMA operand reads are bank-conflict free.
//   * Small query sets (the active rows of a sparse step) split the key range
//     over several workgroups; attn_merge then combines the partial results
//     of every output row in split order (one wave per row).  A merge inside
//     the last-finishing split would need a device-scope release per
//     workgroup, which on gfx950 writes back the XCD's L2: far dearer than
//     one more launch.
//
// fp32 path: the same decomposition on the vector ALU (one wave, one row per
// lane, 32-key tiles in LDS), for fp32 inputs.

#include "attention.cuh"

namespace fdl {

namespace {


// ------------------------------------------------------------------ key list

constexpr int kPrepListWgs = 8;        // workgroups per sequence writing the key list

// grid (key lists, kPrepListWgs + padding workgroups), one key list per sequence or per
// (sequence, KV head).  y < kPrepListWgs: write a slice of the key list (y == 0 also
// appends the uncovered sinks and |I_p|); y >= kPrepListWgs: zero padding rows of the
// sequence when there is no key split (the workgroups of its first list only).  The block and sink lists are brought to
// canonical form first (valid ids, ascending, each once): at most kPrepMaxIds entries each.
template <typename T>
__global__ __launch_bounds__(256) void attn_prep_kernel(const AttnArgs a, int d, bool build_list) {
    __shared__ int s_tmp[17];
    __shared__ int s_blk[kPrepMaxIds];
    __shared__ int s_snk[kPrepMaxIds];
    __shared__ int s_scr[kPrepMaxIds];
    const int li = blockIdx.x;
    const int b = a.blk_per_head ? li / a.Hkv : li;
    const int tid = threadIdx.x;
    if (blockIdx.y >= kPrepListWgs) {
        if (a.blk_per_head && li % a.Hkv != 0) return;
        // padding rows r in [n_q[b], nq_max) of every query head: O = 0, lse = -inf
        // (only without a key split: the split merge writes them otherwise)
        if (!a.n_q || a.n_splits > 1) return;
        const int nq = a.n_q[b];
        const int64_t pad_rows = static_cast<int64_t>(a.Hq) * (a.nq_max - nq);
        const int c4n = d / 4;
        const int64_t items = pad_rows * c4n;
        const int64_t nwg = gridDim.y - kPrepListWgs;
        for (int64_t it = static_cast<int64_t>(blockIdx.y - kPrepListWgs) * blockDim.x + tid; it < items;
             it += nwg * blockDim.x) {
            const int64_t row = it / c4n;
            const int c4 = static_cast<int>(it % c4n);
            const int h = static_cast<int>(row / (a.nq_max - nq));
            const int r = nq + static_cast<int>(row % (a.nq_max - nq));
            T* orow = static_cast<T*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr + 4 * c4;
            for (int e = 0; e < 4; ++e) orow[e] = T(0);
            if (a.lse && c4 == 0) a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] = -INFINITY;
        }
        return;
    }
    if (!a.sparse || !build_list) return;
    const int n_sel = canonical_ids(a.block_idx + static_cast<int64_t>(li) * a.C, a.C, 0, a.nb, s_blk, s_scr, s_tmp);
    int n_blk = n_sel * a.bs;
    if (n_sel > 0 && s_blk[n_sel - 1] == a.nb - 1) n_blk -= a.nb * a.bs - a.P;  // short last block
    int32_t* list = a.kv_list + static_cast<int64_t>(li) * a.key_cap;
    const int G = a.L - a.P;
    const int n_fixed = n_blk + G;
    const int per = (n_fixed + kPrepListWgs - 1) / kPrepListWgs;
    const int lo = blockIdx.y * per, hi = min(n_fixed, lo + per);
    for (int pos = lo + tid; pos < hi; pos += blockDim.x) {
        int key;
        if (pos < n_blk) {
            const int c = pos / a.bs;
            key = s_blk[c] * a.bs + (pos - c * a.bs);
        } else {
            key = a.P + (pos - n_blk);
        }
        list[pos] = key;
    }
    if (blockIdx.y != 0) return;
    int n_unc = canonical_ids(a.sink_idx + static_cast<int64_t>(b) * a.n_sinks, a.n_sinks, 0, a.P, s_snk, s_scr,
                              s_tmp);
    n_unc = filter_ids(s_snk, n_unc, s_scr, s_tmp, [&](int j) { return sorted_contains(s_blk, n_sel, j / a.bs); });
    for (int i = tid; i < n_unc; i += blockDim.x) list[n_fixed + i] = s_snk[i];
    if (tid == 0) a.n_keys[li] = n_fixed + n_unc;
}

// Merge of the key-range splits.  Each thread owns 8 elements of one output row
// (b, h, r); it takes the splits four at a time, and the loads of a group's running
// maxima/sums and partial outputs are independent, so a group costs one memory round
// trip.  Valid rows get
// O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s in split order; padding rows
// (r >= n_q[b]) are written as zero with lse = -inf.
constexpr int kMergeEpt = 8;
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnArgs a) {
    constexpr int TPR = D / kMergeEpt;              // threads per row
    constexpr int RPW = 256 / TPR;                  // rows per workgroup
    constexpr int kMaxSplits = 16;
    const int sub = threadIdx.x % TPR;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RPW + threadIdx.x / TPR;
    const int64_t n_rows = static_cast<int64_t>(a.B) * a.Hq * a.nq_max;
    if (row >= n_rows) return;
    const int r = static_cast<int>(row % a.nq_max);
    const int h = static_cast<int>((row / a.nq_max) % a.Hq);
    const int b = static_cast<int>(row / (static_cast<int64_t>(a.nq_max) * a.Hq));
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    T* orow = static_cast<T*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr + kMergeEpt * sub;
    float o[kMergeEpt];
#pragma unroll
    for (int e = 0; e < kMergeEpt; ++e) o[e] = 0.0f;
    float M = kNegBig, Lsum = 0.0f;
    if (r < nq) {
        // partial of split s at index base + s * step (per row, or per work item when the
        // persistent kernel chose the split count)
        int ns = min(a.n_splits, kMaxSplits);
        int64_t base = row * a.n_splits, step = 1;
        if (a.dyn) {
            const int nqt_max = valid_q_tiles(a, kD128Rows);
            ns = dyn_splits(a, nqt_max);
            if (ns == 1) return;   // the attention kernel wrote this row itself
            const int g = h / a.Gq;
            const int p = r * a.Gq + (h - g * a.Gq);
            base = d128_part_index(a, nqt_max, ns, b, g, 0, p);
            step = static_cast<int64_t>(nqt_max) * kD128Rows;
        }
        // splits in groups of 4: the 4 partials of a group are loaded together, then folded
        // into the running (max, sum, row) with one rescale per group (few registers, so
        // many rows are in flight)
        constexpr int kGroup = 4;
        for (int s0 = 0; s0 < ns; s0 += kGroup) {
            float m[kGroup], l[kGroup];
            f32x4 x[kGroup][2];
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                m[j] = kNegBig;
                l[j] = 0.0f;
                x[j][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                x[j][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                if (s0 + j < ns) {
                    const int64_t idx = base + (s0 + j) * step;
                    m[j] = a.part_ml[2 * idx];
                    l[j] = a.part_ml[2 * idx + 1];
                    const float* po = a.part_o + idx * D + kMergeEpt * sub;
                    x[j][0] = *reinterpret_cast<const f32x4*>(po);
                    x[j][1] = *reinterpret_cast<const f32x4*>(po + 4);
                }
            }
            float Mg = M;
#pragma unroll
            for (int j = 0; j < kGroup; ++j) Mg = fmaxf(Mg, m[j]);
            const float r0 = exp2f(M - Mg);
            Lsum *= r0;
#pragma unroll
            for (int e = 0; e < kMergeEpt; ++e) o[e] *= r0;
            M = Mg;
#pragma unroll
            for (int j = 0; j < kGroup; ++j) {
                const float w = exp2f(m[j] - M);
                Lsum = fmaf(l[j], w, Lsum);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[e] = fmaf(x[j][0][e], w, o[e]);
                    o[4 + e] = fmaf(x[j][1][e], w, o[4 + e]);
                }
            }
        }
        const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
#pragma unroll
        for (int e = 0; e < kMergeEpt; ++e) o[e] *= inv;
    }
    if (sizeof(T) == 2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(o[2 * e], o[2 * e + 1]);
        *reinterpret_cast<u32x4*>(orow) = w;
    } else {
#pragma unroll
        for (int e = 0; e < kMergeEpt; ++e) Elem<T>::store(orow + e, o[e]);
    }
    if (a.lse && sub == 0)
        a.lse[row] = (r < nq && Lsum > 0.0f) ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ bf16 MFMA kernel

template <int D, bool SPARSE>
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
    __shared__ int s_kidx[SPARSE ? 2 : 1][64];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int hf = lane >> 5;
    const int col = lane & 31;
    const WorkUnit u = decode_unit(a, 128);
    if (!u.valid) return;
    const int b = u.b, g = u.g;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows_valid = a.Gq * nq;
    const int rows_all = a.Gq * a.nq_max;
    const int p0 = u.qt * 128;
    const int p = p0 + wv * 32 + col;       // this lane's packed query row
    const bool row_ok = p < rows_valid;
    const int h = g * a.Gq + p % a.Gq;
    const int r = p / a.Gq;

    const int n_keys = SPARSE ? a.n_keys[list_of(a, b, g)] : a.L;
    const int n_tiles = (n_keys + 63) / 64;
    const int t_begin = u.split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);
    const int32_t* klist = SPARSE ? a.kv_list + static_cast<int64_t>(list_of(a, b, g)) * a.key_cap : nullptr;

    // Key index of row `row` of tile t.  Rows outside the split or past n_keys read a
    // clamped valid row instead: such rows are masked (-inf score) or never computed,
    // so the loads need no per-lane branch and the loop body stays straight-line.
    auto fetch_kidx = [&](int t) -> int {   // threads 0..63: key of row tid of tile t, or -1
        const int pos = t * 64 + tid;
        return (t < t_end && pos < n_keys) ? klist[pos] : -1;
    };
    auto key_of = [&](int t, int row) -> int {
        if (SPARSE) return max(s_kidx[t & 1][row], 0);
        return min(t * 64 + row, n_keys - 1);
    };

    // Q fragments (B operand of S^T = K Q^T): lane holds row p, d = 16c + 8hf .. +7.
    // Padding lanes read a valid row; their outputs are never written.
    bf16x8 qf[NQC];
    {
        const int rr = row_ok ? r : 0;
        int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + rr] : rr;
        phys = max(phys, 0);
        const int hh = row_ok ? h : g * a.Gq;
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.qsb + hh * a.qsh +
                               static_cast<int64_t>(phys) * a.qsr;
#pragma unroll
        for (int c = 0; c < NQC; ++c) qf[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * c + 8 * hf));
    }

    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + g * a.ksh;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.vsb + g * a.vsh;

    u32x4 kreg[KPT];
    u32x4 vreg[VPT][2];
    auto load_tile = [&](int t) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int key = key_of(t, i * KROWS + tid / NCH);
            kreg[i] = *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * a.ksr + (tid % NCH) * 8);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int ch = (tid >> 5) + 8 * i;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int key = key_of(t, 2 * (tid & 31) + e);
                vreg[i][e] = *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(key) * a.vsr + ch * 8);
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint8_t* kb = smem + buf * STAGE;
        uint8_t* vb = kb + KBUF;
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int row = i * KROWS + tid / NCH;
            *reinterpret_cast<u32x4*>(kb + row * KP + (tid % NCH) * 16) = kreg[i];
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
        if (SPARSE) {
            if (tid < 64) {
                s_kidx[t_begin & 1][tid] = fetch_kidx(t_begin);
                s_kidx[(t_begin + 1) & 1][tid] = fetch_kidx(t_begin + 1);
            }
            __syncthreads();
        }
        load_tile(t_begin);
        store_tile(0);
      // the loop is entered only after the prologue, so no path reaches it with the
      // Q-fragment loads still outstanding (which would force a full wait per tile)
      for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        __syncthreads();
        load_tile(t + 1);   // past the split's last tile this reads valid rows that are never used
        int next_kidx = -1;
        if (SPARSE && tid < 64) next_kidx = fetch_kidx(t + 2);
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
        const int valid_here = n_keys - t * 64;   // keys of this tile that exist
        if (valid_here < 64) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kl = kb2 * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                    if (kl >= valid_here) st[kb2][i] = -INFINITY;
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
        const float alpha = fast_exp2(m_run - m_new);
        float psum = 0.0f;
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = fast_exp2(fmaf(st[kb2][i], a.sl2, -m_new));
                st[kb2][i] = pv;
                psum += pv;
            }
        l_run = fmaf(l_run, alpha, psum);
        // the output only needs rescaling when some lane's running max moved
        if (__any(m_new != m_run)) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
        }
        m_run = m_new;

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
        store_tile(buf ^ 1);
        if (SPARSE && tid < 64) s_kidx[t & 1][tid] = next_kidx;
      }
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (a.n_splits == 1) {
        if (row_ok) {
            uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.osb + h * a.osh + static_cast<int64_t>(r) * a.osr;
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
        return;
    }
    if (row_ok) {
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

template <int D, bool SPARSE>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnArgs a) {
    __shared__ __attribute__((aligned(16))) float s_k[kF32Keys][D];
    __shared__ __attribute__((aligned(16))) float s_v[kF32Keys][D];
    __shared__ int s_key[kF32Keys];

    const int lane = threadIdx.x;
    const WorkUnit u = decode_unit(a, kF32Rows);
    if (!u.valid) return;
    const int b = u.b, g = u.g;
    const int nq = a.n_q ? a.n_q[b] : a.nq_max;
    const int rows_valid = a.Gq * nq;
    const int rows_all = a.Gq * a.nq_max;
    const int p0 = u.qt * kF32Rows;
    const int p = p0 + lane;
    const bool row_ok = p < rows_valid;
    const int h = g * a.Gq + p % a.Gq;
    const int r = p / a.Gq;
    const int n_keys = SPARSE ? a.n_keys[list_of(a, b, g)] : a.L;
    const int n_tiles = (n_keys + kF32Keys - 1) / kF32Keys;
    const int t_begin = u.split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);
    const int32_t* klist = SPARSE ? a.kv_list + static_cast<int64_t>(list_of(a, b, g)) * a.key_cap : nullptr;

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
            const int pos = t * kF32Keys + lane;
            s_key[lane] = pos < n_keys ? (SPARSE ? klist[pos] : pos) : -1;
        }
        __syncthreads();
        for (int i = lane; i < kF32Keys * D / 4; i += 64) {
            const int row = i / (D / 4);
            const int c4 = i % (D / 4);
            const int key = s_key[row];
            f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
            if (key >= 0) {
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
                s[j] = s_key[j0 + j] >= 0 ? dot * a.sl2 : -INFINITY;
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
        return;
    }
    if (row_ok) {
        const int64_t idx = ((static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r) * a.n_splits + u.split;
#pragma unroll
        for (int e = 0; e < D; ++e) a.part_o[idx * D + e] = acc[e];
        a.part_ml[idx * 2 + 0] = m_run;
        a.part_ml[idx * 2 + 1] = l_run;
    }
}

template <int D>
void launch_kernel(fdl_dtype dtype, const AttnArgs& a, dim3 grid, hipStream_t stream) {
    if (dtype == FDL_BF16) {
        if (a.sparse) hipLaunchKernelGGL((attn_bf16_kernel<D, true>), grid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_bf16_kernel<D, false>), grid, dim3(256), 0, stream, a);
    } else {
        if (a.sparse) hipLaunchKernelGGL((attn_f32_kernel<D, true>), grid, dim3(kF32Rows), 0, stream, a);
        else hipLaunchKernelGGL((attn_f32_kernel<D, false>), grid, dim3(kF32Rows), 0, stream, a);
    }
}


}  // namespace

AttnPlan plan_attention(fdl_dtype dtype, int B, int Hq, int Hkv, int d, int nq_max,
                        int64_t key_bound, bool sparse, bool per_head) {
    AttnPlan pl;
    const bool bf16 = dtype == FDL_BF16;
    const bool d128 = bf16 && d == 128;
    pl.rows_per_tile = d128 ? kD128Rows : bf16 ? 128 : kF32Rows;
    pl.tile_keys = bf16 ? 64 : kF32Keys;
    const int64_t rows = static_cast<int64_t>(Hq / Hkv) * nq_max;
    pl.q_tiles = static_cast<int>((rows + pl.rows_per_tile - 1) / pl.rows_per_tile);
    const int64_t tiles = (key_bound + pl.tile_keys - 1) / pl.tile_keys;
    pl.tiles_total = static_cast<int>(tiles > 0 ? tiles : 1);
    const int64_t units = static_cast<int64_t>(B) * Hkv * pl.q_tiles;
    const int64_t max_splits = tiles / kMinSplitTiles > 1 ? tiles / kMinSplitTiles : 1;
    int64_t splits;
    if (d128) {
        // the kernel picks the split count on the device (it knows the valid rows);
        // the workspace covers the most it can pick
        splits = max_splits < 16 ? max_splits : 16;
    } else {
        const int64_t target = 1024;  // workgroups that keep 256 CUs busy
        splits = (target + units - 1) / units;
        if (splits > max_splits) splits = max_splits;
        if (splits > 16) splits = 16;   // attn_merge holds at most 16 splits per row in registers
    }
    if (splits < 1) splits = 1;
    pl.n_splits = static_cast<int>(splits);
    pl.tiles_per_split = static_cast<int>((tiles + splits - 1) / splits);
    if (pl.tiles_per_split < 1) pl.tiles_per_split = 1;
    pl.key_cap = sparse ? key_bound : 0;
    const int64_t lists = per_head ? static_cast<int64_t>(B) * Hkv : B;
    pl.list_bytes = sparse ? round_up(static_cast<size_t>(lists) * (key_bound + 1) * sizeof(int32_t), 256) : 0;
    pl.part_bytes = 0;
    if (pl.n_splits > 1) {
        int64_t nrows;
        if (d128) {
            const int64_t items = units * pl.n_splits;
            nrows = (items < kD128MaxSlots ? items : kD128MaxSlots) * kD128Rows;
        } else {
            nrows = static_cast<int64_t>(B) * Hq * nq_max * pl.n_splits;
        }
        pl.part_bytes = static_cast<size_t>(nrows) * (d + 2) * sizeof(float);
    }
    pl.ws_bytes = pl.list_bytes + pl.part_bytes;
    return pl;
}

hipError_t launch_attention(fdl_dtype dtype, int d, const AttnArgs& args_in, const AttnPlan& pl,
                            hipStream_t stream) {
    AttnArgs a = args_in;
    a.q_tiles = pl.q_tiles;
    a.n_splits = pl.n_splits;
    a.tiles_per_split = pl.tiles_per_split;
    a.key_cap = static_cast<int>(pl.key_cap);
    uint8_t* ws = reinterpret_cast<uint8_t*>(a.part_o);  // the caller's workspace base
    a.kv_list = nullptr;
    a.n_keys = nullptr;
    if (a.sparse) {
        a.kv_list = reinterpret_cast<int32_t*>(ws);
        a.n_keys = a.kv_list + static_cast<int64_t>(n_lists(a)) * pl.key_cap;
    }
    a.part_o = pl.part_bytes ? reinterpret_cast<float*>(ws + pl.list_bytes) : nullptr;
    a.part_ml = a.part_o ? a.part_o + static_cast<int64_t>(pl.part_bytes / ((d + 2) * sizeof(float))) * d : nullptr;
    a.tiles_total = pl.tiles_total;
    a.bs_magic = a.bs >= 2 ? static_cast<uint32_t>(((uint64_t(1) << 32) + a.bs - 1) / a.bs) : 0u;
    const bool d128 = dtype == FDL_BF16 && d == 128;
    a.dyn = d128 ? 1 : 0;
    a.slots = d128 ? d128_slots() : 0;
    const bool zero_pad = a.n_q && pl.n_splits == 1;
    // the bf16 d = 128 kernel maps small sparse key sets itself; everything else reads the list
    const bool need_list = a.sparse && !(dtype == FDL_BF16 && d == 128 && sparse_map_in_lds(a));
    if (need_list || zero_pad) {
        const int pad_wgs = zero_pad ? 64 : 0;   // extra workgroups that zero the padding rows
        const dim3 pgrid(n_lists(a), kPrepListWgs + pad_wgs);
        if (dtype == FDL_BF16) hipLaunchKernelGGL(attn_prep_kernel<uint16_t>, pgrid, dim3(256), 0, stream, a, d, need_list);
        else hipLaunchKernelGGL(attn_prep_kernel<float>, pgrid, dim3(256), 0, stream, a, d, need_list);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    // groups of q_tiles consecutive slots per XCD: round the group count up to a multiple of 8
    const int64_t groups = static_cast<int64_t>(a.B) * a.Hkv * pl.n_splits;
    const dim3 grid(static_cast<unsigned>((groups + 7) / 8 * 8 * pl.q_tiles));
    hipError_t err = hipSuccess;
    if (d128) err = launch_attn_bf16_d128(a, stream);
    else if (d == 128) launch_kernel<128>(dtype, a, grid, stream);
    else launch_kernel<64>(dtype, a, grid, stream);
    if (err == hipSuccess) err = hipGetLastError();
    if (err != hipSuccess || pl.n_splits == 1) return err;
    const int64_t n_rows = static_cast<int64_t>(a.B) * a.Hq * a.nq_max;
    const int64_t rows_per_wg = 256 / (d / kMergeEpt);
    const dim3 mgrid(static_cast<unsigned>((n_rows + rows_per_wg - 1) / rows_per_wg));
    if (dtype == FDL_BF16) {
        if (d == 128) hipLaunchKernelGGL((attn_merge_kernel<uint16_t, 128>), mgrid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<uint16_t, 64>), mgrid, dim3(256), 0, stream, a);
    } else {
        if (d == 128) hipLaunchKernelGGL((attn_merge_kernel<float, 128>), mgrid, dim3(256), 0, stream, a);
        else hipLaunchKernelGGL((attn_merge_kernel<float, 64>), mgrid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace fdl
