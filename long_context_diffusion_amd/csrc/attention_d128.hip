// bf16 attention, head dim 128: dense or sparse key set, software-pipelined.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
// steps" (3) and (5): dense attention of the active rows (and of every row at a
// block-entry refresh), and attention of the active rows over I_p only.
//
// Per workgroup: 4 waves x 32 query rows of one KV head (grouped-query heads
// interleaved into the rows), 64-key tiles.
//   * K and V tiles go from global memory straight into LDS (global_load_lds,
//     16 bytes per lane), with no staging registers.  Rows are 256 bytes and
//     unpadded; the 16-byte chunk c of row r sits at slot c ^ 2*(r & 7), which
//     keeps both LDS read patterns below free of bank conflicts.
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16, keys on the M axis): one lane owns
//     one query's softmax state.
//   * O^T += V^T P^T: V stays row-major in LDS and the V^T operand is read with
//     ds_read_b64_tr_b16.  In each 16-lane group, lane j points at 4 consecutive
//     d of key key0 + j/4; lane i then receives keys key0..key0+3 at d0 + i, the
//     4 k-slots the MFMA wants.  Two such reads fill one 8-slot operand, whose key
//     order matches the accumulator layout of S^T, so P needs no shuffle.
//   * Pipeline: S for tile t+1 is computed while tile t's softmax and P V run;
//     K runs one tile ahead of V (K tiles t+1, t+2 and V tiles t, t+1 in LDS);
//     the loads for the next tiles are in flight during the whole iteration, and
//     one barrier closes it.
//   * Key indices reach the loads through a 4-deep ring in LDS filled by wave 0:
//     dense keys are t*64 + row; sparse keys are mapped in-kernel from LDS copies
//     of the selected blocks and of the sinks that no block or the generation
//     region holds (or read from the list written by attn_prep when those sets are
//     too large for LDS).

#include "attention.cuh"

namespace fdl {

namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowB = 256;             // bytes per K/V row in LDS
constexpr int kTileB = 64 * kRowB;     // one 64-key tile: 16 KB

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row & 7) << 1); }

template <bool SPARSE>
__global__ __launch_bounds__(256, 2) void attn_d128_kernel(const AttnArgs a) {
    constexpr int D = 128;
    constexpr int NQC = D / 16;   // 16-wide d chunks of Q . K
    constexpr int NDB = D / 32;   // 32-wide d blocks of the output
    // four separate LDS objects, so the compiler can tell a tile being loaded by DMA
    // from the tiles being read (one shared array would force a wait on every read)
    __shared__ __attribute__((aligned(1024))) uint8_t s_k0[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_k1[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_v0[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_v1[kTileB];
    __shared__ int s_kidx[4][64];
    __shared__ int s_blk[SPARSE ? kMapBlocks : 1];
    __shared__ int s_unc[SPARSE ? kMapSinks : 1];
    __shared__ int s_tmp[17];
    __shared__ int s_carry;

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
    const int p = p0 + wv * 32 + col;
    const bool row_ok = p < rows_valid;
    const int h = g * a.Gq + p % a.Gq;
    const int r = p / a.Gq;

    // ---- key set of this sequence
    int n_keys = a.L, n_blk = 0, sink0 = a.L;
    const bool in_lds = !SPARSE || sparse_map_in_lds(a);
    const int32_t* klist = nullptr;
    if (SPARSE) {
        if (in_lds) {
            const int32_t* blk_g = a.block_idx + static_cast<int64_t>(b) * a.C;
            int cnt = 0;
            for (int c = tid; c < a.C; c += blockDim.x) {
                const int v = blk_g[c];
                s_blk[c] = v;
                cnt += v >= 0 ? 1 : 0;
            }
            int n_sel;
            block_exclusive_sum(cnt, s_tmp, &n_sel);
            n_sel = min(n_sel, a.nb);
            n_blk = n_sel * a.bs;
            if (n_sel > 0 && s_blk[n_sel - 1] == a.nb - 1) n_blk -= a.nb * a.bs - a.P;
            sink0 = n_blk + (a.L - a.P);
            if (tid == 0) s_carry = 0;
            __syncthreads();
            const int32_t* snk = a.sink_idx + static_cast<int64_t>(b) * a.n_sinks;
            for (int s0 = 0; s0 < a.n_sinks; s0 += blockDim.x) {
                const int s = s0 + tid;
                int j = -1;
                bool take = false;
                if (s < a.n_sinks) {
                    j = snk[s];
                    take = j >= 0 && j < a.P && (s == 0 || snk[s - 1] != j);
                    if (take) {
                        const int target = j / a.bs;
                        int lo = 0, hi = n_sel;
                        while (lo < hi) {
                            const int mid = (lo + hi) >> 1;
                            if (s_blk[mid] < target) lo = mid + 1; else hi = mid;
                        }
                        take = !(lo < n_sel && s_blk[lo] == target);
                    }
                }
                int total;
                const int off = block_exclusive_sum(take ? 1 : 0, s_tmp, &total) + s_carry;
                if (take) s_unc[off] = j;
                __syncthreads();
                if (tid == 0) s_carry += total;
                __syncthreads();
            }
            n_keys = sink0 + s_carry;
        } else {
            n_keys = a.n_keys[b];
            klist = a.kv_list + static_cast<int64_t>(b) * a.key_cap;
        }
    }
    const int n_tiles = (n_keys + 63) / 64;
    const int t_begin = u.split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);

    // key of position pos of tile t; past the split or past n_keys: row 0 (never used)
    auto key_at = [&](int t, int pos) -> int {
        if (t >= t_end || pos >= n_keys) return 0;
        if (!SPARSE) return pos;
        if (!in_lds) return klist[pos];
        if (pos < n_blk) {
            const int c = pos / a.bs;
            return min(max(s_blk[c] * a.bs + (pos - c * a.bs), 0), a.L - 1);
        }
        if (pos < sink0) return a.P + (pos - n_blk);
        return s_unc[pos - sink0];
    };

    // ---- Q fragments (B operand of S^T = K Q^T): row p, d = 16c + 8hf .. +7
    bf16x8 qf[NQC];
    {
        const int rr = row_ok ? r : 0;
        int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + rr] : rr;
        phys = max(phys, 0);
        const int hh = row_ok ? h : g * a.Gq;
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + b * a.qsb + hh * a.qsh +
                               static_cast<int64_t>(phys) * a.qsr;
#pragma unroll
        for (int c = 0; c < NQC; ++c)
            qf[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * c + 8 * hf));
    }
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + g * a.ksh;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.vsb + g * a.vsh;

    // ---- direct global -> LDS loads of one tile (4 instructions per wave)
    auto issue_tile = [&](const uint16_t* base, int64_t rstride, int t, uint8_t* dst) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int blk1k = 4 * wv + i;                 // 1 KB block of the tile
            const int row = 4 * blk1k + (lane >> 4);
            const int chunk = swz(row, lane & 15);        // global chunk held at slot (lane & 15)
            const int key = s_kidx[t & 3][row];
            const uint16_t* src = base + static_cast<int64_t>(key) * rstride + 8 * chunk;
            __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + 1024 * blk1k), 16, 0, 0);
        }
    };

    // ---- S^T tile = K Q^T from an LDS K tile
    auto qk = [&](const uint8_t* kt, f32x16* st) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
            for (int i = 0; i < 16; ++i) st[kb2][i] = 0.0f;
            const int row = kb2 * 32 + col;
            const uint8_t* krow = kt + row * kRowB;
#pragma unroll
            for (int c = 0; c < NQC; ++c) {
                const bf16x8 ak = *reinterpret_cast<const bf16x8*>(krow + 16 * swz(row, 2 * c + hf));
                st[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak, qf[c], st[kb2], 0, 0, 0);
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
        if (wv == 0) {
            s_kidx[t_begin & 3][lane] = key_at(t_begin, t_begin * 64 + lane);
            s_kidx[(t_begin + 1) & 3][lane] = key_at(t_begin + 1, (t_begin + 1) * 64 + lane);
            s_kidx[(t_begin + 2) & 3][lane] = key_at(t_begin + 2, (t_begin + 2) * 64 + lane);
        }
        __syncthreads();
        issue_tile(kbase, a.ksr, t_begin, s_k0);
        issue_tile(vbase, a.vsr, t_begin, s_v0);
        issue_tile(kbase, a.ksr, t_begin + 1, s_k1);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        f32x16 st[2];
        qk(s_k0, st);

        // One pipelined iteration: tile t's K was read last iteration (it sits in kdma),
        // tile t+1's K is in kread, tile t's V is in vread, tile t+1's V goes to vdma.
        auto iteration = [&](int t, uint8_t* kread, uint8_t* kdma, uint8_t* vread, uint8_t* vdma) {
            // the key map is read before the DMA loads go out: an LDS read issued behind
            // them would have to wait for their completion
            int next_key = 0;
            if (wv == 0) next_key = key_at(t + 3, (t + 3) * 64 + lane);
            issue_tile(kbase, a.ksr, t + 2, kdma);
            issue_tile(vbase, a.vsr, t + 1, vdma);

            // S for tile t+1 (its K is resident) while this tile's softmax runs
            f32x16 sn[2];
            qk(kread, sn);

            const int valid_here = n_keys - t * 64;
            if (valid_here < 64) {
#pragma unroll
                for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int kl = kb2 * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                        if (kl >= valid_here) st[kb2][i] = -INFINITY;
                    }
            }
            float mx = fmaxf(st[0][0], st[0][1]);
#pragma unroll
            for (int i = 2; i < 16; ++i) mx = fmaxf(mx, st[0][i]);
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, st[1][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run, mx * a.sl2);
            const float alpha = fast_exp2(m_run - m_new);
            float psum = 0.0f;
            bf16x8 pf[4];
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float pv = fast_exp2(fmaf(st[kc >> 1][8 * (kc & 1) + j], a.sl2, -m_new));
                    psum += pv;
                    pf[kc][j] = static_cast<__bf16>(pv);
                }
            l_run = fmaf(l_run, alpha, psum);
            if (__any(m_new != m_run)) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
            }
            m_run = m_new;

            // O^T += V^T P^T with transposing LDS reads of the row-major V tile
            const int grp = lane >> 4, j16 = lane & 15;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int e = db * 32 + 16 * (grp & 1) + 4 * (j16 & 3);   // first d of this lane's pointer
#pragma unroll
                for (int kc = 0; kc < 4; ++kc) {
                    const int key0 = kc * 16 + 4 * hf + (j16 >> 2);
                    const int key1 = key0 + 8;
                    uint8_t* p0v = vread + key0 * kRowB + 16 * swz(key0, e >> 3) + 2 * (e & 7);
                    uint8_t* p1v = vread + key1 * kRowB + 16 * swz(key1, e >> 3) + 2 * (e & 7);
                    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0v);
                    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1v);
                    const bf16x8 av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf[kc], acc[db], 0, 0, 0);
                }
            }
            if (wv == 0) s_kidx[(t + 3) & 3][lane] = next_key;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            st[0] = sn[0];
            st[1] = sn[1];
        };
        // even iterations read K from s_k1 and V from s_v0; odd ones the other way round
        for (int t = t_begin; t < t_end; t += 2) {
            iteration(t, s_k1, s_k0, s_v0, s_v1);
            if (t + 1 < t_end) iteration(t + 1, s_k0, s_k1, s_v1, s_v0);
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

}  // namespace

hipError_t launch_attn_bf16_d128(const AttnArgs& a, dim3 grid, hipStream_t stream) {
    if (a.sparse) hipLaunchKernelGGL(attn_d128_kernel<true>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(attn_d128_kernel<false>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fdl
