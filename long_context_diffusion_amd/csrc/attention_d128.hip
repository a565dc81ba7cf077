// bf16 attention, head dim 128: dense or sparse key set.
//
// Focus-dLLM structured summary (paper.rainbus.top/paper/2602.02159), "Method
// steps" (3) and (5): dense attention of the active rows (and of every row at a
// block-entry refresh), and attention of the active rows over I_p only.
//
// A workgroup (8 waves x 32 query rows of one KV head; grouped-query heads are
// interleaved into the rows) walks a range of 64-key tiles, one workgroup per CU
// (two waves per SIMD).  The grid is persistent: it walks (query tile, key split)
// items, and the number of key splits comes from the device-side row counts, so a
// sparse step with few active rows still fills every CU.
//   * K and V tiles go from global memory straight into LDS (global_load_lds, 16
//     bytes per lane) through 4-deep rings: while tile t is finished, the tiles t+1
//     and t+2 are landing, so every load has a whole element to arrive.  K rows are
//     256 bytes, unpadded; 16-byte chunk c of LDS row r of K sits at slot c ^ (r & 15),
//     which makes the 128-bit reads of S = K Q^T conflict-free.  One DMA instruction
//     fills 4 LDS rows, and a lane's 2 rows of a tile are fixed key positions, so every
//     lane maps its own keys: no index ring, no wave waiting on another.
//   * P V reads V^T (rows d, slots keys) with conflict-free 128-bit reads.  When the
//     caller supplies V^T (keys contiguous), a tile of 64 consecutive keys (every tile
//     of a dense range, the tiles inside a selected block or inside [P, L)) is loaded
//     from it straight into the swizzled V^T layout.  Other tiles (sinks, tiles that
//     straddle two parts of I_p, or no V^T given) load V rows into one staging buffer,
//     and each lane turns 2 rows x 8 d into 8 words of V^T one element later
//     (transposing LDS reads of the row-major tile run at about a third of the plain
//     rate on gfx950).
//   * S^T = K Q^T (v_mfma_f32_32x32x16_bf16, keys on the M axis): one lane owns one
//     query's softmax state.  S of tile t+1 is computed while tile t is finished.
//   * O^T += V^T P^T.  Row r of a K tile holds key vt_row(r) of the tile, so the S^T
//     rows a lane holds for one 16-key chunk are 8 consecutive keys: P goes to the
//     MFMA straight from the softmax registers, and V^T slot s is simply key s.
//   * The running max is only raised when a tile's max exceeds it by more than 2^8
//     (exp2 units), so rescaling the accumulators is rare; the final
//     normalisation is exact either way.

#include "attention_tiles.cuh"

namespace fdl {

namespace {

// PER_HEAD (kSparseLds only): every KV head maps its own block list
template <int MODE, bool PER_HEAD = false>
__global__ __launch_bounds__(512) void attn_d128_kernel(const AttnArgs a) {
    constexpr int NQC = 8;   // 16-wide d chunks of Q . K
    constexpr int NDB = 4;   // 32-wide d blocks of the output
    // separate LDS objects for every tile buffer: the compiler tells a tile being loaded by DMA from the
    // tiles being read only when they are different objects
    __shared__ __attribute__((aligned(1024))) uint8_t s_t0[kTileB];   // V^T tiles
    __shared__ __attribute__((aligned(1024))) uint8_t s_t1[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_t2[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_t3[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_k0[kTileB];   // K tiles
    __shared__ __attribute__((aligned(1024))) uint8_t s_k1[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_k2[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_k3[kTileB];
    __shared__ __attribute__((aligned(1024))) uint8_t s_raw[kTileB];  // row-major V of a tile to transpose
    __shared__ int s_blk[MODE == kSparseLds ? kMapBlocks : 1];
    __shared__ int s_unc[MODE == kSparseLds ? kMapSinks : 1];
    __shared__ int s_tmp[17];
    __shared__ uint64_t s_tmp64[8];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5;
    const int col = lane & 31;
    const int g4 = lane >> 4;
    const int qlane = vt_row(8 * wv + g4);   // key position of this lane's first DMA row

    const int nqt_max = valid_q_tiles(a, kD128Rows);
    const int n_splits = dyn_splits(a, nqt_max);
    const int tps = (a.tiles_total + n_splits - 1) / n_splits;
    const int n_items = (a.B * a.Hkv * n_splits + 7) / 8 * 8 * nqt_max;
    const int rows_all = a.Gq * a.nq_max;

    for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
        const WorkUnit u = decode_unit_id(a, kD128Rows, item, n_splits, nqt_max);
        if (!u.valid) continue;
        __syncthreads();   // the previous item's readers of the LDS maps are done
        const int b = u.b, g = u.g;
        const int nq = a.n_q ? a.n_q[b] : a.nq_max;
        const int rows_valid = a.Gq * nq;

        // ---- Q fragments (B operand of S^T = K Q^T): d = 16c + 8hf .. +7 of the row.  Their
        // loads go out before the key map is built, so both round trips overlap.  With a
        // key map to build, the rows go by DMA into the idle V^T tile buffers (wave wv's 32
        // rows at its epilogue staging area, chunk c of row r at slot c ^ (r & 15)) and reach
        // registers after the map is done, so no registers are held across the map.
        const int p = u.qt * kD128Rows + wv * 32 + col;   // 8 waves x 32 rows
        const bool row_ok = p < rows_valid;
        bf16x8 qf[NQC];
        uint8_t* qstage = (wv < 2 ? s_t0 : wv < 4 ? s_t1 : wv < 6 ? s_t2 : s_t3) + (wv & 1) * 8192;
        auto q_row_ptr = [&](int pr) __attribute__((always_inline)) {
            const bool ok = pr < rows_valid;
            const int rr = ok ? pr / a.Gq : 0;
            const int hh = ok ? g * a.Gq + pr % a.Gq : g * a.Gq;
            int phys = a.q_idx ? a.q_idx[static_cast<int64_t>(b) * a.nq_max + rr] : rr;
            phys = max(phys, 0);
            return static_cast<const uint16_t*>(a.q) + b * a.qsb + hh * a.qsh + static_cast<int64_t>(phys) * a.qsr;
        };
        if (MODE == kSparseLds) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 4 * i + (lane >> 4);
                const uint16_t* src = q_row_ptr(u.qt * kD128Rows + wv * 32 + r) + 8 * ((lane & 15) ^ (r & 15));
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(qstage + 1024 * i), 16, 0, 0);
            }
        } else {
            const uint16_t* qrow = q_row_ptr(p);
#pragma unroll
            for (int c = 0; c < NQC; ++c)
                qf[c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 16 * c + 8 * hf));
        }

        // ---- key set of this sequence (build_key_map): blocks, then [P, L), then the sinks
        // no selected block holds; the V-row staging buffer is the sort scratch
        int n_keys = a.L, n_blk = 0, sink0 = a.L;
        const int32_t* klist = nullptr;
        if (MODE == kSparseLds) {
            build_key_map<512, PER_HEAD>(a, b, g, s_blk, s_unc, s_tmp, s_tmp64, reinterpret_cast<int*>(s_raw), n_blk, sink0, n_keys);
            // the Q rows have landed in this wave's staging area: fragments to registers, then
            // every wave is done with the staging areas before tile loads overwrite them
            __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
            for (int c = 0; c < NQC; ++c)
                qf[c] = *reinterpret_cast<const bf16x8*>(qstage + col * kRowB + 16 * ((2 * c + hf) ^ (col & 15)));
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        } else if (MODE == kSparseList) {
            n_keys = a.n_keys[list_of(a, b, g)];
            klist = a.kv_list + static_cast<int64_t>(list_of(a, b, g)) * a.key_cap;
        }
        const int n_tiles = (n_keys + 63) / 64;
        const int t_begin = u.split * tps;
        const int t_end = min(n_tiles, t_begin + tps);

        // Rows of this lane's 2 key positions of tile t, qlane and qlane + 8 (LDS rows
        // 8wv + g4 and 8wv + 4 + g4; row 0 past the split or the key set), in two halves
        // one element apart: keys_fetch reads what the key map holds
        // for them (LDS, or the key list in global memory), keys_finish forms the rows.
        // The fetch is issued a whole element before its use, so no wave waits on it.
        // A tile that lies inside one selected block (block sizes that are multiples of
        // 64) or inside [P, L) maps position q to base + q: one broadcast lookup (or
        // none) for the whole tile; only tiles that straddle a boundary map key by key.
        // kr[6] is that base, or kNoBase.
        constexpr int kNoBase = -0x40000000;
        const bool bs64 = a.bs % 64 == 0;
        auto keys_fetch = [&](int t, int (&kr)[7]) __attribute__((always_inline)) {
            const int q0 = t * 64 + qlane;
            kr[6] = kNoBase;
            if (MODE == kSparseLds) {
                const int t0q = t * 64;
                if (bs64 && t0q + 64 <= n_blk) {
                    const int c = div_magic(t0q, a.bs, a.bs_magic);
                    kr[6] = s_blk[c] * a.bs - c * a.bs;
                    return;
                }
                if (t0q >= n_blk && t0q + 64 <= sink0) {
                    kr[6] = a.P - n_blk;
                    return;
                }
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = q0 + 8 * i;
                if (MODE == kSparseList) {
                    kr[3 * i] = (t < t_end && q < n_keys) ? klist[q] : 0;
                } else if (MODE == kSparseLds) {
                    // both LDS lookups use in-range indices
                    const int qb = q < n_blk ? q : 0;
                    const int c = div_magic(qb, a.bs, a.bs_magic);
                    kr[3 * i] = s_blk[c];
                    kr[3 * i + 1] = s_unc[min(max(q - sink0, 0), kMapSinks - 1)];
                    kr[3 * i + 2] = qb - c * a.bs;
                }
            }
        };
        auto keys_finish = [&](int t, const int (&kr)[7], int (&key)[2]) __attribute__((always_inline)) {
            const int q0 = t * 64 + qlane;
            const bool live = t < t_end;
            const bool whole = MODE == kSparseLds && kr[6] != kNoBase;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int q = q0 + 8 * i;
                const bool ok = live && q < n_keys;
                int k;
                if (MODE == kDense) {
                    k = q;
                } else if (MODE == kSparseList) {
                    k = kr[3 * i];
                } else if (whole) {
                    k = kr[6] + q;
                } else {
                    const int kb = min(max(kr[3 * i] * a.bs + kr[3 * i + 2], 0), a.L - 1);
                    k = q < n_blk ? kb : (q < sink0 ? a.P + (q - n_blk) : kr[3 * i + 1]);
                }
                // over a dense range a position past the keys (or a tile past the split) reads
                // the last key's row: its scores are masked, and a clamp is cheaper than a select
                key[i] = MODE == kDense ? min(q, n_keys - 1) : (ok ? k : 0);
            }
        };
        // Tiles of 64 consecutive keys (every tile of a dense range; in I_p the tiles
        // inside one selected block or inside [P, L), exactly those keys_fetch maps with
        // one base) load V^T directly when the caller supplies it; the others load V
        // rows and transpose them in LDS.  Both tests are uniform over the workgroup.
        const bool use_vt = MODE != kSparseList && a.vt != nullptr;
        const int n_blk_u = __builtin_amdgcn_readfirstlane(n_blk);
        const int sink0_u = __builtin_amdgcn_readfirstlane(sink0);
        auto whole_tile = [&](int t) __attribute__((always_inline)) {
            if (MODE == kDense) return true;
            if (MODE == kSparseList) return false;
            const int t0q = t * 64;
            return (bs64 && t0q + 64 <= n_blk_u) || (t0q >= n_blk_u && t0q + 64 <= sink0_u);
        };
        auto tile_k0 = [&](int t, const int (&kr)[7]) __attribute__((always_inline)) {
            return (MODE == kDense ? 0 : kr[6]) + t * 64;
        };
        bool raw_next = true;

        const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + b * a.ksb + g * a.ksh;
        const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + b * a.vsb + g * a.vsh;
        const int ksr = static_cast<int>(a.ksr), vsr = static_cast<int>(a.vsr);

        // ---- direct global -> LDS loads of one tile's rows (2 instructions per wave)
        auto issue_k = [&](const int (&key)[2], uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int r = 8 * wv + 4 * i + g4;
                const uint16_t* src = kbase + static_cast<int64_t>(key[i]) * ksr + 8 * swz_k(r, lane & 15);
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + 1024 * (2 * wv + i)), 16, 0, 0);
            }
        };
        auto issue_v = [&](const int (&key)[2], uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint16_t* src = vbase + static_cast<int64_t>(key[i]) * vsr + 8 * (lane & 15);
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + 1024 * (2 * wv + i)), 16, 0, 0);
            }
        };
        // A tile of 64 consecutive keys k0 .. k0+63 (k0 a multiple of 8) straight from V^T
        // in global memory into its swizzled LDS layout: instruction 2wv + i fills rows
        // d = 16wv + 8i .. +7, lane l chunk l % 8 of row d, i.e. keys
        // k0 + 8 ((l % 8) ^ vt_swz(d)) .. +7 (16 contiguous bytes).  Chunks at or past
        // n_keys (only in the last tile of a dense key range; n_keys is a multiple of 8)
        // read the row's last chunk instead: their probabilities are zero.
        const uint16_t* vtbase = static_cast<const uint16_t*>(a.vt) + b * a.vtsb + g * a.vtsh;
        const int vtsd = a.vtsd;
        auto issue_vt = [&](int k0, uint8_t* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int d = 16 * wv + 8 * i + (lane >> 3);
                int kk = k0 + 8 * ((lane & 7) ^ vt_swz(d));
                if (MODE == kDense) kk = min(kk, n_keys - 8);
                const uint16_t* src = vtbase + d * vtsd + kk;
                __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + 1024 * (2 * wv + i)), 16, 0, 0);
            }
        };

        // ---- S^T tile (two 32-key blocks) = K Q^T from an LDS K tile.  The swizzled
        // offset of (row col, chunk 2c + hf) is kofs ^ 32c; key block kb adds 8 KB.
        const int kofs = col * kRowB + ((16 * hf) ^ (16 * (col & 15)));
        auto qk = [&](const uint8_t* kt, f32x16 (&st)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                // all 8 fragments of the key block in flight before the first MFMA
                bf16x8 kf[NQC];
#pragma unroll
                for (int c = 0; c < NQC; ++c)
                    kf[c] = *reinterpret_cast<const bf16x8*>(kt + kb * 32 * kRowB + (kofs ^ (32 * c)));
#pragma unroll
                for (int i = 0; i < 16; ++i) st[kb][i] = 0.0f;
#pragma unroll
                for (int c = 0; c < NQC; ++c)
                    st[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[c], qf[c], st[kb], 0, 0, 0);
            }
        };

        // V^T operand of (kc, db): row d = 32db + col, chunk 2kc + hf, at
        // 4096 db + (tofs ^ 32 (kc ^ db)), since vt_swz(32db + col) = vt_swz(col) ^ 2db
        const int tofs = col * 128 + ((16 * hf) ^ (16 * vt_swz(col)));

        // ---- V tile -> V^T: lane (k, c8) moves rows 2k, 2k+1 x d = 8c8 .. 8c8+7
        const int tr_c8 = tid & 15, tr_k = tid >> 4;   // rows 2k, 2k+1 go to slots vt_row(2k), +1
        auto transpose_load = [&](const uint8_t* vraw, u32x4& ra, u32x4& rb) __attribute__((always_inline)) {
            ra = *reinterpret_cast<const u32x4*>(vraw + (2 * tr_k) * kRowB + 16 * tr_c8);
            rb = *reinterpret_cast<const u32x4*>(vraw + (2 * tr_k + 1) * kRowB + 16 * tr_c8);
        };
        auto transpose_store = [&](const u32x4& ra, const u32x4& rb, uint8_t* vt) __attribute__((always_inline)) {
            // vt_off(8 c8 + e, s) = A ^ (128 e + 16 (e / 2)), A formed here from a lane id
            // that passes an empty asm, so the 8 addresses are not hoisted out of the tile
            // loop (where they would stay live and spill).  The stores are written as asm:
            // the compiler cannot tell this slot from the one a V^T load of the same
            // element is filling (more tile buffers take LDS loads than it tracks apart)
            // and would wait for that load first.  No load into this slot is in flight:
            // the tile was loaded row-major, and the loads of older tiles landed before
            // the previous barrier.
            int el = tid;
            asm volatile("" : "+v"(el));
            const int c8 = el & 15, sl = vt_row(2 * (el >> 4));
            const uint32_t A = static_cast<uint32_t>(reinterpret_cast<size_t>((lds_void*)vt)) + 1024 * c8 +
                               2 * (sl & 7) + 16 * (((sl >> 3) ^ (4 * (c8 & 1)) ^ (c8 >> 1)) & 7);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t x = ra[e >> 1], y = rb[e >> 1];
                const uint32_t w = (e & 1) ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
                const uint32_t addr = A ^ (128 * e + 16 * (e >> 1));
                asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(w) : "memory");
            }
        };
        auto transpose_v = [&](const uint8_t* vraw, uint8_t* vt) __attribute__((always_inline)) {
            u32x4 ra, rb;
            transpose_load(vraw, ra, rb);
            transpose_store(ra, rb, vt);
        };
        f32x16 acc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[db][i] = 0.0f;
        float m_run = kNegBig;
        float l_run = 0.0f;

        if (t_begin < t_end) {
            // Ping-pong schedule.  Every wave runs the element sequence
            //   M(-1) | V(0) | M(0) | V(1) | M(1) | ... | M(n-1)
            // with a workgroup barrier after each element, where for tile t = t0 + j
            //   V(j): softmax of S(t) -> P(t); this wave's share of K(t+2) and of V^T(t+2)
            //         (or of the V rows of t+2, into the staging buffer) is loaded; if
            //         V(t+1) was staged, this wave transposes its own rows into V^T(t+1)
            //   M(j): O += V(t) P(t) from V^T(t); S(t+1) = K(t+1) Q^T
            // Waves 4..7 run one element behind waves 0..3 (one extra barrier up front,
            // waves 0..3 take theirs at the end).  Wave w and wave w+4 share a SIMD, so
            // while one of them is in an MFMA element the other is in a VALU element.
            // A wave reads the staging buffer's rows it loaded itself before loading the
            // next staged tile over them, so staging needs no barrier; four stages of K and
            // V^T keep each tile until both halves of the workgroup are done with it.
            const bool late = wv >= 4;
            int kn[2];
            int kr[7] = {0, 0, 0, 0, 0, 0, 0};   // map lookups of the next tile to load
            // V of tile t0: V^T straight into s_t0, or rows into s_t2 (free until tile
            // t0+2 loads) transposed below; V of tile t0+1: V^T into s_t1 or rows into s_raw
            keys_fetch(t_begin, kr);
            const bool vt0 = use_vt && whole_tile(t_begin);
            const int k00 = tile_k0(t_begin, kr);
            keys_finish(t_begin, kr, kn);
            issue_k(kn, s_k0);
            if (vt0) issue_vt(k00, s_t0); else issue_v(kn, s_t2);
            keys_fetch(t_begin + 1, kr);
            const bool vt1 = use_vt && whole_tile(t_begin + 1);
            const int k01 = tile_k0(t_begin + 1, kr);
            keys_finish(t_begin + 1, kr, kn);
            issue_k(kn, s_k1);
            if (vt1) issue_vt(k01, s_t1); else issue_v(kn, s_raw);
            raw_next = !vt1;
            keys_fetch(t_begin + 2, kr);
            __builtin_amdgcn_s_waitcnt(0);
            if (!vt0) transpose_v(s_t2, s_t0);
            __syncthreads();   // K(t0), K(t0+1), V^T(t0) and V(t0+1) are complete
            if (late) barrier_keep<0>();

            f32x16 st[2];
            bf16x8 pf[4];
            qk(s_k0, st);     // M(-1)
            barrier_keep<0>();

            auto elem_v = [&](int t, uint8_t* kdma, uint8_t* tdma, uint8_t* tnext) __attribute__((always_inline)) {
                // Over I_p the wave in its softmax element issues ahead of its partner's MFMA
                // stream (measured: the sparse launch 3 % faster); over a dense range the same
                // priority made the kernel 10 % slower, so there both waves keep priority 0.
                if (MODE != kDense) __builtin_amdgcn_s_setprio(1);
                // rows of tile t+2 from the lookups fetched one element ago; the lookups of
                // tile t+3 go out before the loads of tile t+2, so those stay the newest
                // memory operations (barrier_keep<4> leaves exactly them in flight).  This
                // wave's rows of V(t+1) (landed by the end of its previous M element) are
                // read early, so the LDS round trip hides behind the softmax.
                const bool vt2 = use_vt && whole_tile(t + 2);
                const int k02 = tile_k0(t + 2, kr);
                keys_finish(t + 2, kr, kn);
                keys_fetch(t + 3, kr);
                issue_k(kn, kdma);
                const bool raw1 = raw_next;   // V(t+1) sits row-major in s_raw
                // Over I_p the transpose is split around the softmax (the LDS round trip hides
                // behind it; in key-list mode every tile is staged).  Over a dense range a
                // tile is staged only when no V^T is given: there the transpose is one block,
                // so the other tiles carry no registers for it (the compiler set them to zero
                // on every tile, 8 VALU moves) -- the sparse kernels have no registers to spare
                // for the block's address arithmetic.
                constexpr bool kSplitTranspose = MODE != kDense;
                u32x4 ra, rb;
                if (kSplitTranspose) {
                    if (raw1) transpose_load(s_raw, ra, rb);
                } else if (__builtin_expect(raw1, 0)) {
                    transpose_v(s_raw, tnext);
                }
                if (vt2) {
                    issue_vt(k02, tdma);
                } else {
                    // this wave's rows of s_raw are read before its DMA overwrites them
                    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
                    issue_v(kn, s_raw);
                }
                raw_next = !vt2;
                const int valid_here = n_keys - t * 64;
                // only the last tile of a key range is short: a real, rare branch (if-converted,
                // its 32 compares and selects ran on every tile)
                if (__builtin_expect(valid_here < 64, 0)) {
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int r = kb * 32 + 8 * (i >> 2) + 4 * hf + (i & 3);
                            if (vt_row(r) >= valid_here) st[kb][i] = -INFINITY;
                        }
                }
                // max and sum as 4 independent chains each (short dependency chains)
                float mq[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    mq[c] = fmaxf(st[c >> 1][8 * (c & 1)], st[c >> 1][8 * (c & 1) + 1]);
#pragma unroll
                    for (int j = 2; j < 8; ++j) mq[c] = fmaxf(mq[c], st[c >> 1][8 * (c & 1) + j]);
                }
                float mx = fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3]));
                mx = fmaxf(mx, xhalf(mx));
                const float mc = mx * a.sl2;
                const bool need = mc > m_run + kSlack;
                // a rare, real branch: if-converted, the 64 multiplies ran on every tile
                if (__builtin_expect(__any(need), 0)) {
                    const float m_new = need ? mc : m_run;
                    const float alpha = fast_exp2(m_run - m_new);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
                    l_run *= alpha;
                    m_run = m_new;
                }
                const float mneg = -m_run;
                float ps[4];
#pragma unroll
                for (int kc = 0; kc < 4; ++kc)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const float pv = fast_exp2(fmaf(st[kc >> 1][8 * (kc & 1) + j], a.sl2, mneg));
                        ps[kc] = j == 0 ? pv : ps[kc] + pv;   // (0 + pv would be one more add)
                        pf[kc][j] = static_cast<__bf16>(pv);
                    }
                l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
                if (kSplitTranspose && raw1) transpose_store(ra, rb, tnext);
                if (MODE != kDense) __builtin_amdgcn_s_setprio(0);
                barrier_keep<4>();   // the loads of tile t+2 may stay in flight
            };
            auto elem_m = [&](const uint8_t* tread, const uint8_t* kread) __attribute__((always_inline)) {
                // O^T += V^T P^T, then S(t+1) = K(t+1) Q^T, as one stream of 32 MFMAs whose
                // LDS fragments (16 of V^T, then 16 of K) are read through a rolling window of
                // 4: each read is issued 4 MFMAs ahead of the one it feeds
                auto frag = [&](int j) __attribute__((always_inline)) {
                    if (j < 16) {   // V^T fragment: key chunk j / 4, head-dim block j % 4
                        return *reinterpret_cast<const bf16x8*>(tread + (j & 3) * 4096 + (tofs ^ (32 * ((j >> 2) ^ (j & 3)))));
                    }
                    const int c = j - 16;   // K fragment: key block c / 8, head-dim chunk c % 8
                    return *reinterpret_cast<const bf16x8*>(kread + (c >> 3) * 32 * kRowB + (kofs ^ (32 * (c & 7))));
                };
                bf16x8 w[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) w[j] = frag(j);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int i = 0; i < 16; ++i) st[kb][i] = 0.0f;
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const bf16x8 cur = w[j & 3];
                    if (j + 4 < 32) w[j & 3] = frag(j + 4);
                    if (j < 16) {
                        acc[j & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, pf[j >> 2], acc[j & 3], 0, 0, 0);
                    } else {
                        const int c = j - 16;
                        st[c >> 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cur, qf[c & 7], st[c >> 3], 0, 0, 0);
                    }
                }
                if (MODE != kDense) {
                    // over I_p the scheduler otherwise places each fragment read right before
                    // its MFMA, which then waits for the LDS round trip: keep 4 reads ahead
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // 4 LDS reads
#pragma unroll
                    for (int j = 0; j < 28; ++j) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // the last 4 MFMAs
                }
                barrier_keep<0>();   // this wave's loads of the next tile have landed
            };
            // tile t0 + j: K in s_k[j % 4], V^T in s_t[j % 4]
            for (int t = t_begin; t < t_end; t += 4) {
                elem_v(t, s_k2, s_t2, s_t1);
                elem_m(s_t0, s_k1);
                if (t + 1 < t_end) {
                    elem_v(t + 1, s_k3, s_t3, s_t2);
                    elem_m(s_t1, s_k2);
                }
                if (t + 2 < t_end) {
                    elem_v(t + 2, s_k0, s_t0, s_t3);
                    elem_m(s_t2, s_k3);
                }
                if (t + 3 < t_end) {
                    elem_v(t + 3, s_k1, s_t1, s_t0);
                    elem_m(s_t3, s_k0);
                }
            }
            if (!late) barrier_keep<0>();
            __builtin_amdgcn_s_waitcnt(0);   // drain the loads past the split before LDS is reused
        }

        // ---- epilogue: normalised rows in bf16 (one split) or unnormalised fp32 partials.
        // Each wave stages its 32 rows in LDS, then stores whole rows: bf16 rows (256 B, chunk
        // c of row i at slot c ^ (i & 15)) 4 per instruction, fp32 rows (512 B, chunk c at
        // slot c ^ (i & 31)) 2 per instruction.  Stored straight from the accumulator layout,
        // every instruction would write 16-byte pieces of 32 different rows, which drains
        // several times slower.  The loop ended on a barrier that every wave reached with its
        // loads landed, so no tile buffer is in use any more.
        const float l_tot = l_run + xhalf(l_run);
        const int row0 = u.qt * kD128Rows + wv * 32;   // logical row of this wave's row 0
        if (n_splits == 1) {
            uint8_t* stage = (wv < 2 ? s_t0 : wv < 4 ? s_t1 : wv < 6 ? s_t2 : s_t3) + (wv & 1) * 8192;
            const float sc = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            // The lane id goes through an empty asm, so the per-lane offsets below are formed
            // here rather than hoisted above the tile loop (where they would stay live and spill).
            int el = lane;
            asm volatile("" : "+v"(el));
            // chunk c of row i at 256 i + 16 (c ^ (i & 15)) = (256 i + 16 (i & 15)) ^ 16 c
            const int wbase = (el & 31) * 256 + 16 * (el & 15) + 8 * (el >> 5);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    // d = 32 db + 8 qd + 4 hf .. +3: half of 16-byte chunk 4 db + qd
                    u32x2 w;
                    w[0] = pack_bf16x2(acc[db][4 * qd + 0] * sc, acc[db][4 * qd + 1] * sc);
                    w[1] = pack_bf16x2(acc[db][4 * qd + 2] * sc, acc[db][4 * qd + 3] * sc);
                    *reinterpret_cast<u32x2*>(stage + (wbase ^ (16 * (4 * db + qd)))) = w;
                }
            const int cc = el & 15;
            // row i = 4k + lane/16: (i & 15) = 4 (k & 3) + lane/16
            const int rbase = 256 * (el >> 4) + ((16 * cc) ^ (16 * (el >> 4)));
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = 4 * k + (el >> 4);
                const int pr = row0 + i;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stage + 1024 * k + (rbase ^ (64 * (k & 3))));
                if (pr < rows_all) {
                    const int rr = pr / a.Gq;
                    const int hh = g * a.Gq + pr % a.Gq;
                    uint16_t* orow = static_cast<uint16_t*>(a.o) + b * a.osb + hh * a.osh + static_cast<int64_t>(rr) * a.osr;
                    *reinterpret_cast<u32x4*>(orow + 8 * cc) = pr < rows_valid ? v : u32x4{0u, 0u, 0u, 0u};
                }
            }
        } else {
            uint8_t* stage = wv == 0 ? s_t0 : wv == 1 ? s_t1 : wv == 2 ? s_t2 : wv == 3 ? s_t3 :
                             wv == 4 ? s_k0 : wv == 5 ? s_k1 : wv == 6 ? s_k2 : s_k3;
            int el = lane;
            asm volatile("" : "+v"(el));
            const int i0 = el & 31;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qd = 0; qd < 4; ++qd) {
                    // d = 32 db + 8 qd + 4 hf .. +3: 16-byte chunk 8 db + 2 qd + hf of row i0
                    const int c = 8 * db + 2 * qd + (el >> 5);
                    const f32x4 w = {acc[db][4 * qd + 0], acc[db][4 * qd + 1], acc[db][4 * qd + 2], acc[db][4 * qd + 3]};
                    *reinterpret_cast<f32x4*>(stage + 512 * i0 + 16 * (c ^ i0)) = w;
                }
            const int64_t pidx0 = d128_part_index(a, nqt_max, n_splits, b, g, u.split, row0);
            const int cc = el & 31;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const int i = 2 * k + (el >> 5);
                const f32x4 v = *reinterpret_cast<const f32x4*>(stage + 512 * i + 16 * (cc ^ i));
                if (row0 + i < rows_valid) *reinterpret_cast<f32x4*>(a.part_o + (pidx0 + i) * 128 + 4 * cc) = v;
            }
        }
        // softmax statistics, one lane per row
        const int r = p / a.Gq;
        const int h = g * a.Gq + p % a.Gq;
        if (hf == 0) {
            if (n_splits == 1) {
                if (a.lse && p < rows_all)
                    a.lse[(static_cast<int64_t>(b) * a.Hq + h) * a.nq_max + r] =
                        row_ok && l_tot > 0.0f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
            } else if (row_ok) {
                const int64_t idx = d128_part_index(a, nqt_max, n_splits, b, g, u.split, p);
                a.part_ml[idx * 2 + 0] = m_run;
                a.part_ml[idx * 2 + 1] = l_tot;
            }
        }
    }
}

}  // namespace

int d128_slots() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, attn_d128_kernel<kSparseLds>, 512, 0) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        int slots = cus * per_cu;
        slots = slots < kD128MaxSlots ? slots : kD128MaxSlots;
        cached[dev] = slots / 8 * 8 > 0 ? slots / 8 * 8 : 8;
    }
    return cached[dev];
}

hipError_t launch_attn_bf16_d128(const AttnArgs& args, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.slots));
    AttnArgs a = args;
    // V^T serves the tiles of consecutive keys when every such tile starts on a 16-byte
    // chunk: L a multiple of 8, and in I_p blocks of whole 64-key tiles and P a multiple
    // of 8 (then the tiles of [P, L) start at P + 64 i too).  Otherwise V rows serve all.
    if (a.vt) {
        const bool ok = a.L % 8 == 0 && (!a.sparse || (sparse_map_in_lds(a) && a.bs % 64 == 0 && a.P % 8 == 0));
        if (!ok) a.vt = nullptr;
    }
    if (!a.sparse) hipLaunchKernelGGL(attn_d128_kernel<kDense>, grid, dim3(512), 0, stream, a);
    else if (sparse_map_in_lds(a) && a.blk_per_head)
        hipLaunchKernelGGL((attn_d128_kernel<kSparseLds, true>), grid, dim3(512), 0, stream, a);
    else if (sparse_map_in_lds(a)) hipLaunchKernelGGL(attn_d128_kernel<kSparseLds>, grid, dim3(512), 0, stream, a);
    else hipLaunchKernelGGL(attn_d128_kernel<kSparseList>, grid, dim3(512), 0, stream, a);
    return hipGetLastError();
}

}  // namespace fdl
