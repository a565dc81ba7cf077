"""GPU paths that the workloads do not reach, each against the fp64 oracle.

  * Index lists in any form: block and sink lists with -1 entries first or in between,
    repeated ids, descending order and out-of-range ids are taken as the set of their valid
    ids (the attention's key set is I_p of that set), on the bf16 d = 128 kernel (key map in
    LDS), its key-list variant (more than 1024 blocks or sinks) and the d = 64 / fp32 kernels.
  * The key-list variant of the bf16 d = 128 kernel at its own sizes: more than 1024 sinks,
    more than 1024 selected blocks.
  * fp32 inputs at head dim 128: dense and sparse attention, and the sink scores.
  * Sink identification without a log-sum-exp argument (the library computes it).
"""
import math

import numpy as np
import pytest
import torch

from oracle import focus_oracle as O
from parity import assert_close, assert_selection

pytestmark = pytest.mark.gpu

DEV = "cuda"


def F():
    import long_context_diffusion_amd as lib
    return lib


def log(msg):
    print(msg, flush=True)


def rand_qkv(seed, B, Hq, Hkv, L, d, dtype, q_rows, sigma=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn((B, Hq, q_rows, d), generator=g, device=DEV) * sigma
    k = torch.randn((B, Hkv, L, d), generator=g, device=DEV) * sigma
    v = torch.randn((B, Hkv, L, d), generator=g, device=DEV) * sigma
    return q.to(dtype), k.to(dtype), v.to(dtype)


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def dkey(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


def oracle_sparse(q, k, v, rows, sinks, blocks, bs, P, L, d, b):
    """The oracle on the set of valid ids of each list (the canonical reading of a list)."""
    snk = sorted({int(j) for j in sinks if 0 <= int(j) < L})
    nb = -(-P // bs)
    blk = sorted({int(c) for c in blocks if 0 <= int(c) < nb})
    I_p = O.key_set(np.array(snk, dtype=np.int64), np.array(blk, dtype=np.int64), bs, P, L)
    return O.sparse_attention(f64(q)[b][:, rows], f64(k)[b], f64(v)[b], I_p, 1 / math.sqrt(d))


@pytest.mark.parametrize("dtype,d,with_vt", [(torch.bfloat16, 128, True), (torch.bfloat16, 128, False),
                                             (torch.bfloat16, 64, False), (torch.float32, 64, False),
                                             (torch.float32, 128, False)])
def test_index_lists_in_any_form(dtype, d, with_vt):
    B, Hq, Hkv, P, bs = 4, 4, 2, 1280, 64       # nb = 20
    L = P + 192
    q, k, v = rand_qkv(31 + d, B, Hq, Hkv, L, d, dtype, q_rows=L, sigma=0.5)
    blocks = torch.tensor([[-1, 3, 7, 7, 19, -1],           # leading -1, a repeat, trailing -1
                           [12, 4, 9, -1, 0, 4],            # any order, -1 in between, a repeat
                           [25, -7, 2, 2, 2, 30],           # out-of-range ids
                           [-1, -1, -1, -1, -1, -1]], dtype=torch.int32, device=DEV)
    sinks = torch.tensor([[-1, 900, 5, 900, 1300],          # repeat, a sink in the generation region
                          [200, 100, -1, 250, 64],          # descending parts, one inside block 4
                          [L + 5, 3, -2, 3, 1279],
                          [-1, -1, 7, -1, -1]], dtype=torch.int32, device=DEV)
    rows = torch.tensor([[0, 9, 640, L - 1, 1300, 20], [1, 2, 3, -1, -1, -1], [50, 60, 70, 80, -1, -1],
                         [L - 2, -1, -1, -1, -1, -1]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([6, 3, 4, 1], dtype=torch.int32, device=DEV)
    vt = F().transpose_v(v) if with_vt else None
    o, lse = F().sparse_attention(q, k, v, P, sinks, blocks, bs, vt=vt, q_idx=rows, n_q=n_rows, nq_max=6,
                                  want_lse=True)
    torch.cuda.synchronize()
    worst = 0.0
    for b in range(B):
        nr = int(n_rows[b])
        r = rows[b, :nr].cpu().numpy()
        ref, lref = oracle_sparse(q, k, v, r, sinks[b].cpu().numpy(), blocks[b].cpu().numpy(), bs, P, L, d, b)
        err = assert_close(f64(o[b, :, :nr]), ref, dkey(dtype), f"lists b{b}")
        worst = max(worst, err[0])
        assert float(np.max(np.abs(lse[b, :, :nr].cpu().numpy() - lref))) <= 1e-4
        assert np.all(f64(o[b, :, nr:]) == 0)
    log(f"index lists {dtype} d={d} vt={with_vt}: max abs err {worst:.3e}")


@pytest.mark.parametrize("case", ["many_sinks", "many_blocks", "many_blocks_unsorted"])
def test_d128_key_list_variant(case):
    """bf16 d = 128 with more than 1024 sinks or selected blocks: the kernel reads the key
    list attn_prep writes instead of mapping the parts in LDS."""
    B, Hq, Hkv, d = 1, 8, 2, 128
    rng = np.random.default_rng(7)
    if case == "many_sinks":
        P, bs, L = 3968, 64, 4096
        blk = np.array([0, 5, 17, 61], dtype=np.int64)
        snk = np.sort(rng.choice(P, 1100, replace=False))
    else:
        P, bs, L = 4000, 2, 4160                              # nb = 2000
        blk = np.sort(rng.choice(P // bs, 1100, replace=False))
        snk = np.array([1, 77, 3999], dtype=np.int64)
    q, k, v = rand_qkv(5, B, Hq, Hkv, L, d, torch.bfloat16, q_rows=L, sigma=0.5)
    rows_np = np.sort(rng.choice(L, 150, replace=False)).astype(np.int32)
    rows = torch.from_numpy(rows_np).reshape(1, -1).to(DEV)
    blk_in = blk[::-1].copy() if case == "many_blocks_unsorted" else blk
    blocks = torch.from_numpy(blk_in.astype(np.int32)).reshape(1, -1).to(DEV)
    sinks = torch.from_numpy(snk.astype(np.int32)).reshape(1, -1).to(DEV)
    o, lse = F().sparse_attention(q, k, v, P, sinks, blocks, bs, vt=F().transpose_v(v), q_idx=rows,
                                  want_lse=True)
    torch.cuda.synchronize()
    ref, lref = oracle_sparse(q, k, v, rows_np, snk, blk, bs, P, L, d, 0)
    err = assert_close(f64(o[0]), ref, "bf16", f"key list {case}")
    assert float(np.max(np.abs(lse[0].cpu().numpy() - lref))) <= 1e-4
    log(f"d128 key list {case}: max abs err {err[0]:.3e}, rel {err[1]:.3e}")


def test_fp32_head_dim_128():
    """fp32 inputs, head dim 128: dense attention with lse, sparse attention, sink scores."""
    B, Hq, Hkv, P, d, bs = 2, 4, 2, 960, 128, 64
    L = P + 64
    q, k, v = rand_qkv(9, B, Hq, Hkv, L, d, torch.float32, q_rows=L, sigma=0.125)
    rows = torch.tensor([[0, 5, 6, 7, 500, 1000, L - 1], [8, 9, 10, 11, 12, -1, -1]], dtype=torch.int32,
                        device=DEV)
    n_rows = torch.tensor([7, 5], dtype=torch.int32, device=DEV)
    kw = dict(q_idx=rows, n_q=n_rows, nq_max=7)
    od, lse = F().dense_attention(q, k, v, **kw)
    sinks, scores = F().sink_identify(q, k, lse, 6, want_scores=True, **kw)
    blocks = torch.tensor([[0, 3, 14], [2, 9, 11]], dtype=torch.int32, device=DEV)
    os_, lse_s = F().sparse_attention(q, k, v, P, sinks, blocks, bs, want_lse=True, **kw)
    torch.cuda.synchronize()
    s = 1 / math.sqrt(d)
    for b in range(B):
        nr = int(n_rows[b])
        r = rows[b, :nr].cpu().numpy()
        Qa, K, V = f64(q)[b][:, r], f64(k)[b], f64(v)[b]
        o_ref, l_ref = O.dense_attention(Qa, K, V, s)
        assert_close(f64(od[b, :, :nr]), o_ref, "f32", f"fp32 d128 dense b{b}")
        assert float(np.max(np.abs(lse[b, :, :nr].cpu().numpy() - l_ref))) <= 1e-5
        sc = O.sink_scores(Qa, K, l_ref, s)
        rel = float(np.max(np.abs(scores[b].cpu().numpy() - sc) / np.maximum(sc, 1e-30)))
        assert rel < 1e-4, f"fp32 d128 sink scores rel err {rel:.3e}"
        assert_selection(sinks[b].cpu().numpy(), O.sink_select(sc, 6), sc, f"fp32 d128 sinks b{b}")
        I_p = O.key_set(sinks[b].cpu().numpy(), blocks[b].cpu().numpy(), bs, P, L)
        o_ref, _ = O.sparse_attention(Qa, K, V, I_p, s)
        assert_close(f64(os_[b, :, :nr]), o_ref, "f32", f"fp32 d128 sparse b{b}")


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_sink_identify_computes_lse(dtype, d):
    """Without an lse argument the library computes the log-sum-exp of the same rows itself:
    the same sinks and scores as with the lse of dense attention."""
    B, Hq, Hkv, L = 2, 8, 4, 2100
    q, k, _ = rand_qkv(13, B, Hq, Hkv, L, d, dtype, q_rows=L, sigma=0.5)
    rows = torch.tensor([[0, 1, 2, 900, 2099], [10, 20, 30, -1, -1]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([5, 3], dtype=torch.int32, device=DEV)
    kw = dict(q_idx=rows, n_q=n_rows, nq_max=5)
    _, lse = F().dense_attention(q, k, k, **kw)
    s1, sc1 = F().sink_identify(q, k, lse, 9, want_scores=True, **kw)
    s2, sc2 = F().sink_identify(q, k, None, 9, want_scores=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(sc1, sc2)
    for b in range(B):
        nr = int(n_rows[b])
        r = rows[b, :nr].cpu().numpy()
        _, l_ref = O.dense_attention(f64(q)[b][:, r], f64(k)[b], f64(k)[b], 1 / math.sqrt(d))
        sc = O.sink_scores(f64(q)[b][:, r], f64(k)[b], l_ref, 1 / math.sqrt(d))
        assert_selection(s2[b].cpu().numpy(), O.sink_select(sc, 9), sc, f"sinks without lse b{b}")
