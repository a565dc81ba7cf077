"""Edge cases of every entry point on the GPU, each checked against the fp64 oracle."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import focus_oracle as O
from parity import assert_close, assert_selection, valid

pytestmark = pytest.mark.gpu

DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def F():
    import long_context_diffusion_amd as lib
    return lib


def rand_qkv(seed, B, Hq, Hkv, L, d, dtype, sigma=0.125, q_rows=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    q = torch.randn((B, Hq, q_rows or L, d), generator=g, device=DEV) * sigma
    k = torch.randn((B, Hkv, L, d), generator=g, device=DEV) * sigma
    v = torch.randn((B, Hkv, L, d), generator=g, device=DEV) * sigma
    return q.to(dtype), k.to(dtype), v.to(dtype)


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def dkey(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


# ------------------------------------------------------------------ PCGI

def run_pcgi_case(conf, mask, n_t, rho, w):
    conf_t = torch.from_numpy(np.ascontiguousarray(conf, dtype=np.float32)).to(DEV)
    mask_t = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).to(DEV)
    B, L = conf.shape
    k = F().focus_count(n_t, rho)
    nq_max = max(min(k * w, L), 1)
    focus, n_focus, active, n_active = F().pcgi_select(conf_t, mask_t, n_t, rho, w, k_cap=max(k, 1),
                                                       nq_max=nq_max)
    torch.cuda.synchronize()
    for b in range(B):
        f_o = O.pcgi_focus(conf[b], mask[b].astype(bool), k)
        a_o = O.window_active(f_o, w, L)
        assert int(n_focus[b]) == len(f_o) and int(n_active[b]) == len(a_o)
        assert list(focus[b, : len(f_o)].cpu().numpy()) == list(f_o)
        assert np.all(focus[b, len(f_o):].cpu().numpy() == -1)
        assert list(active[b, : len(a_o)].cpu().numpy()) == list(a_o)
        assert np.all(active[b, len(a_o):].cpu().numpy() == -1)


def test_pcgi_hand_fixture():
    for case in json.load(open(os.path.join(GOLDEN, "pcgi_window_hand.json")))["cases"]:
        L = case["L"]
        mask = np.zeros((1, L), dtype=np.uint8)
        mask[0, case["mask"]] = 1
        conf = np.zeros((1, L), dtype=np.float32)
        for i, c in case["conf"].items():
            conf[0, int(i)] = c
        for w in case["windows"]:
            run_pcgi_case(conf, mask, case["n_t"], case["rho"], int(w))


@pytest.mark.parametrize("L,frac,n_t,rho,w", [
    (64, 0.5, 4, 2.0, 8),          # rank path, heavy ties
    (1100, 0.9, 40, 2.0, 9),       # ~990 candidates: rank path with many keys per slice
    (3000, 0.9, 16, 2.0, 33),      # 2700 candidates: radix select over LDS keys
    (20000, 0.6, 20, 2.0, 8),      # 12000 candidates: radix select over global keys
    (5000, 0.001, 30, 2.0, 7),     # fewer masked slots than k
    (777, 0.3, 0, 2.0, 5),         # k = 0
    (500, 0.4, 3, 1.5, 1200),      # windows wider than the sequence
])
def test_pcgi_paths_with_ties(L, frac, n_t, rho, w):
    rng = np.random.default_rng(L)
    B = 3
    mask = (rng.random((B, L)) < frac).astype(np.uint8)
    conf = (rng.integers(0, 16, size=(B, L)) / 16.0).astype(np.float32)   # many exact ties
    conf[1] = -conf[1]                                                    # negative values
    conf[2, ::7] = -0.0                                                   # -0.0 ties with +0.0
    run_pcgi_case(conf, mask, n_t, rho, w)


# ------------------------------------------------------------------ attention

def gpu_sparse(q, k, v, P, sinks, blocks, bs, q_idx=None, n_q=None, nq_max=None):
    return F().sparse_attention(q, k, v, P, sinks, blocks, bs, q_idx=q_idx, n_q=n_q, nq_max=nq_max,
                                want_lse=True)


@pytest.mark.parametrize("dtype,d,Hq,Hkv", [(torch.float32, 64, 4, 4), (torch.bfloat16, 128, 6, 2),
                                             (torch.bfloat16, 64, 3, 1)])
def test_sparse_equals_dense_when_nothing_is_pruned(dtype, d, Hq, Hkv):
    B, L, P, bs = 2, 700, 640, 64
    q, k, v = rand_qkv(1, B, Hq, Hkv, L, d, dtype)
    nb = -(-P // bs)
    blocks = torch.arange(nb, dtype=torch.int32, device=DEV).repeat(B, 1).contiguous()
    sinks = torch.tensor([[3, 650], [0, 699]], dtype=torch.int32, device=DEV)   # all covered
    o_s, l_s = gpu_sparse(q, k, v, P, sinks, blocks, bs)
    o_d, l_d = F().dense_attention(q, k, v)
    torch.cuda.synchronize()
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    assert float((o_s.float() - o_d.float()).abs().max()) <= tol
    assert float((l_s - l_d).abs().max()) <= 1e-4
    qf, kf, vf = f64(q), f64(k), f64(v)
    for b in range(B):
        ref, lref = O.dense_attention(qf[b], kf[b], vf[b], 1 / math.sqrt(d))
        assert_close(f64(o_s[b]), ref, dkey(dtype), "sparse(all) vs oracle dense")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sparse_key_set_edges(dtype):
    """Sinks inside selected blocks, in the generation region, -1 entries, duplicates,
    a short last block, and C larger than the number of blocks."""
    B, Hq, Hkv, L, P, d, bs = 3, 4, 2, 900, 850, 64, 64       # nb = 14, last block has 18 keys
    q, k, v = rand_qkv(2, B, Hq, Hkv, L, d, dtype, q_rows=L)
    nb = -(-P // bs)
    blocks = torch.tensor([[0, 5, 13, -1, -1, -1], [2, 3, 4, 7, 12, 13], [1, -1, -1, -1, -1, -1]],
                          dtype=torch.int32, device=DEV)
    sinks = torch.tensor([[1, 70, 320, 849, 860], [200, 200, 201, 448, -1], [-1, -1, 5, 64, 899]],
                         dtype=torch.int32, device=DEV)
    rows = torch.tensor([[0, 10, 500, 899, -1], [3, 4, 5, -1, -1], [850, -1, -1, -1, -1]],
                        dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([4, 3, 1], dtype=torch.int32, device=DEV)
    o, lse = gpu_sparse(q, k, v, P, sinks, blocks, bs, q_idx=rows, n_q=n_rows, nq_max=5)
    torch.cuda.synchronize()
    qf, kf, vf = f64(q), f64(k), f64(v)
    for b in range(B):
        nr = int(n_rows[b])
        ridx = rows[b, :nr].cpu().numpy()
        I_p = O.key_set(valid(sinks[b].cpu().numpy()), valid(blocks[b].cpu().numpy()), bs, P, L)
        ref, lref = O.sparse_attention(qf[b][:, ridx], kf[b], vf[b], I_p, 1 / math.sqrt(d))
        assert_close(f64(o[b, :, :nr]), ref, dkey(dtype), f"sparse edges b{b}")
        assert float(np.max(np.abs(lse[b, :, :nr].cpu().numpy() - lref))) <= 1e-4
        assert np.all(f64(o[b, :, nr:]) == 0) and np.all(np.isneginf(lse[b, :, nr:].cpu().numpy()))
    assert nb == 14


def test_empty_key_set_and_no_active_rows():
    B, Hq, Hkv, L, d = 1, 2, 2, 256, 64
    q, k, v = rand_qkv(3, B, Hq, Hkv, L, d, torch.bfloat16)
    # P = L, no blocks, no sinks: nothing to attend
    o, lse = gpu_sparse(q, k, v, L, None, None, 64, nq_max=8)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isinf(lse)) and torch.all(lse < 0)
    # zero valid rows: every row is padding
    n0 = torch.zeros((B,), dtype=torch.int32, device=DEV)
    idx = torch.full((B, 8), -1, dtype=torch.int32, device=DEV)
    o, lse = F().dense_attention(q, k, v, q_idx=idx, n_q=n0, nq_max=8)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isinf(lse))


def test_strided_query_layout():
    """Q given as a [B, H, L, d] view of a [B, L, H, d] tensor (row stride H*d)."""
    B, Hq, Hkv, L, d = 2, 4, 4, 300, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(4)
    q_blhd = (torch.randn((B, L, Hq, d), generator=g, device=DEV) * 0.125).to(torch.bfloat16)
    q = q_blhd.permute(0, 2, 1, 3)
    _, k, v = rand_qkv(5, B, Hq, Hkv, L, d, torch.bfloat16)
    o, lse = F().dense_attention(q, k, v)
    o_ref, _ = F().dense_attention(q.contiguous(), k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    qf, kf, vf = f64(q), f64(k), f64(v)
    ref, _ = O.dense_attention(qf[1], kf[1], vf[1], 1 / math.sqrt(d))
    assert_close(f64(o[1]), ref, "bf16", "strided Q")


def _vt_pair(call, v):
    """The call with V^T and without it must give bit-identical results."""
    o1, l1 = call(F().transpose_v(v))
    o2, l2 = call(None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), f"outputs differ with V^T: max {float((o1.float() - o2.float()).abs().max())}"
    assert torch.equal(l1, l2), "lse differs with V^T"
    return o1, l1


@pytest.mark.parametrize("L,nrows", [(1000, 37), (1000, 300), (1003, 37), (4096, 512)])
def test_dense_with_vt(L, nrows):
    """Dense key range from V^T (ragged last tile; L not a multiple of 8 ignores V^T)."""
    B, Hq, Hkv, d = 2, 8, 2, 128
    q, k, v = rand_qkv(L + nrows, B, Hq, Hkv, L, d, torch.bfloat16, sigma=1.0)
    g = torch.Generator().manual_seed(nrows)
    rows = torch.stack([torch.randperm(L, generator=g)[:nrows].sort().values for _ in range(B)]).to(torch.int32).to(DEV)
    n_q = torch.tensor([nrows, nrows - 5], dtype=torch.int32, device=DEV)
    o, lse = _vt_pair(lambda vt: F().dense_attention(q, k, v, vt=vt, q_idx=rows, n_q=n_q, nq_max=nrows), v)
    ref, _ = O.dense_attention(f64(q)[1][:, rows[1, :nrows - 5].cpu().numpy()], f64(k)[1], f64(v)[1], 1 / math.sqrt(d))
    assert_close(f64(o[1, :, :nrows - 5]), ref, "bf16", "dense with V^T")


@pytest.mark.parametrize("P,bs,blk,snk", [
    (4096, 128, [0, 3, 4, 17, 31], [3, 130, 1000, 4100]),     # whole tiles, a sinks tile
    (4000, 128, [1, 2, 30, 31], [5, 3990, 4001]),               # ragged last block selected
    (4000, 128, [0, 9], []),                                    # no sinks
    (4096, 64, [0, 1, 2, 63], [100, 200, 300]),
    (4032, 192, [0, 5, 20], [7]),
    (4001, 128, [0, 31], [2]),                                  # P not a multiple of 8: V rows only
])
def test_sparse_with_vt(P, bs, blk, snk):
    """Sparse key sets from V^T where tiles hold consecutive keys, V rows elsewhere."""
    B, Hq, Hkv, d = 1, 8, 4, 128
    L = P + 512
    q, k, v = rand_qkv(P + bs, B, Hq, Hkv, L, d, torch.bfloat16, sigma=1.0, q_rows=64)
    rows = torch.arange(0, 64, 2, dtype=torch.int32, device=DEV).reshape(1, -1)
    blocks = torch.tensor([blk], dtype=torch.int32, device=DEV)
    sinks = torch.tensor([snk], dtype=torch.int32, device=DEV) if snk else None
    o, lse = _vt_pair(lambda vt: F().sparse_attention(q, k, v, P, sinks, blocks, bs, vt=vt, q_idx=rows,
                                                      want_lse=True), v)
    I_p = O.key_set(np.array(snk, dtype=np.int64), np.array(blk, dtype=np.int64), bs, P, L)
    ref, _ = O.sparse_attention(f64(q)[0][:, rows[0].cpu().numpy()], f64(k)[0], f64(v)[0], I_p, 1 / math.sqrt(d))
    assert_close(f64(o[0]), ref, "bf16", "sparse with V^T")


def test_vt_strided_view():
    """V^T as a view into a wider buffer (d-row stride above L)."""
    B, Hq, Hkv, L, d = 1, 4, 4, 2048, 128
    q, k, v = rand_qkv(5, B, Hq, Hkv, L, d, torch.bfloat16, sigma=1.0, q_rows=40)
    wide = torch.zeros((B, Hkv, d, L + 64), dtype=torch.bfloat16, device=DEV)
    wide[..., :L] = v.transpose(2, 3)
    vt = wide[..., :L]
    o1, _ = F().dense_attention(q, k, v, vt=vt)
    o2, _ = F().dense_attention(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ------------------------------------------------------------------ sinks and blocks

@pytest.mark.parametrize("L", [1000, 40000])   # LDS selection, and the global-memory fallback
def test_sinks_and_blocks_small(L):
    B, Hq, Hkv, d = 2, 4, 2, 64
    P, bs = L - 37, 48
    q, k, _ = rand_qkv(6, B, Hq, Hkv, L, d, torch.bfloat16, sigma=1.0, q_rows=L)
    rows = torch.tensor([[0, 7, 8, 9, L - 1, -1], [100, 101, -1, -1, -1, -1]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([5, 2], dtype=torch.int32, device=DEV)
    _, lse = F().dense_attention(q, k, k, q_idx=rows, n_q=n_rows, nq_max=6)
    for n_sinks in (0, 1, 13):
        sinks, scores = F().sink_identify(q, k, lse, n_sinks, q_idx=rows, n_q=n_rows, nq_max=6, want_scores=True)
        torch.cuda.synchronize()
        qf, kf = f64(q), f64(k)
        for b in range(B):
            nr = int(n_rows[b])
            r = rows[b, :nr].cpu().numpy()
            _, lref = O.dense_attention(qf[b][:, r], kf[b], kf[b], 1 / math.sqrt(d))
            sc = O.sink_scores(qf[b][:, r], kf[b], lref, 1 / math.sqrt(d))
            assert_selection(sinks[b, :n_sinks].cpu().numpy(), O.sink_select(sc, n_sinks), sc, "sinks")
    nb = -(-P // bs)
    for C in (0, 5, nb, nb + 9):
        blocks, R, kbar = F().block_score_topc(q, k, P, bs, C, q_idx=rows, n_q=n_rows, nq_max=6,
                                               want_R=True, want_kbar=True)
        torch.cuda.synchronize()
        qf, kf = f64(q), f64(k)
        for b in range(B):
            nr = int(n_rows[b])
            r = rows[b, :nr].cpu().numpy()
            kb = O.block_means(kf[b], P, bs)
            assert np.array_equal(kbar[b].cpu().numpy(), kb.astype(np.float32))
            Rr = O.block_relevance(qf[b][:, r], kb, 1 / math.sqrt(d))
            assert_selection(blocks[b, :C].cpu().numpy(), O.top_blocks(Rr, C), Rr, f"blocks C={C}")
            assert np.all(blocks[b, min(C, nb):C].cpu().numpy() == -1)


@pytest.mark.parametrize("L,n_sinks", [(2000, 5), (32768, 16), (32768, 300), (33000, 7)])
def test_uniform_scores_pick_the_lowest_indices(L, n_sinks):
    """Zero queries give every key the same attention mass and every block the same
    relevance (exact ties): both selections must return the lowest positions.  The cases
    take the per-thread-maximum sink select (L <= 32768), its radix fallback when too
    many scores tie at the threshold (300 sinks), and the radix select (L > 32768)."""
    B, Hq, Hkv, d = 1, 4, 2, 64
    P, bs, C = L - 48, 64, 6
    _, k, _ = rand_qkv(11, B, Hq, Hkv, L, d, torch.bfloat16)
    q = torch.zeros((B, Hq, 8, d), dtype=torch.bfloat16, device=DEV)
    rows = torch.tensor([[0, 1, 2, 3, 4, 5, 6, 7]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([8], dtype=torch.int32, device=DEV)
    # lse of zero queries: log(L) for every row
    lse = torch.full((B, Hq, 8), math.log(L), dtype=torch.float32, device=DEV)
    sinks, scores = F().sink_identify(q, k, lse, n_sinks, q_idx=rows, n_q=n_rows, nq_max=8, want_scores=True)
    blocks, R, _ = F().block_score_topc(q, k, P, bs, C, q_idx=rows, n_q=n_rows, nq_max=8, want_R=True)
    torch.cuda.synchronize()
    sc = scores[0].cpu().numpy()
    assert np.all(sc == sc[0])
    assert list(sinks[0].cpu().numpy()) == list(range(n_sinks))
    assert np.all(R[0].cpu().numpy() == 0.0)
    assert list(blocks[0].cpu().numpy()) == list(range(C))


@pytest.mark.parametrize("nb", [1024, 1025, 2048, 2049, 3001])
def test_block_select_size_regimes(nb):
    """Block top-C at the edges of its three selection regimes: a rank over distinct keys
    (nb <= 1024), a radix select over LDS keys (nb <= 2048) and over the relevance in global
    memory (larger nb).  Random queries check the selection against the oracle; zero
    queries tie every block at R = 0, where the lowest indices must win."""
    B, Hq, Hkv, d, bs = 2, 4, 2, 64, 8
    P = nb * bs - 3                           # ragged last block
    L = P + 40
    q, k, _ = rand_qkv(nb, B, Hq, Hkv, L, d, torch.bfloat16, sigma=1.0, q_rows=16)
    rows = torch.tensor([[0, 3, 5, 9, 15], [2, 4, -1, -1, -1]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([5, 2], dtype=torch.int32, device=DEV)
    qf, kf = f64(q), f64(k)
    kb = [O.block_means(kf[b], P, bs) for b in range(B)]
    for C in (1, 37, nb // 3, nb - 1):
        blocks, R, _ = F().block_score_topc(q, k, P, bs, C, q_idx=rows, n_q=n_rows, nq_max=5, want_R=True)
        torch.cuda.synchronize()
        for b in range(B):
            r = rows[b, :int(n_rows[b])].cpu().numpy()
            Rr = O.block_relevance(qf[b][:, r], kb[b], 1 / math.sqrt(d))
            assert_selection(blocks[b].cpu().numpy(), O.top_blocks(Rr, C), Rr, f"nb={nb} C={C} b={b}")
    zq = torch.zeros_like(q)
    for C in (1, nb // 2):
        blocks, R, _ = F().block_score_topc(zq, k, P, bs, C, q_idx=rows, n_q=n_rows, nq_max=5, want_R=True)
        torch.cuda.synchronize()
        assert np.all(R.cpu().numpy() == 0.0)
        for b in range(B):
            assert list(blocks[b].cpu().numpy()) == list(range(C)), f"ties nb={nb} C={C} b={b}"


# ------------------------------------------------------------------ determinism and graphs

def _small_step(runner, conf, mask, qs, ks, vs):
    runner.sparse_step(conf, mask, qs, ks, vs)
    return [o.clone() for o in runner.out] + [runner.sinks.clone()] + [b.clone() for b in runner.blocks]


def _small_runner_and_inputs():
    from long_context_diffusion_amd.step import StepRunner
    from workloads import configs, synth
    wl = configs.CTX8K_MHA
    import dataclasses
    wl = dataclasses.replace(wl, layers=3, l_dense=1)
    conf, mask = synth.step_inputs(wl)
    qs, ks, vs = [], [], []
    for l in range(wl.layers):
        kk, vv = synth.make_kv(wl, l, DEV)
        ks.append(kk)
        vs.append(vv)
        qs.append(synth.make_q(wl, l, 0, DEV))
    run = StepRunner(B=wl.B, L=wl.L, P=wl.P, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, dtype=torch.bfloat16, n_t=wl.n_t,
                     rho=wl.rho, w=wl.w, bs=wl.bs, C=wl.C, n_sinks=wl.n_sinks, layers=wl.layers,
                     l_dense=wl.l_dense, scale=wl.scale, device=DEV)
    return run, torch.from_numpy(conf).to(DEV), torch.from_numpy(mask).to(DEV), qs, ks, vs


def test_repeat_runs_are_bit_identical():
    run, conf, mask, qs, ks, vs = _small_runner_and_inputs()
    first = _small_step(run, conf, mask, qs, ks, vs)
    for _ in range(2):
        again = _small_step(run, conf, mask, qs, ks, vs)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)


def test_graph_replays_match_eager():
    run, conf, mask, qs, ks, vs = _small_runner_and_inputs()
    eager = _small_step(run, conf, mask, qs, ks, vs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.sparse_step(conf, mask, qs, ks, vs)
    for rep in range(3):
        for o in run.out:             # eager work between replays: scribble over the outputs
            o.fill_(7.0)
        run.sinks.fill_(-5)
        for kb in run.kbar.values():  # and over the block means the second stream writes
            kb.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in run.out] + [run.sinks.clone()] + [b.clone() for b in run.blocks]
        for a, b in zip(eager, got):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
