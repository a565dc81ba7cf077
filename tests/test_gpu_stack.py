"""HIP path vs the fp64 oracle on the two 32K workloads, run as the benchmark runs them.

32K LLaDA-shaped stack: the whole 32-layer sparse step runs on the GPU
(StepRunner, the sequence bench.py times); the oracle then checks I_focus and
I_active exactly, the dense layers and sinks at layer l_dense on every active
row, and block top-C plus sparse attention on a sample of the deeper layers
(every row of those layers).  All 30 block selections are checked for form.

32K Dream-shaped batch of 4: the block-entry dense refresh of all 28 layers
(outputs checked on sampled rows of the first and last layer), then 7 sparse
steps with evolving confidence; every step's PCGI sets are checked exactly and
two steps are checked in full on sampled layers.
"""
import numpy as np
import pytest
import torch

import long_context_diffusion_amd as F
from workloads import configs, synth

pytestmark = pytest.mark.gpu


def _runner(wl, dev):
    from long_context_diffusion_amd.step import StepRunner
    return StepRunner(B=wl.B, L=wl.L, P=wl.P, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, dtype=synth.torch_dtype(wl),
                      n_t=wl.n_t, rho=wl.rho, w=wl.w, bs=wl.bs, C=wl.C, n_sinks=wl.n_sinks,
                      layers=wl.layers, l_dense=wl.l_dense, scale=wl.scale, device=dev)


class LazyQ:
    """Per-layer Q of one step, drawn when a layer asks for it (keeps HBM use bounded)."""

    def __init__(self, wl, step, dev):
        self.wl, self.step, self.dev = wl, step, dev

    def __getitem__(self, l):
        return synth.make_q(self.wl, l, self.step, self.dev)


def _check_step(wl, run, conf, mask, qget, kvget, layers_checked, tag):
    import gpu_cases
    from oracle import focus_oracle as O
    from parity import assert_close, assert_selection, valid

    actives = gpu_cases.check_pcgi(wl, conf, mask, run.focus, run.n_focus, run.active, run.n_active)
    out = {"max_err": 0.0, "max_rel": 0.0, "swaps": 0}
    for b in range(wl.B):
        act = actives[b]
        na = len(act)
        sinks_gpu = valid(run.sinks[b, : wl.n_sinks].cpu().numpy())
        for l in layers_checked:
            Q = synth.to_f64(qget(l)[b])
            K, V = (synth.to_f64(t[b]) for t in kvget(l))
            Qa = Q[:, act]
            if l < wl.l_dense:
                if l == wl.l_dense - 1:
                    o_ref, lse_ref = O.dense_attention(Qa, K, V, wl.scale)
                    e = assert_close(synth.to_f64(run.out[l][b, :, :na]), o_ref, wl.dtype, f"{tag} dense l{l}")
                    lerr = float(np.max(np.abs(run.lse[b, :, :na].cpu().numpy() - lse_ref)))
                    assert lerr <= gpu_cases.LSE_TOL, f"{tag} lse err {lerr:.3e}"
                    sc = O.sink_scores(Qa, K, lse_ref, wl.scale)
                    same = assert_selection(sinks_gpu, O.sink_select(sc, wl.n_sinks), sc, f"{tag} sinks b{b}")
                    out["swaps"] += 0 if same else 1
                else:
                    rows = np.sort(np.random.default_rng(l).choice(na, min(na, 64), replace=False))
                    o_ref, _ = O.dense_attention(Qa[:, rows], K, V, wl.scale)
                    e = assert_close(synth.to_f64(run.out[l][b][:, rows]), o_ref, wl.dtype, f"{tag} dense l{l}")
            else:
                R = O.block_relevance(Qa, O.block_means(K, wl.P, wl.bs), wl.scale)
                blk_gpu = run.blocks[l][b, : wl.C].cpu().numpy()
                same = assert_selection(blk_gpu, O.top_blocks(R, wl.C), R, f"{tag} blocks l{l} b{b}")
                out["swaps"] += 0 if same else 1
                I_p = O.key_set(sinks_gpu, valid(blk_gpu), wl.bs, wl.P, wl.L)
                o_ref, _ = O.sparse_attention(Qa, K, V, I_p, wl.scale)
                e = assert_close(synth.to_f64(run.out[l][b, :, :na]), o_ref, wl.dtype, f"{tag} sparse l{l}")
            out["max_err"] = max(out["max_err"], e[0])
            out["max_rel"] = max(out["max_rel"], e[1])
    return out


def _check_block_form(wl, run):
    for l in range(wl.l_dense, wl.layers):
        blk = run.blocks[l][:, : wl.C].cpu().numpy()
        for b in range(wl.B):
            v = blk[b][blk[b] >= 0]
            assert len(v) == min(wl.C, wl.nb) and np.all(np.diff(v) > 0) and v.max() < wl.nb


def test_ctx32k_stack_sparse_step():
    import gpu_cases
    wl = configs.CTX32K_STACK
    dev = "cuda"
    gpu_cases.log(f"case {wl.name}: drawing {wl.layers} layers")
    conf, mask = synth.step_inputs(wl)
    qs, ks, vs = [], [], []
    for l in range(wl.layers):
        k, v = synth.make_kv(wl, l, dev)
        ks.append(k)
        vs.append(v)
        qs.append(synth.make_q(wl, l, 0, dev))
    vts = [F.transpose_v(v) for v in vs]
    run = _runner(wl, dev)
    run.sparse_step(gpu_cases.to_dev(conf), gpu_cases.to_dev(mask), qs, ks, vs, vts=vts)
    torch.cuda.synchronize()
    gpu_cases.log("GPU step done; checking against the oracle")
    _check_block_form(wl, run)
    res = _check_step(wl, run, conf, mask, lambda l: qs[l], lambda l: (ks[l], vs[l]),
                      layers_checked=[0, 1, 2, 3, 17, 31], tag="32k")
    assert sorted(valid_sinks(run)) == sorted(synth.sink_positions(wl, 0).tolist())
    gpu_cases.log(f"{wl.name}: {res}")


def valid_sinks(run):
    s = run.sinks[0].cpu().numpy()
    return [int(x) for x in s if x >= 0]


def test_ctx32k_gqa_batch4_refresh():
    import gpu_cases
    from oracle import focus_oracle as O
    from parity import assert_close
    wl = configs.CTX32K_GQA_B4
    dev = "cuda"
    gpu_cases.log(f"case {wl.name}: block-entry refresh of {wl.layers} layers")
    run = _runner(wl, dev)
    q0 = LazyQ(wl, 0, dev)
    kept = {}
    for l in range(wl.layers):
        k, v = synth.make_kv(wl, l, dev)
        q = q0[l]
        o = torch.empty_like(q)
        F.dense_attention(q, k, v, vt=F.transpose_v(v), out=o, want_lse=False, scale=wl.scale,
                          workspace=run.workspace)
        if l in (0, wl.layers - 1):
            kept[l] = (q, k, v, o)
        else:
            del q, k, v, o
    torch.cuda.synchronize()
    res = 0.0
    for l, (q, k, v, o) in kept.items():
        for b in range(wl.B):
            rows = synth.sample_rows(wl.L, 48, 100 * l + b)
            Q = synth.to_f64(q[b][:, rows])
            K, V = synth.to_f64(k[b]), synth.to_f64(v[b])
            o_ref, _ = O.dense_attention(Q, K, V, wl.scale)
            e = assert_close(synth.to_f64(o[b][:, rows]), o_ref, wl.dtype, f"refresh l{l} b{b}")
            res = max(res, e[0])
    gpu_cases.log(f"{wl.name} refresh: max abs err {res:.3e}")


def test_ctx32k_gqa_batch4_sparse_steps():
    import gpu_cases
    wl = configs.CTX32K_GQA_B4
    dev = "cuda"
    run = _runner(wl, dev)
    kv = {}

    def kvget(l):
        if l not in kv:
            kv[l] = synth.make_kv(wl, l, dev)
        return kv[l]

    ks = [kvget(l)[0] for l in range(wl.layers)]
    vs = [kvget(l)[1] for l in range(wl.layers)]
    vts = [F.transpose_v(v) for v in vs]
    for t in range(1, wl.steps):
        gpu_cases.log(f"case {wl.name}: sparse step {t}")
        states = [synth.scenario(wl, b)[t] for b in range(wl.B)]
        conf = np.stack([c for _, c in states])
        mask = np.stack([m.astype(np.uint8) for m, _ in states])
        qt = LazyQ(wl, t, dev)
        run.sparse_step(gpu_cases.to_dev(conf), gpu_cases.to_dev(mask), qt, ks, vs, vts=vts)
        torch.cuda.synchronize()
        gpu_cases.check_pcgi(wl, conf, mask, run.focus, run.n_focus, run.active, run.n_active)
        _check_block_form(wl, run)
        if t in (1, wl.steps - 1):
            res = _check_step(wl, run, conf, mask, lambda l: qt[l], kvget, layers_checked=[1, 2, wl.layers - 1],
                              tag=f"step{t}")
            gpu_cases.log(f"{wl.name} step {t}: {res}")
