"""Approximate-KV refresh and block-means refresh on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import focus_oracle as O

pytestmark = pytest.mark.gpu

DEV = "cuda"


def F():
    import long_context_diffusion_amd as lib
    return lib


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def _rand(g, shape, dtype):
    return torch.randn(shape, generator=g, device=DEV).to(dtype)


@pytest.mark.parametrize("dtype,d,with_vt", [(torch.float32, 64, False), (torch.bfloat16, 64, False),
                                             (torch.bfloat16, 128, True)])
def test_kv_and_means_refresh_small(dtype, d, with_vt):
    B, Hkv, L, P, bs = 2, 2, 304, 250, 16
    g = torch.Generator(device=DEV)
    g.manual_seed(d)
    k, v = _rand(g, (B, Hkv, L, d), dtype), _rand(g, (B, Hkv, L, d), dtype)
    rows = torch.tensor([[3, 4, 40, 47, 48, 199, 245, 249, 250, 290, 7, 8],
                         [0, 15, 16, -1, 100, 303, 9, 9, 9, 9, 9, 9]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([10, 6], dtype=torch.int32, device=DEV)   # entries past n_rows are ignored
    n_max = rows.shape[1]
    k_new, v_new = _rand(g, (B, Hkv, n_max, d), dtype), _rand(g, (B, Hkv, n_max, d), dtype)
    kf, vf = f64(k), f64(v)
    kbar = F().block_means(k, P, bs)
    kbar_old = kbar.clone()
    vt = F().transpose_v(v) if with_vt else None
    F().kv_refresh(rows, k_new, v_new, k, v, n_rows=n_rows, vt=vt)
    F().block_means_refresh(k, P, bs, rows, kbar, n_rows=n_rows)
    torch.cuda.synchronize()
    for b in range(B):
        n = int(n_rows[b])
        r = rows[b, :n].cpu().numpy()
        K2, V2 = O.kv_refresh(kf[b], vf[b], r, f64(k_new)[b][:, :n], f64(v_new)[b][:, :n])
        assert np.array_equal(f64(k)[b], K2) and np.array_equal(f64(v)[b], V2), f"cache b{b}"
        ref = O.block_means(K2, P, bs).astype(np.float32)
        assert np.array_equal(kbar[b].cpu().numpy(), ref), f"means b{b}"
        untouched = np.setdiff1d(np.arange(ref.shape[1]), O.refreshed_blocks(r, P, bs))
        assert torch.equal(kbar[b][:, untouched], kbar_old[b][:, untouched])
    if with_vt:
        assert torch.equal(vt, v.transpose(2, 3))


def test_refresh_at_32k_with_active_rows():
    """U(t) = I_active of the 32K step: the refreshed rows and V^T land where the oracle puts
    them, and the means equal the oracle's on every touched block and stay as they were
    elsewhere.  (Scoring and attention over a refreshed cache: test_cached_step_*.)"""
    import gpu_cases
    from workloads import configs, synth
    wl = configs.CTX32K_STACK
    conf, mask = synth.step_inputs(wl)
    _, _, active, n_active = gpu_cases.gpu_select(wl, conf, mask, DEV)
    k, v = synth.make_kv(wl, 2, DEV)
    vt = F().transpose_v(v)
    kbar = F().block_means(k, wl.P, wl.bs)
    kbar_old = kbar.clone()
    g = torch.Generator(device=DEV)
    g.manual_seed(32)
    n_max = active.shape[1]
    k_new = _rand(g, (wl.B, wl.Hkv, n_max, wl.d), k.dtype)
    v_new = _rand(g, (wl.B, wl.Hkv, n_max, wl.d), v.dtype)
    F().kv_refresh(active, k_new, v_new, k, v, n_rows=n_active, vt=vt)
    F().block_means_refresh(k, wl.P, wl.bs, active, kbar, n_rows=n_active)
    torch.cuda.synchronize()
    na = int(n_active[0])
    r = active[0, :na].cpu().numpy()
    kn, vn = f64(k_new[0]), f64(v_new[0])
    for j in np.linspace(0, na - 1, 16).astype(int):
        assert np.array_equal(f64(k[0][:, int(r[j])]), kn[:, j]) and np.array_equal(f64(v[0][:, int(r[j])]), vn[:, j])
        assert torch.equal(vt[0][:, :, int(r[j])], v[0][:, int(r[j])])
    touched = O.refreshed_blocks(r, wl.P, wl.bs)
    kf = f64(k[0])
    for blk in touched:
        lo, hi = blk * wl.bs, min((blk + 1) * wl.bs, wl.P)
        ref = O.block_means(kf[:, lo:hi], hi - lo, hi - lo)[:, 0].astype(np.float32)
        assert np.array_equal(kbar[0][:, blk].cpu().numpy(), ref), f"block {blk}"
    untouched = np.setdiff1d(np.arange(wl.nb), touched)
    assert torch.equal(kbar[0][:, untouched], kbar_old[0][:, untouched])
    gpu_cases.log(f"refresh: {na} rows, {len(touched)} prompt blocks touched")


# ------------------------------------------------------------------ the cached-means step

def _cached_setup(layers=3, l_dense=1):
    """The 8K workload cut to a few layers, its inputs, and per-layer new K/V rows."""
    import dataclasses
    from long_context_diffusion_amd.step import StepRunner
    from workloads import configs, synth
    wl = dataclasses.replace(configs.CTX8K_MHA, layers=layers, l_dense=l_dense)
    conf, mask = synth.step_inputs(wl)
    qs, ks, vs = [], [], []
    for l in range(wl.layers):
        k, v = synth.make_kv(wl, l, DEV)
        ks.append(k)
        vs.append(v)
        qs.append(synth.make_q(wl, l, 0, DEV))

    def runner():
        return StepRunner(B=wl.B, L=wl.L, P=wl.P, Hq=wl.Hq, Hkv=wl.Hkv, d=wl.d, dtype=torch.bfloat16,
                          n_t=wl.n_t, rho=wl.rho, w=wl.w, bs=wl.bs, C=wl.C, n_sinks=wl.n_sinks,
                          layers=wl.layers, l_dense=wl.l_dense, scale=wl.scale, device=DEV)
    run = runner()
    g = torch.Generator(device=DEV)
    g.manual_seed(88)
    shp = (wl.B, wl.Hkv, run.nq_max, wl.d)
    knew = [(torch.randn(shp, generator=g, device=DEV) * wl.sigma).to(torch.bfloat16) for _ in range(wl.layers)]
    vnew = [(torch.randn(shp, generator=g, device=DEV) * wl.sigma).to(torch.bfloat16) for _ in range(wl.layers)]
    return wl, run, runner, torch.from_numpy(conf).to(DEV), torch.from_numpy(mask).to(DEV), qs, ks, vs, knew, vnew, \
        (conf, mask)


def test_cached_step_against_full_means_and_oracle():
    """A cached-means step (each layer: refresh its cache rows, refresh the touched block means,
    score from the kept means, attend) gives bit for bit what a full-means step gives on the
    refreshed caches, and the oracle's refresh -> block means -> relevance -> top-C -> sparse
    attention on a sampled layer."""
    import gpu_cases
    from parity import assert_close, assert_selection, valid
    wl, run, runner, conf, mask, qs, ks, vs, knew, vnew, host = _cached_setup()
    ks0 = [synth_f64(k) for k in ks]
    vs0 = [synth_f64(v) for v in vs]
    vts = [F().transpose_v(v) for v in vs]
    run.init_means(ks)
    run.cached_step(conf, mask, qs, ks, vs, knew, vnew, vts=vts)
    torch.cuda.synchronize()
    # the full-means step on the caches the cached step left behind
    full = runner()
    full.sparse_step(conf, mask, qs, ks, vs, vts=vts)
    torch.cuda.synchronize()
    for l in range(wl.l_dense, wl.layers):
        assert torch.equal(run.kbar[l], full.kbar[l]), f"kept means differ from a full pass, layer {l}"
        assert torch.equal(run.blocks[l], full.blocks[l]), f"blocks differ, layer {l}"
    for l in range(wl.layers):
        assert torch.equal(run.out[l], full.out[l]), f"outputs differ, layer {l}"
    assert torch.equal(run.sinks, full.sinks)
    for l in range(wl.layers):
        assert torch.equal(vts[l], vs[l].transpose(2, 3)), f"V^T not refreshed, layer {l}"
    # oracle: the refreshed cache of the last layer and everything downstream of it
    conf_h, mask_h = host
    actives = gpu_cases.check_pcgi(wl, conf_h, mask_h, run.focus, run.n_focus, run.active, run.n_active)
    act = actives[0]
    na = len(act)
    l = wl.layers - 1
    K2, V2 = O.kv_refresh(ks0[l][0], vs0[l][0], act, f64(knew[l][0])[:, :na], f64(vnew[l][0])[:, :na])
    assert np.array_equal(K2, f64(ks[l][0])) and np.array_equal(V2, f64(vs[l][0])), "refreshed cache"
    Qa = synth_f64(qs[l])[0][:, act]
    kb = O.block_means(K2, wl.P, wl.bs)
    assert np.array_equal(run.kbar[l][0].cpu().numpy(), kb.astype(np.float32)), "kept means vs oracle"
    R = O.block_relevance(Qa, kb, wl.scale)
    blk = run.blocks[l][0, : wl.C].cpu().numpy()
    assert_selection(blk, O.top_blocks(R, wl.C), R, "cached blocks")
    I_p = O.key_set(valid(run.sinks[0].cpu().numpy()), valid(blk), wl.bs, wl.P, wl.L)
    o_ref, _ = O.sparse_attention(Qa, K2, V2, I_p, wl.scale)
    err = assert_close(synth_f64(run.out[l][0, :, :na]), o_ref, "bf16", "cached sparse O")
    gpu_cases.log(f"cached step: {na} refreshed rows, max abs err {err[0]:.3e}, rel {err[1]:.3e}")


def test_cached_step_graph_replays():
    """The cached step captured in a HIP graph: every replay (the refresh rewrites the same rows,
    so the step is repeatable) equals the eager step, with eager work between replays."""
    wl, run, runner, conf, mask, qs, ks, vs, knew, vnew, _ = _cached_setup()
    vts = [F().transpose_v(v) for v in vs]
    run.init_means(ks)
    run.cached_step(conf, mask, qs, ks, vs, knew, vnew, vts=vts)
    torch.cuda.synchronize()
    sparse = range(wl.l_dense, wl.layers)   # the dense layers select no blocks
    eager = [o.clone() for o in run.out] + [run.blocks[l].clone() for l in sparse] + [run.sinks.clone()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.cached_step(conf, mask, qs, ks, vs, knew, vnew, vts=vts)
    for rep in range(3):
        for o in run.out:
            o.fill_(5.0)
        for l in sparse:
            run.blocks[l].fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in run.out] + [run.blocks[l].clone() for l in sparse] + [run.sinks.clone()]
        for a, b in zip(eager, got):
            assert torch.equal(a, b), f"replay {rep} differs from the eager cached step"


def synth_f64(t):
    return f64(t)


@pytest.mark.parametrize("dtype,d,with_vt,bs", [(torch.float32, 64, False, 16), (torch.bfloat16, 64, False, 100),
                                                (torch.bfloat16, 128, True, 64), (torch.float32, 128, True, 128)])
def test_fused_refresh_equals_two_calls(dtype, d, with_vt, bs):
    """fdl_kv_refresh_means gives bit for bit the caches, V^T and means of fdl_kv_refresh
    followed by fdl_block_means_refresh, for ascending and unordered row lists with -1
    entries, rows inside and past the prompt, and ragged counts."""
    print(f"fused refresh dtype={dtype} d={d} vt={with_vt} bs={bs}", flush=True)
    B, Hkv, L, P = 2, 3, 520, 400
    g = torch.Generator(device=DEV)
    g.manual_seed(7 * d + bs)
    k, v = _rand(g, (B, Hkv, L, d), dtype), _rand(g, (B, Hkv, L, d), dtype)
    rows = torch.tensor([[3, 4, 40, 47, 48, 199, 245, 399, 400, 519, 7, 8, 150, 151],
                         [250, 0, 15, -1, 100, 303, 16, 17, 450, 9, 399, 398, 1, 2]], dtype=torch.int32, device=DEV)
    n_rows = torch.tensor([10, 14], dtype=torch.int32, device=DEV)
    n_max = rows.shape[1]
    k_new, v_new = _rand(g, (B, Hkv, n_max, d), dtype), _rand(g, (B, Hkv, n_max, d), dtype)
    kbar0 = F().block_means(k, P, bs)
    k1, v1, kb1 = k.clone(), v.clone(), kbar0.clone()
    vt1 = F().transpose_v(v1) if with_vt else None
    F().kv_refresh(rows, k_new, v_new, k1, v1, n_rows=n_rows, vt=vt1)
    F().block_means_refresh(k1, P, bs, rows, kb1, n_rows=n_rows)
    k2, v2, kb2 = k.clone(), v.clone(), kbar0.clone()
    vt2 = F().transpose_v(v2) if with_vt else None
    F().kv_refresh_means(rows, k_new, v_new, k2, v2, P, bs, kb2, n_rows=n_rows, vt=vt2)
    torch.cuda.synchronize()
    assert torch.equal(k1, k2) and torch.equal(v1, v2)
    assert torch.equal(kb1, kb2), "means"
    if with_vt:
        assert torch.equal(vt1, vt2)
    # and both equal a full pass over the refreshed keys
    assert torch.equal(kb2, F().block_means(k2, P, bs))
