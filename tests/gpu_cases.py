"""Shared runners for the GPU parity tests: one step through the C ABI, then the oracle.

The HIP path and the oracle receive the same arrays: inputs are drawn once on
the GPU by ``workloads.synth`` and copied to the host (exact fp64 upcast) for
the oracle.  Nothing the oracle compares against comes from the HIP path
except the index sets used for the output comparison, and those are first
checked against the oracle's own sets.
"""
from __future__ import annotations

import numpy as np
import torch

import long_context_diffusion_amd as F
from oracle import focus_oracle as O
from parity import assert_close, assert_exact_set, assert_selection, valid
from workloads import synth

LSE_TOL = 1e-4


def log(msg):
    print(msg, flush=True)


def to_dev(a, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def gpu_select(wl, conf, mask, device="cuda"):
    """PCGI through the library; k and the active-row capacity are the library's own."""
    return F.pcgi_select(to_dev(conf, device), to_dev(mask, device), wl.n_t, wl.rho, wl.w)


def check_pcgi(wl, conf, mask, focus, n_focus, active, n_active):
    """Exact I_focus and I_active for every sequence; returns the oracle's active sets."""
    focus, n_focus = focus.cpu().numpy(), n_focus.cpu().numpy()
    active, n_active = active.cpu().numpy(), n_active.cpu().numpy()
    actives = []
    k_o = O.focus_count(wl.n_t, wl.rho)
    for b in range(wl.B):
        f_o = O.pcgi_focus(conf[b], mask[b], k_o)
        a_o = O.window_active(f_o, wl.w, wl.L)
        assert n_focus[b] == len(f_o) and n_active[b] == len(a_o)
        assert_exact_set(focus[b, : n_focus[b]], f_o, f"I_focus[{b}]")
        assert np.all(focus[b, n_focus[b]:] == -1)
        assert_exact_set(active[b, : n_active[b]], a_o, f"I_active[{b}]")
        assert np.all(active[b, n_active[b]:] == -1)
        actives.append(a_o)
    return actives


def one_layer_step(wl, layer=0, step=0, device="cuda", check_refresh_rows=64, seed=0):
    """Runs PCGI, dense-on-active + lse, sinks, block top-C and sparse attention for one
    layer on the GPU, and checks every output against the oracle."""
    conf, mask = synth.step_inputs(wl, step)
    K, V = synth.make_kv(wl, layer, device)
    Q = synth.make_q(wl, layer, step, device)
    focus, n_focus, active, n_active = gpu_select(wl, conf, mask, device)
    kw = dict(q_idx=active, n_q=n_active, nq_max=active.shape[1], scale=wl.scale)
    VT = F.transpose_v(V)   # read by the bf16 d = 128 path, ignored by the others
    Od, lse = F.dense_attention(Q, K, V, vt=VT, **kw)
    sinks, scores = F.sink_identify(Q, K, lse, wl.n_sinks, want_scores=True, **kw)
    blocks, R, kbar = F.block_score_topc(Q, K, wl.P, wl.bs, wl.C, want_R=True, want_kbar=True, **kw)
    # the same scoring from means computed ahead by fdl_block_means (no keys passed)
    kbar_ahead = F.block_means(K, wl.P, wl.bs)
    blocks_ahead, R_ahead, _ = F.block_score_topc(Q, None, wl.P, wl.bs, wl.C, kbar=kbar_ahead, L=wl.L,
                                                  want_R=True, **kw)
    Os, lse_s = F.sparse_attention(Q, K, V, wl.P, sinks, blocks, wl.bs, vt=VT, want_lse=True, **kw)
    refresh = None
    if check_refresh_rows:
        refresh, _ = F.dense_attention(Q, K, V, vt=VT, scale=wl.scale, want_lse=False)
    # without V^T every tile transposes V rows on chip: the same values reach the MFMAs
    Od_rows, lse_rows = F.dense_attention(Q, K, V, **kw)
    Os_rows, lse_s_rows = F.sparse_attention(Q, K, V, wl.P, sinks, blocks, wl.bs, want_lse=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(Od, Od_rows) and torch.equal(lse, lse_rows), "dense attention differs without V^T"
    assert torch.equal(Os, Os_rows) and torch.equal(lse_s, lse_s_rows), "sparse attention differs without V^T"

    actives = check_pcgi(wl, conf, mask, focus, n_focus, active, n_active)
    assert torch.equal(kbar_ahead, kbar) and torch.equal(R_ahead, R) and torch.equal(blocks_ahead, blocks), \
        "scoring from precomputed block means differs"
    Kf, Vf, Qf = synth.to_f64(K), synth.to_f64(V), synth.to_f64(Q)
    res = {"max_err": 0.0, "max_rel": 0.0, "set_swaps": 0}
    n_act = n_active.cpu().numpy()

    def note(err_rel):
        res["max_err"] = max(res["max_err"], err_rel[0])
        res["max_rel"] = max(res["max_rel"], err_rel[1])

    for b in range(wl.B):
        act = actives[b]
        na = len(act)
        Qa = Qf[b][:, act]
        # dense attention on the active rows (layers 1..l_dense)
        o_ref, lse_ref = O.dense_attention(Qa, Kf[b], Vf[b], wl.scale)
        note(assert_close(synth.to_f64(Od[b, :, :na]), o_ref, wl.dtype, f"dense-active O[{b}]"))
        lerr = float(np.max(np.abs(lse[b, :, :na].cpu().numpy() - lse_ref)))
        assert lerr <= LSE_TOL, f"lse[{b}] err {lerr:.3e}"
        assert np.all(synth.to_f64(Od[b, :, na:]) == 0) and np.all(np.isneginf(lse[b, :, na:].cpu().numpy()))
        # sinks
        sc_ref = O.sink_scores(Qa, Kf[b], lse_ref, wl.scale)
        s_ref = O.sink_select(sc_ref, wl.n_sinks)
        same = assert_selection(sinks[b].cpu().numpy(), s_ref, sc_ref, f"I_sink[{b}]")
        res["set_swaps"] += 0 if same else 1
        sc_gpu = scores[b].cpu().numpy().astype(np.float64)
        s_err = float(np.max(np.abs(sc_gpu - sc_ref) / np.maximum(sc_ref, 1e-30)))
        res["sink_score_rel_err"] = max(res.get("sink_score_rel_err", 0.0), s_err)
        assert s_err < 1e-3, f"sink scores rel err {s_err:.3e}"
        # block means, relevance, top-C
        kb_ref = O.block_means(Kf[b], wl.P, wl.bs)
        assert np.array_equal(kbar[b].cpu().numpy(), kb_ref.astype(np.float32)), "block means not exact"
        R_ref = O.block_relevance(Qa, kb_ref, wl.scale)
        R_gpu = R[b].cpu().numpy()
        # 8-term partial dot products run in fp32, everything above them in fp64
        r_err = float(np.max(np.abs(R_gpu - R_ref)) / np.max(np.abs(R_ref)))
        res["R_rel_err"] = max(res.get("R_rel_err", 0.0), r_err)
        assert r_err <= 1e-6, f"relevance rel err {r_err:.3e}"
        c_ref = O.top_blocks(R_ref, wl.C)
        same = assert_selection(blocks[b].cpu().numpy(), c_ref, R_ref, f"blocks[{b}]")
        res["set_swaps"] += 0 if same else 1
        # sparse attention over I_p built from the GPU's (checked) sets
        I_p = O.key_set(valid(sinks[b].cpu().numpy()), valid(blocks[b].cpu().numpy()), wl.bs, wl.P, wl.L)
        os_ref, lse_s_ref = O.sparse_attention(Qa, Kf[b], Vf[b], I_p, wl.scale)
        note(assert_close(synth.to_f64(Os[b, :, :na]), os_ref, wl.dtype, f"sparse O[{b}]"))
        lerr = float(np.max(np.abs(lse_s[b, :, :na].cpu().numpy() - lse_s_ref)))
        assert lerr <= LSE_TOL, f"sparse lse[{b}] err {lerr:.3e}"
        assert np.all(synth.to_f64(Os[b, :, na:]) == 0)
        # block-entry refresh: every row attends to every key (row sample)
        if refresh is not None:
            rows = synth.sample_rows(wl.L, check_refresh_rows, seed + b)
            r_ref, _ = O.dense_attention(Qf[b][:, rows], Kf[b], Vf[b], wl.scale)
            note(assert_close(synth.to_f64(refresh[b][:, rows]), r_ref, wl.dtype, f"refresh O[{b}]"))
    return res
