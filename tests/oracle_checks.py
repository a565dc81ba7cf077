"""Pins of the fp64 oracle: checks against things other than the oracle itself.

Every check reads the oracle through the module object ``O`` at call time, so
a test can plant a mistake in the oracle (monkeypatching one of its functions)
and confirm that some check fails.  Each check raises AssertionError on a
mismatch.  Sources of truth, per check:
  * hand-worked fixtures in tests/golden (values derived by hand from the
    definitions on the Focus-dLLM summary page; the pages print no example);
  * brute force: dominance of a selection over every non-selected candidate,
    and exhaustive enumeration of all subsets on tiny inputs;
  * exact rational arithmetic (fractions.Fraction) for block means and
    relevance;
  * a library routine: torch's scaled_dot_product_attention and scipy's
    softmax / logsumexp in fp64 on the CPU;
  * closed forms and invariants: total sink mass = heads x rows, constant V,
    single key, key permutation, sparse == dense when nothing is pruned.
"""
from __future__ import annotations

import dataclasses
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import scipy.special
import scipy.spatial.distance
import torch

from oracle import focus_oracle as O
from workloads import configs, synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ selections

def dominance_ok(values, candidates, chosen, k) -> bool:
    """True iff `chosen` is the top-k of `candidates` (larger value, then lower index)."""
    cand = set(int(c) for c in candidates)
    ch = [int(c) for c in chosen]
    if len(ch) != len(set(ch)) or list(ch) != sorted(ch):
        return False
    if not set(ch) <= cand or len(ch) != min(max(k, 0), len(cand)):
        return False
    for i in ch:
        for j in cand - set(ch):
            vi, vj = float(values[i]), float(values[j])
            if not (vi > vj or (vi == vj and i < j)):
                return False
    return True


def check_focus_count():
    for n_t, rho, k in [(4, 2.0, 8), (8, 2.0, 16), (3, 2.5, 7), (3, 0.5, 1), (16, 4.0, 64),
                        (0, 4.0, 0), (5, 0.1, 0), (10, 0.3, 3)]:
        assert O.focus_count(n_t, rho) == k, (n_t, rho)


def check_pcgi_dominance(trials=300, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(rng.integers(1, 48))
        mask = rng.random(L) < rng.random()
        conf = (rng.integers(0, 9, size=L) / 8.0).astype(np.float32)   # forced ties
        k = int(rng.integers(0, L + 3))
        got = O.pcgi_focus(conf, mask, k)
        assert dominance_ok(conf, np.flatnonzero(mask), got, k), (L, k, got)


def check_pcgi_exhaustive(trials=150, seed=1):
    """On tiny inputs exactly one subset of the candidates dominates the rest."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(rng.integers(1, 10))
        mask = rng.random(L) < 0.7
        conf = (rng.integers(0, 4, size=L) / 4.0).astype(np.float32)
        k = int(rng.integers(0, L + 2))
        cand = np.flatnonzero(mask)
        size = min(k, len(cand))
        winners = [c for c in itertools.combinations(cand, size)
                   if dominance_ok(conf, cand, c, k)]
        assert len(winners) == 1
        assert list(O.pcgi_focus(conf, mask, k)) == list(winners[0])


def check_pcgi_window_fixture():
    for case in _golden("pcgi_window_hand.json")["cases"]:
        L = case["L"]
        mask = np.zeros(L, dtype=bool)
        mask[case["mask"]] = True
        conf = np.zeros(L, dtype=np.float32)
        for i, c in case["conf"].items():
            conf[int(i)] = c
        k = O.focus_count(case["n_t"], case["rho"])
        assert k == case["k"], case["why"]
        focus = O.pcgi_focus(conf, mask, k)
        assert list(focus) == case["focus"], case["why"]
        for w, expect in case["windows"].items():
            assert list(O.window_active(focus, int(w), L)) == expect, (w, case["why"])


def check_window_closed_forms(seed=2):
    rng = np.random.default_rng(seed)
    for _ in range(100):
        L = int(rng.integers(4, 300))
        focus = np.sort(rng.choice(L, size=int(rng.integers(1, min(L, 6) + 1)), replace=False))
        assert list(O.window_active(focus, 2 * L + int(rng.integers(0, 3)), L)) == list(range(L))
        assert list(O.window_active(focus, 1, L)) == list(focus)
    for w in range(1, 12):
        L = 50
        left = O.window_active([0], w, L)
        right = O.window_active([L - 1], w, L)
        assert len(left) == w - w // 2 and left[0] == 0
        assert len(right) == w // 2 + 1 and right[-1] == L - 1
        mid = O.window_active([25], w, L)
        assert len(mid) == w and 25 in mid and np.all(np.diff(mid) == 1)
        assert mid[0] == 25 - w // 2
    # disjoint interior windows: k*w positions
    focus = [20, 60, 100, 140]
    for w in (3, 8, 16, 33):
        assert len(O.window_active(focus, w, 400)) == len(focus) * w


# ------------------------------------------------------------------ attention

def check_attention_closed_form():
    for case in _golden("attention_closed_form.json")["cases"]:
        Q, K, V = (np.array(case[x], dtype=np.float64) for x in ("q", "k", "v"))
        d = Q.shape[-1]
        out, lse = O.attention(Q, K, V, 1.0 / math.sqrt(d))
        for h in range(case["Hq"]):
            for i, row in enumerate(case["o"][h]):
                if row is None:
                    continue
                _close(out[h, i], row, 1e-12, case["name"])
                _close(lse[h, i], case["lse"][h][i], 1e-12, case["name"] + " lse")


def _sdpa(Q, K, V, scale):
    Hq, Hkv = Q.shape[0], K.shape[0]
    q = torch.from_numpy(Q)[None]
    k = torch.from_numpy(K)[None]
    v = torch.from_numpy(V)[None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, scale=scale, enable_gqa=(Hq != Hkv))
    return o[0].numpy()


def check_attention_vs_library(seed=3):
    rng = np.random.default_rng(seed)
    for Hq, Hkv, n, m, d in [(1, 1, 5, 9, 8), (4, 4, 7, 13, 16), (6, 2, 3, 17, 8),
                             (28, 4, 2, 40, 4), (2, 1, 1, 1, 64)]:
        Q = rng.normal(size=(Hq, n, d))
        K = rng.normal(size=(Hkv, m, d))
        V = rng.normal(size=(Hkv, m, d))
        scale = 1.0 / math.sqrt(d)
        out, lse = O.attention(Q, K, V, scale)
        _close(out, _sdpa(Q, K, V, scale), 1e-12, f"sdpa {Hq}/{Hkv}")
        G = Hq // Hkv
        for h in range(Hq):
            S = Q[h] @ K[h // G].T * scale
            _close(lse[h], scipy.special.logsumexp(S, axis=1), 1e-12, "lse")


def check_attention_invariants(seed=4):
    rng = np.random.default_rng(seed)
    Hq, Hkv, n, m, d = 4, 2, 6, 11, 8
    Q = rng.normal(size=(Hq, n, d))
    K = rng.normal(size=(Hkv, m, d))
    V = rng.normal(size=(Hkv, m, d))
    s = 0.3
    out, lse = O.attention(Q, K, V, s)
    # constant V rows -> O equals that row
    Vc = np.broadcast_to(rng.normal(size=(Hkv, 1, d)), (Hkv, m, d)).copy()
    oc, _ = O.attention(Q, K, Vc, s)
    for h in range(Hq):
        _close(oc[h], np.broadcast_to(Vc[h // 2, 0], (n, d)), 1e-12, "constant V")
    # one key -> O = v and lse = q.k*s
    o1, l1 = O.attention(Q, K[:, :1], V[:, :1], s)
    for h in range(Hq):
        _close(o1[h], np.broadcast_to(V[h // 2, 0], (n, d)), 1e-12, "single key")
        _close(l1[h], Q[h] @ K[h // 2, 0] * s, 1e-12, "single key lse")
    # permuting keys and values together leaves O and lse unchanged
    perm = rng.permutation(m)
    op, lp = O.attention(Q, K[:, perm], V[:, perm], s)
    _close(op, out, 1e-12, "key permutation")
    _close(lp, lse, 1e-12, "key permutation lse")
    # permuting query rows permutes the output rows
    qp = rng.permutation(n)
    oq, _ = O.attention(Q[:, qp], K, V, s)
    _close(oq, out[:, qp], 1e-12, "query permutation")
    # no keys: zero output, lse = -inf
    oe, le = O.attention(Q, K[:, :0], V[:, :0], s)
    assert np.all(oe == 0) and np.all(np.isneginf(le))


# ------------------------------------------------------------------ sinks

def check_sink_scores_vs_library(seed=5):
    rng = np.random.default_rng(seed)
    for Hq, Hkv, n, L, d in [(4, 4, 5, 30, 8), (6, 2, 3, 41, 4), (2, 1, 1, 7, 16)]:
        Q = rng.normal(size=(Hq, n, d))
        K = rng.normal(size=(Hkv, L, d))
        s = 1.0 / math.sqrt(d)
        _, lse = O.attention(Q, K, K, s)
        got = O.sink_scores(Q, K, lse, s)
        expect = np.zeros(L)
        G = Hq // Hkv
        for h in range(Hq):
            expect += scipy.special.softmax(Q[h] @ K[h // G].T * s, axis=1).sum(axis=0)
        _close(got, expect, 1e-12, "sink scores")
        # every query row spreads unit mass over the keys
        _close(got.sum(), Hq * n, 1e-9, "total attention mass")


def check_sink_select_dominance(seed=6):
    rng = np.random.default_rng(seed)
    for _ in range(200):
        L = int(rng.integers(1, 60))
        scores = rng.integers(0, 6, size=L) / 5.0
        n = int(rng.integers(0, L + 2))
        assert dominance_ok(scores, range(L), O.sink_select(scores, n), n)
        R = rng.integers(-3, 4, size=L).astype(np.float64)
        assert dominance_ok(R, range(L), O.top_blocks(R, n), n)


def check_sink_recovery(seeds=(0, 1, 2)):
    """Sinks injected by the generator are the ones the oracle identifies."""
    base = configs.TINY_2K_F32
    for seed in seeds:
        wl = base if seed == 0 else dataclasses.replace(base, seed=seed, sinks_fixed=())
        conf, mask = synth.step_inputs(wl)
        K, V = (synth.to_f64(t)[0] for t in synth.make_kv(wl, 0))
        Q = synth.to_f64(synth.make_q(wl, 0))[0]
        focus = O.pcgi_focus(conf[0], mask[0], O.focus_count(wl.n_t, wl.rho))
        active = O.window_active(focus, wl.w, wl.L)
        _, lse = O.dense_attention(Q[:, active], K, V, wl.scale)
        sinks = O.sink_select(O.sink_scores(Q[:, active], K, lse, wl.scale), wl.n_sinks)
        assert list(sinks) == list(synth.sink_positions(wl, 0)), (seed, sinks)


# ------------------------------------------------------------------ block pruning

def _bf16_grid(rng, shape):
    """Random values exactly representable in bf16 (8 significant bits)."""
    mant = rng.integers(-255, 256, size=shape)
    expo = rng.integers(-12, 2, size=shape)
    return np.ldexp(mant.astype(np.float64), expo)


def check_block_means_exact(seed=7):
    rng = np.random.default_rng(seed)
    for Hkv, P, extra, bs, d in [(2, 13, 3, 4, 3), (1, 16, 0, 4, 2), (3, 7, 2, 8, 2), (1, 1, 1, 1, 1)]:
        K = _bf16_grid(rng, (Hkv, P + extra, d))
        kbar = O.block_means(K, P, bs)
        nb = -(-P // bs)
        assert kbar.shape == (Hkv, nb, d)
        for g in range(Hkv):
            for b in range(nb):
                lo, hi = b * bs, min(b * bs + bs, P)
                for e in range(d):
                    exact = sum(Fraction(float(K[g, j, e])) for j in range(lo, hi)) / (hi - lo)
                    # the sum is exact in fp64; the one division rounds correctly
                    assert float(kbar[g, b, e]) == float(exact), (g, b, e)
    wl = configs.TINY_2K_F32
    K = synth.to_f64(synth.make_kv(wl, 0)[0])[0]
    kbar = O.block_means(K, wl.P, wl.bs)
    for g, b, e in [(0, 0, 0), (1, 10, 5), (3, 30, 63), (2, 23, 17)]:
        lo, hi = b * wl.bs, min(b * wl.bs + wl.bs, wl.P)
        exact = sum(Fraction(float(K[g, j, e])) for j in range(lo, hi)) / (hi - lo)
        assert float(kbar[g, b, e]) == float(exact)


def check_relevance_bruteforce(seed=8):
    rng = np.random.default_rng(seed)
    for Hq, Hkv, n, P, bs, d in [(2, 2, 3, 10, 4, 3), (4, 2, 2, 9, 3, 2), (3, 1, 1, 5, 5, 2)]:
        Q = _bf16_grid(rng, (Hq, n, d))
        K = _bf16_grid(rng, (Hkv, P + 2, d))
        scale = 0.25
        R = O.block_relevance(Q, O.block_means(K, P, bs), scale)
        nb = -(-P // bs)
        G = Hq // Hkv
        for b in range(nb):
            lo, hi = b * bs, min(b * bs + bs, P)
            total = Fraction(0)
            for h in range(Hq):
                for i in range(n):
                    for e in range(d):
                        mean = sum(Fraction(float(K[h // G, j, e])) for j in range(lo, hi)) / (hi - lo)
                        total += Fraction(float(Q[h, i, e])) * mean
            assert abs(float(R[b]) - float(total) * scale) <= 1e-12 * (1 + abs(float(total))), b
    # one head, one query row: R_b = scale * q . kbar_b
    q = rng.normal(size=(1, 1, 4))
    K = rng.normal(size=(1, 12, 4))
    kbar = O.block_means(K, 12, 4)
    _close(O.block_relevance(q, kbar, 0.5), 0.5 * kbar[0] @ q[0, 0], 1e-12, "single row")


def check_block_fixture():
    for case in _golden("block_keyset_hand.json")["cases"]:
        K = np.array(case["k"], dtype=np.float64)
        Q = np.array(case["q"], dtype=np.float64)
        kbar = O.block_means(K, case["P"], case["bs"])
        _close(kbar, case["kbar"], 0.0, "kbar")
        R = O.block_relevance(Q, kbar, case["scale"])
        _close(R, case["R"], 1e-15, "R")
        for C, sel in case["C"].items():
            blocks = O.top_blocks(R, int(C))
            assert list(blocks) == sel["blocks"], (C, case["why"])
            I_p = O.key_set(sel["sinks"], blocks, case["bs"], case["P"], case["L"])
            assert list(I_p) == sel["I_p"], (C, case["why"])


def check_key_set(seed=9):
    rng = np.random.default_rng(seed)
    for _ in range(100):
        bs = int(rng.integers(1, 9))
        P = int(rng.integers(1, 60))
        L = P + int(rng.integers(0, 20))
        nb = -(-P // bs)
        blocks = np.sort(rng.choice(nb, size=int(rng.integers(0, nb + 1)), replace=False))
        sinks = np.sort(rng.choice(L, size=int(rng.integers(0, min(L, 6) + 1)), replace=False))
        I_p = O.key_set(sinks, blocks, bs, P, L)
        members = [j for j in range(L)
                   if j >= P or j in set(sinks.tolist()) or (j // bs) in set(blocks.tolist())]
        assert list(I_p) == members
    # every block kept: the whole sequence; nothing kept: the generation region
    assert list(O.key_set([], range(8), 4, 30, 37)) == list(range(37))
    assert list(O.key_set([], [], 4, 30, 37)) == list(range(30, 37))
    assert list(O.key_set([1, 2, 33], [0], 4, 30, 37)) == [0, 1, 2, 3] + list(range(30, 37))


# ------------------------------------------------------------------ sparse step

def _tiny_inputs(wl=configs.TINY_2K_F32):
    conf, mask = synth.step_inputs(wl)
    K, V = (synth.to_f64(t)[0] for t in synth.make_kv(wl, 0))
    Q = synth.to_f64(synth.make_q(wl, 0))[0]
    return conf[0], mask[0], Q, K, V


def check_sparse_equals_dense():
    """Every block kept and a window over the whole sequence: sparse == dense."""
    wl = configs.TINY_2K_F32
    conf, mask, Q, K, V = _tiny_inputs(wl)
    focus = O.pcgi_focus(conf, mask, O.focus_count(wl.n_t, wl.rho))
    active = O.window_active(focus, 2 * wl.L, wl.L)
    assert list(active) == list(range(wl.L))
    Qa = Q[:, active[::17]]
    dense, dlse = O.dense_attention(Qa, K, V, wl.scale)
    R = O.block_relevance(Qa, O.block_means(K, wl.P, wl.bs), wl.scale)
    blocks = O.top_blocks(R, wl.nb)
    I_p = O.key_set([], blocks, wl.bs, wl.P, wl.L)
    sparse, slse = O.sparse_attention(Qa, K, V, I_p, wl.scale)
    _close(sparse, dense, 1e-13, "sparse == dense")
    _close(slse, dlse, 1e-12, "sparse == dense lse")


def check_sparse_vs_library(seed=10):
    wl = configs.TINY_2K_F32
    conf, mask, Q, K, V = _tiny_inputs(wl)
    rng = np.random.default_rng(seed)
    active = np.sort(rng.choice(wl.L, 24, replace=False))
    sinks = [3, 700, 2040]
    blocks = np.sort(rng.choice(wl.nb, 5, replace=False))
    I_p = O.key_set(sinks, blocks, wl.bs, wl.P, wl.L)
    out, _ = O.sparse_attention(Q[:, active], K, V, I_p, wl.scale)
    ref = _sdpa(Q[:, active].copy(), K[:, I_p].copy(), V[:, I_p].copy(), wl.scale)
    _close(out, ref, 1e-12, "sparse vs library on the gathered keys")
    # no sinks, no blocks: attention over the generation region only
    I_gen = O.key_set([], [], wl.bs, wl.P, wl.L)
    out, _ = O.sparse_attention(Q[:, active], K, V, I_gen, wl.scale)
    ref = _sdpa(Q[:, active].copy(), K[:, wl.P:].copy(), V[:, wl.P:].copy(), wl.scale)
    _close(out, ref, 1e-12, "generation region only")


def check_step_composition():
    """The one-layer driver reproduces its parts and keeps the sink blocks."""
    wl = configs.TINY_2K_F32
    conf, mask, Q, K, V = _tiny_inputs(wl)
    st = O.sparse_step(conf, mask, lambda l: (Q, K, V), layers=1, l_dense=1, n_t=wl.n_t,
                       rho=wl.rho, w=wl.w, P=wl.P, bs=wl.bs, C=wl.C, n_sinks=wl.n_sinks,
                       scale=wl.scale)
    assert len(st.focus) == 8   # k = floor(2 * 4) stated by the 2K workload
    assert list(st.sinks) == list(wl.sinks_fixed)
    assert {s // wl.bs for s in wl.sinks_fixed} <= set(st.blocks[0].tolist())
    out, _ = O.sparse_attention(Q[:, st.active], K, V,
                                O.key_set(st.sinks, st.blocks[0], wl.bs, wl.P, wl.L), wl.scale)
    _close(st.out[("sparse", 0)], out, 0.0, "driver sparse output")



def _touched_by_enumeration(rows, P, bs):
    """Blocks b of [0, ceil(P/bs)) whose span [b*bs, min((b+1)*bs, P)) holds a refreshed row:
    each block is tested against every row, with no division."""
    nb = -(-P // bs)
    out = []
    for b in range(nb):
        lo, hi = b * bs, min((b + 1) * bs, P)
        if any(lo <= int(r) < hi for r in rows):
            out.append(b)
    return out


def _check_touched_blocks(rows, P, bs, touched):
    assert list(touched) == _touched_by_enumeration(rows, P, bs), f"touched blocks {list(touched)}"


def check_refreshed_blocks(seed=12):
    """The blocks a refresh touches, against enumeration over the blocks: rows at and past
    the prompt end (one inside the prompt's last, short block span if it were not cut at P),
    negative entries, repeats, a row in the last prompt block, and random lists."""
    cases = [
        ([250, 251, 255, 290, -1], 250, 16),       # only rows >= P: nothing touched
        ([0, 15, 16, 249], 250, 16),               # block edges and the short last block
        ([239, 240, 240, 7, 7], 250, 16),          # repeats, any order
        ([], 250, 16),
        ([63, 64, 127, 128], 129, 64),             # last block of one key
    ]
    rng = np.random.default_rng(seed)
    for _ in range(40):
        P = int(rng.integers(1, 400))
        bs = int(rng.integers(1, 70))
        rows = rng.integers(-3, P + 40, size=int(rng.integers(0, 30))).tolist()
        cases.append((rows, P, bs))
    for rows, P, bs in cases:
        _check_touched_blocks(rows, P, bs, O.refreshed_blocks(rows, P, bs))


def check_kv_refresh(seed=11):
    """The refreshed cache: new rows where U(t) says, cached rows elsewhere; refreshing
    rows with their own values changes nothing; and the block means of the refreshed cache
    equal the old means plus the incremental correction sum(new - old) / |block| of the
    refreshed blocks only (an independent formula for the same result)."""
    rng = np.random.default_rng(seed)
    Hkv, L, d, P, bs = 2, 300, 16, 250, 16
    K = _bf16_grid(rng, (Hkv, L, d))
    V = _bf16_grid(rng, (Hkv, L, d))
    rows = np.array([3, 4, 40, 47, 48, 199, 245, 249, 250, 290, -1])
    valid = rows[rows >= 0]
    Kn = _bf16_grid(rng, (Hkv, len(rows), d))
    Vn = _bf16_grid(rng, (Hkv, len(rows), d))
    K2, V2 = O.kv_refresh(K, V, rows, Kn, Vn)
    for j, r in enumerate(rows):
        if r >= 0:
            assert np.array_equal(K2[:, r], Kn[:, j]) and np.array_equal(V2[:, r], Vn[:, j])
    keep = np.setdiff1d(np.arange(L), valid)
    assert np.array_equal(K2[:, keep], K[:, keep]) and np.array_equal(V2[:, keep], V[:, keep])
    K3, V3 = O.kv_refresh(K, V, valid, K[:, valid], V[:, valid])
    assert np.array_equal(K3, K) and np.array_equal(V3, V)
    old, new = O.block_means(K, P, bs), O.block_means(K2, P, bs)
    touched = O.refreshed_blocks(rows, P, bs)
    _check_touched_blocks(rows, P, bs, touched)
    inc = old.copy()
    for j, r in enumerate(rows):
        if 0 <= r < P:
            b = r // bs
            size = min((b + 1) * bs, P) - b * bs
            inc[:, b] += (Kn[:, j] - K[:, r]) / size
    _close(new, inc, 1e-12, "incremental block means")
    untouched = np.setdiff1d(np.arange(old.shape[1]), touched)
    assert np.array_equal(new[:, untouched], old[:, untouched])


def check_confidence_fixture():
    """Hand-worked confidences, tokens and unmask choices (tests/golden/confidence_hand.json)."""
    for case in _golden("confidence_hand.json")["cases"]:
        logits = np.log(np.asarray(case["logits_exp"], dtype=np.float64))
        mask = np.zeros(case["L"], dtype=bool)
        mask[case["masked"]] = True
        conf, tokens, chosen = O.unmask_step(logits, np.array(case["positions"]), mask, case["n_t"])
        _close(conf, case["conf"], 1e-15, "fixture confidence")
        assert list(tokens) == case["tokens"], f"fixture tokens {list(tokens)}"
        assert list(chosen) == case["chosen"], f"fixture unmask {list(chosen)}"


def check_confidence_vs_library(seed=13):
    """c against scipy's softmax on random rows; closed forms: uniform logits give 1/V and
    token 0, one logit T above V-1 zeros gives e^T / (e^T + V - 1); shifting a row leaves
    c unchanged; argmax by brute force with planted ties."""
    rng = np.random.default_rng(seed)
    for V in (2, 5, 97, 1000):
        for _ in range(5):
            z = rng.normal(size=V) * rng.uniform(0.1, 6.0)
            z[rng.integers(V)] = z.max()                 # an exact tie at the max
            c, tok = O.token_confidence(z)
            _close(c, scipy.special.softmax(z).max(), 1e-14, "confidence vs scipy")
            assert tok == min(i for i in range(V) if z[i] == z.max())
            _close(O.token_confidence(z + 7.25)[0], c, 1e-14, "shift invariance")
        c, tok = O.token_confidence(np.full(V, -3.5))
        _close(c, 1.0 / V, 1e-15, "uniform confidence")
        assert tok == 0
        for T in (0.0, 1.0, 9.0):
            z = np.zeros(V)
            z[V // 2] = T
            c, tok = O.token_confidence(z)
            _close(c, math.exp(T) / (math.exp(T) + V - 1), 1e-14, "one peak")
            assert tok == (V // 2 if T > 0 else 0)


def check_unmask_dominance(trials=200, seed=14):
    """The unmasked set is the top n(t) of the masked rows by confidence (dominance), with
    planted ties and rows whose position is no longer masked."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        L = int(rng.integers(8, 80))
        M = int(rng.integers(1, L))
        positions = np.sort(rng.choice(L, M, replace=False))
        mask = rng.random(L) < 0.7
        V = int(rng.integers(2, 9))
        logits = np.log(rng.integers(1, 4, size=(M, V)).astype(np.float64))   # many equal confidences
        n_t = int(rng.integers(0, M + 2))
        conf, _, chosen = O.unmask_step(logits, positions, mask, n_t)
        row_of = {int(p): r for r, p in enumerate(positions)}
        cand = [int(p) for p in positions if mask[p]]
        assert dominance_ok({p: conf[row_of[p]] for p in cand}, cand, chosen, n_t)


def check_per_head_relevance(trials=40, seed=17):
    """Per-KV-head relevance: summed over the KV heads it is the shared R_b (pinned by its
    own checks); with one KV head it is R_b; each head's top-C dominates its own scores."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        Hkv = int(rng.choice([1, 2, 3]))
        Hq = Hkv * int(rng.integers(1, 4))
        n, d, nb = int(rng.integers(0, 6)), int(rng.integers(1, 6)), int(rng.integers(1, 9))
        Q = rng.normal(size=(Hq, n, d))
        kbar = rng.normal(size=(Hkv, nb, d))
        s = float(rng.uniform(0.1, 1.0))
        Rg = O.block_relevance_per_head(Q, kbar, s)
        assert Rg.shape == (Hkv, nb)
        _close(Rg.sum(axis=0), O.block_relevance(Q, kbar, s), 1e-12, "sum over KV heads")
        if Hkv == 1:
            _close(Rg[0], O.block_relevance(Q, kbar, s), 1e-12, "one KV head")
        C = int(rng.integers(0, nb + 2))
        for g in range(Hkv):
            assert dominance_ok(Rg[g], range(nb), O.top_blocks(Rg[g], C), C)


def check_max_relevance(trials=40, seed=18):
    """Max aggregator: one query of one head gives s q.kbar; identical queries over one KV
    head give the summed relevance divided by their count; adding a query never lowers a
    score; the per-head scores reduce to the shared ones by a max over the KV heads; no
    query gives -inf."""
    rng = np.random.default_rng(seed)
    q = rng.normal(size=5)
    kbar = rng.normal(size=(1, 4, 5))
    _close(O.block_relevance_max(q.reshape(1, 1, 5), kbar, 0.5), 0.5 * kbar[0] @ q, 1e-12, "one query")
    Q = np.broadcast_to(q, (3, 4, 5))
    _close(O.block_relevance_max(Q, kbar, 0.5), O.block_relevance(Q, kbar, 0.5) / 12, 1e-12, "identical queries")
    assert np.all(O.block_relevance_max(np.zeros((2, 0, 5)), kbar, 0.5) == -np.inf)
    for _ in range(trials):
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.integers(1, 3))
        n, d, nb = int(rng.integers(1, 6)), int(rng.integers(1, 6)), int(rng.integers(1, 8))
        Q = rng.normal(size=(Hq, n, d))
        kb = rng.normal(size=(Hkv, nb, d))
        R = O.block_relevance_max(Q, kb, 0.3)
        Rg = O.block_relevance_max(Q, kb, 0.3, per_head=True)
        _close(Rg.max(axis=0), R, 0.0, "max over KV heads")
        more = np.concatenate([Q, rng.normal(size=(Hq, 2, d))], axis=1)
        assert np.all(O.block_relevance_max(more, kb, 0.3) >= R - 1e-12 * np.abs(R))   # matmul rounding


def check_paper_defaults():
    """alpha = 0.5 keeps half of an even block count, 0 keeps all, 1 none; N_sinks at
    32K and 8K (Summary, "Reproducibility")."""
    assert O.blocks_kept(504, 0.5) == 252 and O.blocks_kept(7, 0.5) == 4
    assert O.blocks_kept(504, 0.0) == 504 and O.blocks_kept(504, 1.0) == 0
    assert O.paper_sink_count(32768) == 327 and O.paper_sink_count(8192) == 81 and O.paper_sink_count(99) == 0


def check_step_variants():
    """The step with a dense tail runs dense attention in its last layers and sparse in
    the others; with one KV head the per-head step equals the shared one."""
    wl = configs.TINY_2K_F32
    conf, mask, Q, K, V = _tiny_inputs(wl)
    rng = np.random.default_rng(19)
    Qs = [Q, Q[:, :, ::-1].copy(), Q * 0.5]
    kw = dict(layers=3, l_dense=1, n_t=wl.n_t, rho=wl.rho, w=wl.w, P=wl.P, bs=wl.bs, C=wl.C,
              n_sinks=wl.n_sinks, scale=wl.scale)
    st = O.sparse_step(conf, mask, lambda l: (Qs[l], K, V), dense_tail=1, **kw)
    Qa = Qs[2][:, st.active]
    _close(st.out[2], O.dense_attention(Qa, K, V, wl.scale)[0], 0.0, "dense tail layer")
    assert 1 in st.blocks and 2 not in st.blocks
    I_p = O.key_set(st.sinks, st.blocks[1], wl.bs, wl.P, wl.L)
    _close(st.out[1], O.sparse_attention(Qs[1][:, st.active], K, V, I_p, wl.scale)[0], 0.0, "sparse layer")
    K1, V1 = K[:1], V[:1]
    shared = O.sparse_step(conf, mask, lambda l: (Qs[l], K1, V1), **kw)
    ph = O.sparse_step(conf, mask, lambda l: (Qs[l], K1, V1), per_head=True, **kw)
    for l in (1, 2):
        assert list(ph.blocks[l][0]) == list(shared.blocks[l])
        _close(ph.out[l], shared.out[l], 1e-12, f"per-head layer {l}")
    # two KV heads, one attending over every key and one over a subset: the first head's
    # output is dense attention, the second's sparse attention over its own set
    L = 40
    Qh = rng.normal(size=(2, 3, 4))
    Kh, Vh = rng.normal(size=(2, L, 4)), rng.normal(size=(2, L, 4))
    sub = np.array([0, 3, 7, 21, 39])
    O2, _ = O.sparse_attention_per_head(Qh, Kh, Vh, [np.arange(L), sub], 0.5)
    _close(O2[:1], O.dense_attention(Qh[:1], Kh[:1], Vh[:1], 0.5)[0], 1e-12, "per-head set of all keys")
    _close(O2[1:], O.sparse_attention(Qh[1:], Kh[1:], Vh[1:], sub, 0.5)[0], 1e-12, "per-head subset")


def check_dcu_budget_fixture():
    """Hand-worked budget splits and a mandatory window (tests/golden/dcu_budget_hand.json)."""
    g = _golden("dcu_budget_hand.json")
    for case in g["cases"]:
        got = O.dcu_budgets(case["activity"], case["total"])
        assert list(got) == case["budgets"], f"budgets {list(got)} for {case}"
    for case in g["window_cases"]:
        got = O.dcu_mandatory(case["key_tokens"], case["w_m"], case["L"])
        assert list(got) == case["mandatory"], f"window {list(got)}"


def check_dcu_distance_vs_library(seed=15):
    """Cosine distance against scipy.spatial.distance.cosine; closed forms: a vector and a
    positive multiple of it give 0, its negative 2, orthogonal vectors 1; zero rows give 0."""
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(12, 33))
    y = x + rng.normal(size=(12, 33)) * rng.uniform(0.0, 2.0, size=(12, 1))
    d = O.dcu_distance(x, y)
    for i in range(12):
        _close(d[i], scipy.spatial.distance.cosine(x[i], y[i]), 1e-12, "cosine distance")
    e = np.eye(4)
    _close(O.dcu_distance(np.stack([e[0], e[1], e[2], np.zeros(4)]),
                          np.stack([3 * e[0], -2 * e[1], e[3], e[0]])), [0.0, 2.0, 1.0, 0.0], 1e-15, "closed forms")


def check_dcu_selection(trials=120, seed=16):
    """Budgets sum to the total and stay within one token of the proportional share;
    each update set holds the mandatory window and the top-budget others (dominance)."""
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        layers, L, H = int(rng.integers(1, 6)), int(rng.integers(4, 60)), int(rng.integers(1, 9))
        x = rng.normal(size=(layers, L, H))
        y = x + rng.normal(size=(layers, L, H)) * rng.uniform(0, 1, size=(layers, 1, 1))
        y[:, ::5] = x[:, ::5]                            # unchanged tokens: d = 0 ties
        keys = rng.integers(-1, L, size=int(rng.integers(0, 4)))
        w_m = int(rng.integers(1, 7))
        total = int(rng.integers(0, layers * L))
        d, act, budgets, sets = O.dcu_select(x, y, keys, w_m, total)
        assert int(budgets.sum()) == total
        share = total * act / act.sum() if act.sum() > 0 else np.full(layers, total / layers)
        assert np.all(np.abs(budgets - share) < 1.0)
        must = set(int(j) for j in O.dcu_mandatory(keys, w_m, L))
        brute = set(j for c in keys if c >= 0 for j in range(c - w_m // 2, c - w_m // 2 + w_m) if 0 <= j < L)
        assert must == brute
        for l in range(layers):
            got = [int(j) for j in sets[l]]
            assert got == sorted(set(got)) and must <= set(got)
            rest = [j for j in range(L) if j not in must]
            extra = sorted(set(got) - must)
            assert dominance_ok(d[l], rest, extra, int(budgets[l]))


ALL_CHECKS = [
    check_focus_count, check_pcgi_dominance, check_pcgi_exhaustive, check_pcgi_window_fixture,
    check_window_closed_forms, check_attention_closed_form, check_attention_vs_library,
    check_attention_invariants, check_sink_scores_vs_library, check_sink_select_dominance,
    check_sink_recovery, check_block_means_exact, check_relevance_bruteforce,
    check_block_fixture, check_key_set, check_sparse_equals_dense, check_sparse_vs_library,
    check_step_composition, check_kv_refresh, check_refreshed_blocks,
    check_confidence_fixture, check_confidence_vs_library, check_unmask_dominance,
    check_dcu_budget_fixture, check_dcu_distance_vs_library, check_dcu_selection,
    check_per_head_relevance, check_max_relevance, check_paper_defaults, check_step_variants,
]
