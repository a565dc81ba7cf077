"""Dynamic cache update scoring (fdl_dcu_select) on the GPU against the fp64 oracle.

Per token the distance must lie within the fp32 error bound of the kernel's arithmetic
(`dist_tol`); the activity is the fp64 sum of the kernel's own distances; the budgets and the
update sets are the oracle's decisions taken on the kernel's activities and distances (the
integer results decided in the kernel's precision), exactly, and on small inputs the update
sets also equal the oracle's own fp64 selection up to swaps inside the 1e-5 band at the cut.
"""
import numpy as np
import pytest
import torch

from oracle import focus_oracle as O
from parity import assert_selection
from workloads import synth as S

pytestmark = pytest.mark.gpu

DEV = "cuda"


def F():
    import long_context_diffusion_amd as lib
    return lib


def log(msg):
    print(msg, flush=True)


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def dist_tol(x, y, d_ref):
    """Bound on |d_gpu - d| per token.  Each fp32 sum takes H/64 terms per lane and a 6-level
    tree: relative error gamma = (H/64 + 8) 2^-24 of the sum of its absolute terms.  Through
    d = (|x-y|^2 - (|x|-|y|)^2) / (2|x||y|) that gives at most about 5 gamma |x-y|^2/(2|x||y|)
    + gamma d; the test allows twice that, plus H 2^-52 for the oracle's own fp64 cosine
    (a dot product of H terms, relative to |x||y|)."""
    H = x.shape[-1]
    gamma = (H / 64 + 8) * 2.0 ** -24
    P = ((x - y) ** 2).sum(-1)
    st = np.sqrt((x * x).sum(-1) * (y * y).sum(-1))
    scale = np.divide(P, 2.0 * st, out=np.zeros_like(P), where=st > 0)
    return 10.0 * gamma * scale + 2.0 * gamma * np.abs(d_ref) + H * 2.0 ** -52


def check_budgets(b_g, act_g, total, what):
    """Budgets equal to the oracle's split of the kernel's activities; a difference is allowed
    only where the oracle's fractional parts sit within 1e-9 of a tie (the kernel sums the
    activities in another order)."""
    b_o = O.dcu_budgets(act_g, total)
    assert int(b_g.sum()) == total, f"{what}: budgets sum to {b_g.sum()}, not {total}"
    if np.array_equal(b_g, b_o):
        return
    a = np.asarray(act_g, dtype=np.float64)
    q = total * a / a.sum() if a.sum() > 0 else np.full(len(a), total / len(a))
    frac = q - np.floor(q)
    diff = np.flatnonzero(b_g != b_o)
    assert np.all(np.abs(b_g - b_o) <= 1), f"{what}: budgets {b_g} vs {b_o}"
    spread = frac[diff].max() - frac[diff].min()
    near_int = np.minimum(frac[diff], 1 - frac[diff]).max()
    assert spread < 1e-9 or near_int < 1e-9, f"{what}: budgets {b_g} vs {b_o} away from a tie"


def run_case(x_now, x_prev, keys, w_m, total, what, oracle_select=True, sample=None):
    """One call; every output against the oracle (all tokens, or `sample` tokens per layer)."""
    B, NL, L, H = x_now.shape
    keys_g = None if keys is None else torch.from_numpy(keys).to(DEV)
    log(f"[dcu] {what}: B={B} NL={NL} L={L} H={H} keys={0 if keys is None else keys.shape[1]} "
        f"w_m={w_m} total={total} {x_now.dtype}")
    dist, act, bud, upd, n_upd = F().dcu_select(x_now, x_prev, keys_g, w_m, total)
    torch.cuda.synchronize()
    dist_h = dist.cpu().numpy().astype(np.float64)
    act_h = act.cpu().numpy()
    bud_h = bud.cpu().numpy()
    n_h = n_upd.cpu().numpy()
    upd_h = upd.cpu().numpy()
    rng = np.random.default_rng(1)
    worst = 0.0
    for b in range(B):
        must = O.dcu_mandatory([] if keys is None else keys[b], w_m, L)
        check_budgets(bud_h[b], act_h[b], total, f"{what} b{b}")
        if oracle_select:
            d_full = [O.dcu_distance(f64(x_now[b, l]), f64(x_prev[b, l])) for l in range(NL)]
            bud_o = O.dcu_budgets(np.array([d.sum() for d in d_full]), total)
        for l in range(NL):
            rows = np.arange(L) if sample is None else np.unique(np.r_[0, L - 1, rng.integers(0, L, sample)])
            x = f64(x_now[b, l, rows])
            y = f64(x_prev[b, l, rows])
            d_o = d_full[l][rows] if oracle_select else O.dcu_distance(x, y)
            err = np.abs(dist_h[b, l, rows] - d_o)
            tol = dist_tol(x, y, d_o)
            bad = np.flatnonzero(err > tol)
            assert bad.size == 0, (f"{what} b{b} l{l}: d at rows {rows[bad[:5]]}: gpu "
                                   f"{dist_h[b, l, rows[bad[:5]]]} oracle {d_o[bad[:5]]} tol {tol[bad[:5]]}")
            worst = max(worst, float((err / tol).max()))
            assert np.all(dist_h[b, l] >= 0.0)
            s = float(dist_h[b, l].sum())
            assert abs(act_h[b, l] - s) <= 1e-12 * s + 1e-300, f"{what} b{b} l{l}: activity"
            got = upd_h[b, l, : n_h[b, l]]
            expect = O.dcu_update_set(dist_h[b, l], must, int(bud_h[b, l]))
            assert np.array_equal(got, expect), (f"{what} b{b} l{l}: update set of {len(got)} vs {len(expect)}, "
                                                 f"first differences {np.setxor1d(got, expect)[:10]}")
            if oracle_select and np.array_equal(bud_o, bud_h[b]):
                # the oracle's own fp64 decision, up to swaps within 1e-5 of the cut, widened by
                # the oracle's rounding error (H 2^-52: an unchanged token's 1 - cos comes out
                # as a few 1e-16 of either sign, not 0)
                rest = np.setdiff1d(got, must)
                exp_rest = np.setdiff1d(O.dcu_update_set(d_full[l], must, int(bud_h[b, l])), must)
                assert_selection(rest, exp_rest, d_full[l], f"{what} b{b} l{l} (fp64 oracle)",
                                 abs_band=H * 2.0 ** -52)
    log(f"[dcu] {what}: ok, worst d error {worst:.3f} of its bound")


def test_dcu_fp32_ragged():
    x_now, x_prev = S.make_dcu_inputs(2, 5, 1037, 200, seed=21, device=DEV, dtype=torch.float32, zero_rows=3)
    keys = S.make_key_tokens(2, 3, 0, 1037, seed=21, pad=2)
    keys[0, 0], keys[1, 1], keys[1, 3] = 0, 1036, 5000      # the two ends, an entry past L
    run_case(x_now, x_prev, keys, 5, 600, "fp32 ragged")


def test_dcu_bf16_tail_and_strides():
    # H = 196: 24 full 16-byte vectors and a 4-element tail; layer-major storage viewed as
    # [B, NL, L, H] with a row stride of 200
    base_now, base_prev = S.make_dcu_inputs(3, 2, 700, 200, seed=22, device=DEV, dtype=torch.bfloat16)
    x_now = base_now.permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)[..., :196]
    x_prev = base_prev.permute(1, 0, 2, 3).contiguous().permute(1, 0, 2, 3)[..., :196]
    assert x_now.stride(2) == 200 and x_now.stride(0) == 700 * 200
    run_case(x_now, x_prev, None, 1, 900, "bf16 tail, strided, no keys")
    keys = np.array([[3, 3, 699, -1], [350, 0, 100, 101], [-7, 20, 20, 20]], dtype=np.int32)   # repeats
    run_case(x_now, x_prev, keys, 8, 2000, "bf16 tail, strided, keys")


@pytest.mark.parametrize("total", [0, 1, 7 * 300, 10 ** 6])
def test_dcu_budget_extremes(total):
    x_now, x_prev = S.make_dcu_inputs(1, 7, 300, 64, seed=23, device=DEV, dtype=torch.bfloat16, unchanged=0.5)
    keys = S.make_key_tokens(1, 4, 200, 300, seed=23)
    run_case(x_now, x_prev, keys, 6, total, f"total {total}")


def test_dcu_degenerate():
    # no change anywhere: every distance is 0, the budget is split evenly and the ties go to
    # the lowest positions
    x_now, _ = S.make_dcu_inputs(2, 3, 129, 32, seed=24, device=DEV, dtype=torch.float32)
    run_case(x_now, x_now.clone(), None, 1, 100, "unchanged inputs")
    # zero inputs, a window wider than the sequence, one layer, one token
    z = torch.zeros((1, 2, 40, 16), dtype=torch.bfloat16, device=DEV)
    run_case(z, z.clone(), np.array([[10]], dtype=np.int32), 1000, 5, "zero inputs, window over all")
    x1, y1 = S.make_dcu_inputs(1, 1, 1, 8, seed=25, device=DEV, dtype=torch.float32)
    run_case(x1, y1, np.array([[-1]], dtype=np.int32), 3, 1, "one token")


def test_dcu_errors():
    x = torch.zeros((1, 2, 8, 16), dtype=torch.float32, device=DEV)
    with pytest.raises(F().FdlError):
        F().dcu_select(x, x, torch.zeros((1, 2), dtype=torch.int32, device=DEV), 0, 4)    # w_m < 1 with keys
    with pytest.raises(F().FdlError):
        F().dcu_select(x, x, None, 1, -1)                                                 # negative budget
    with pytest.raises(F().FdlError):
        F().dcu_select(x[..., 1:], x[..., 1:], None, 1, 4)                                # misaligned rows


def test_dcu_full_size():
    """32 layers of a 32768-token sequence, hidden size 4096, bf16: the configuration bench.py
    times.  Distances on 256 sampled tokens per layer, every activity, budget and update set."""
    B, NL, L, H = 1, 32, 32768, 4096
    x_now, x_prev = S.make_dcu_inputs(B, NL, L, H, seed=26, device=DEV, dtype=torch.bfloat16)
    keys = S.make_key_tokens(B, 16, L - 512, L, seed=26)
    run_case(x_now, x_prev, keys, 32, NL * L // 10, "32 layers x 32768 tokens", oracle_select=False, sample=256)
