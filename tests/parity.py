"""Comparison rules between the HIP path and the fp64 oracle.

Index sets must be equal, except that a selection may swap members whose oracle
score lies within 1e-5 * |cut| of the oracle's cut score (the k-th / C-th
value): an fp32 or fp64 rounding difference can legitimately reorder such
near-ties.  PCGI gets no band (its keys are compared exactly on both sides).
Outputs: max abs error <= 1e-5 for fp32 inputs, <= 2e-2 for bf16 inputs (fp32
accumulation).  A relative check (max abs error / max |reference|) is held to
1e-5 (fp32) and 1e-2 (bf16, about 2.5 units in the last place of the largest
output): the absolute bf16 bound alone is larger than the outputs themselves
(|O| is a few 1e-3 with the workloads' sigma = 1/8), so the relative one is the
bound that bites.
"""
import numpy as np

ABS_TOL = {"f32": 1e-5, "bf16": 2e-2}
REL_TOL = {"f32": 1e-5, "bf16": 1e-2}
TIE_BAND = 1e-5


def valid(idx):
    idx = np.asarray(idx).ravel()
    return idx[idx >= 0]


def assert_exact_set(got, expect, what):
    got, expect = valid(got), np.asarray(expect)
    assert np.array_equal(got, expect), f"{what}: got {got[:20]}... expected {expect[:20]}..."


def assert_selection(got, expect, scores, what, abs_band=0.0):
    """Selection equal to the oracle's, up to swaps inside the tie band at the cut (TIE_BAND
    relative to the cut, widened by `abs_band` where the oracle's own scores carry an absolute
    rounding error).

    Returns True when the sets are identical."""
    got, expect = valid(got), np.asarray(expect)
    assert np.all(np.diff(got) > 0), f"{what}: not strictly ascending"
    assert len(got) == len(expect), f"{what}: {len(got)} selected, expected {len(expect)}"
    if np.array_equal(got, expect):
        return True
    scores = np.asarray(scores, dtype=np.float64)
    cut = scores[expect].min() if len(expect) else 0.0
    band = TIE_BAND * abs(cut) + abs_band
    diff = np.setxor1d(got, expect)
    far = diff[np.abs(scores[diff] - cut) > band]
    assert far.size == 0, (f"{what}: members {far[:10]} differ outside the tie band "
                           f"(cut {cut:.9g}, scores {scores[far[:10]]})")
    return False


def assert_close(got, ref, dtype, what, rows=None):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    rel = err / scale if scale > 0 else err
    assert err <= ABS_TOL[dtype], f"{what}: max abs err {err:.3e} > {ABS_TOL[dtype]:.0e}"
    assert rel <= REL_TOL[dtype], f"{what}: max rel err {rel:.3e} > {REL_TOL[dtype]:.0e}"
    return err, rel
