"""Token confidence and unmasking on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

from oracle import focus_oracle as O
from parity import assert_selection

pytestmark = pytest.mark.gpu

DEV = "cuda"


def F():
    import long_context_diffusion_amd as lib
    return lib


def f64(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def log(msg):
    print(msg, flush=True)


def run_case(logits, pos, mask, n_t, n_rows=None, check_rows=None):
    """One call on the GPU, then every output against the oracle: c within 2e-6 relative,
    tokens exact, the unmasked set up to swaps inside the 1e-5 band at the cut, mask, conf
    and tokens updated exactly where the contract says."""
    B, M, V = logits.shape
    L = mask.shape[1]
    mask_g = mask.clone()
    conf_g = torch.full((B, L), -9.0, dtype=torch.float32, device=DEV)
    tok_g = torch.full((B, L), -5, dtype=torch.int32, device=DEV)
    un = F().confidence_unmask(logits, pos, mask_g, conf_g, n_t, n_rows=n_rows, tokens=tok_g)
    torch.cuda.synchronize()
    z = f64(logits)
    worst = 0.0
    for b in range(B):
        n = int(n_rows[b]) if n_rows is not None else M
        p = pos[b, :n].cpu().numpy().astype(np.int64)
        keep = (p >= 0) & (p < L)
        rows = np.flatnonzero(keep)
        mk = mask[b].cpu().numpy().astype(bool)
        conf_o, tok_o, chosen_o = O.unmask_step(z[b][rows], p[rows], mk, n_t)
        chosen_g = un[b].cpu().numpy()
        chosen_g = chosen_g[chosen_g >= 0]
        cand = [int(q) for q in p[rows] if mk[q]]
        c_of = {int(q): conf_o[i] for i, q in enumerate(p[rows])}
        scores = np.zeros(L)
        for q in cand:
            scores[q] = c_of[q]
        assert_selection(chosen_g, chosen_o, scores, f"unmasked b{b}")
        cg = conf_g[b].cpu().numpy().astype(np.float64)
        tg = tok_g[b].cpu().numpy()
        mg = mask_g[b].cpu().numpy().astype(bool)
        chosen_set = set(int(q) for q in chosen_g)
        sample = rows if check_rows is None else rows[:check_rows]
        for i in sample:
            q = int(p[i])
            j = list(rows).index(i)
            if q in chosen_set:
                assert cg[q] == 0.0 and not mg[q] and tg[q] == tok_o[j], f"unmasked row {q}"
            elif mk[q]:
                rel = abs(cg[q] - conf_o[j]) / conf_o[j]
                worst = max(worst, rel)
                assert rel <= 2e-6, f"confidence of {q}: {cg[q]} vs {conf_o[j]}"
                assert mg[q] and tg[q] == -5
            else:
                assert cg[q] == 0.0 and not mg[q]
        untouched = np.setdiff1d(np.arange(L), p[rows])
        assert np.all(cg[untouched] == -9.0) and np.all(tg[untouched] == -5)
        assert np.array_equal(mg[untouched], mk[untouched])
    return worst


@pytest.mark.parametrize("dtype,V", [(torch.bfloat16, 1000), (torch.bfloat16, 16389), (torch.float32, 1003),
                                     (torch.float32, 8192)])
def test_confidence_small(dtype, V):
    B, M, L = 3, 37, 300
    from workloads import synth
    # rows must start on 16-byte boundaries: a ragged V is a view of padded rows
    per16 = 16 // torch.tensor([], dtype=dtype).element_size()
    Vp = -(-V // per16) * per16
    wide = synth.make_logits(B, M, Vp, seed=V, device=DEV, dtype=dtype)
    logits = wide[..., :V]
    # planted ties: rows 3 and 9 of sequence 0 identical (equal confidence); two equal maxima
    logits[0, 9] = logits[0, 3]
    top = logits[1, 5].float().max()
    logits[1, 5, 7] = top.to(dtype)
    logits[1, 5, V - 2] = top.to(dtype)
    g = torch.Generator().manual_seed(V)
    pos = torch.stack([torch.randperm(L, generator=g)[:M].sort().values for _ in range(B)]).to(torch.int32)
    mask = (torch.rand((B, L), generator=g) < 0.8).to(torch.uint8)
    mask[0, pos[0, 3]] = 1
    mask[0, pos[0, 9]] = 1
    n_rows = torch.tensor([M, M - 4, 20], dtype=torch.int32)
    pos[1, M - 4:] = -1   # padding rows past n_rows
    pos[2, 20:] = 12345
    worst = 0.0
    for n_t in (0, 1, 5, M + 3):
        worst = max(worst, run_case(logits, pos.to(DEV), mask.to(DEV), n_t, n_rows=n_rows.to(DEV)))
    log(f"confidence {dtype} V={V}: worst relative error of c {worst:.2e}")


def test_confidence_ties_pick_lowest_position():
    """Identical rows tie exactly: the lowest positions are unmasked; uniform logits give
    token 0 and c = 1/V."""
    B, M, V, L = 1, 10, 512, 64
    logits = torch.zeros((B, M, V), dtype=torch.bfloat16, device=DEV)
    pos = torch.arange(3, 3 + 5 * M, 5, dtype=torch.int32, device=DEV).reshape(1, -1)
    mask = torch.ones((B, L), dtype=torch.uint8, device=DEV)
    conf = torch.zeros((B, L), dtype=torch.float32, device=DEV)
    tok = torch.full((B, L), -1, dtype=torch.int32, device=DEV)
    un = F().confidence_unmask(logits, pos, mask, conf, 4, tokens=tok)
    torch.cuda.synchronize()
    assert un[0].tolist() == pos[0, :4].tolist()
    assert tok[0, pos[0, :4].long()].tolist() == [0, 0, 0, 0]
    assert np.allclose(conf[0, pos[0, 4:].long()].cpu().numpy(), 1.0 / V, rtol=1e-6, atol=0)


def test_confidence_llada_vocabulary_256_rows():
    """The 32K step's 256 masked rows over a 126464-token vocabulary, bf16 logits, n(t) = 16."""
    from workloads import configs, synth
    wl = configs.CTX32K_STACK
    V = 126464
    _, mask_np = synth.step_inputs(wl)
    mask = torch.from_numpy(mask_np).to(DEV)
    pos = torch.from_numpy(np.flatnonzero(mask_np[0]).astype(np.int32)).reshape(1, -1).to(DEV)
    logits = synth.make_logits(1, pos.shape[1], V, seed=4, device=DEV)
    worst = run_case(logits, pos, mask, wl.n_t)
    log(f"confidence 32K masked rows, V={V}: worst relative error of c {worst:.2e}")
