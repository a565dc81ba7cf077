"""Plain fp64 CPU oracle of one Focus-dLLM sparse denoising step.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the entry module and
the CPU-baseline leg of the benchmark may import or run this file.  It shares
no code with the HIP library: the two meet only in the arrays drawn by
``workloads.synth``.  It is deliberately slow and literal: each function is
the definition written out in fp64 NumPy (plain Python where the definition is
a selection), with no blocking, fusion or reordering beyond it.

Citations.  "Summary" is the structured summary of the paper "Focus-dLLM:
Accelerating Long-Context Diffusion LLM Inference via Confidence-Guided
Context Focusing" at paper.rainbus.top/paper/2602.02159.  Its sections used
here: "Prerequisites" (前置知识, with the sub-sections on dLLMs, attention
sinks, the approximate KV cache and semi-autoregressive remasking), "Core
method" (核心方法), "Method steps" (方法步骤详情, numbered (1)-(5)) and
"Reproducibility" (复现评估).  "Abstract" is the paper's abstract at
paperdance.org/p/2602.02159.

Numeric model.  Inputs arrive as the exact fp64 upcast of the fp32 or bf16
arrays the GPU receives.  Confidences are compared as the fp32 values given.
Selections order by value, larger first, then by lower index.

Readings (the pages leave these open; each is fixed here and listed with its
reason in the design notes):
  R1 window: exactly w positions [p - floor(w/2), p - floor(w/2) + w), clipped
     to [0, L).
  R2 attention: scale 1/sqrt(d), no mask (bidirectional), query head h reads
     KV head floor(h * Hkv / Hq); inputs are already rotary-embedded.
  R3 sinks: score_j = sum over heads and active queries of the normalised
     attention probability of key j at layer l_dense; the n_sinks largest win.
  R4 relevance: R_b = scale * sum over heads h and active queries i of
     q_{h,i} . kbar_{g(h),b}; one block set per sequence and layer, shared by
     all heads.
  R5 key set: I_p = I_sink U (selected prompt blocks) U [P, L), each key once.
     Without the generation region, attention with every block kept and a
     window covering the sequence could not equal dense attention.
  R13 alpha: the share of prompt blocks pruned, C = nb - floor(alpha nb).
  R14 N_sinks = floor(0.01 L) (the pages' M read as the sequence length).
  R15 dense tail: the last layers of a step attend densely (the pages report that
     Dream needs its last 4 layers kept).
  R16 per-KV-head blocks: R_{g,b} sums over the query heads of KV head g only, and
     each KV head keeps its own top-C; its query heads attend over its own I_p.
  R17 max aggregator: R_b = scale * max over heads and queries of q . kbar.
  R12 confidence: the largest softmax probability of a masked position's
     predicted distribution; its argmax (lowest id among equal maxima) is the
     predicted token; the n(t) most confident masked rows are unmasked.
  D1-D4 (the DCU workload of the fifth page): cosine distance of the normalised
     inputs, proportional budgets by largest remainder, mandatory windows around
     given key tokens, top-budget of the other tokens.

Pins (tests marked "not gpu"): brute-force dominance and exhaustive subset
checks for every selection, exact rational block means, closed-form and
hand-worked attention fixtures, a library softmax/attention routine on small
inputs, the sparse == dense reduction, recovery of injected sinks, and the KV
refresh against the identity refresh and the incremental block-means formula.  The
pages print no worked example, so no pin holds a value printed on a page.
Parity of the readings R1, R3, R4, R5 against the authors' own code is
unpinned: the pins fix the oracle to these readings, not the readings to the
paper.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


# ------------------------------------------------------------------ selections

def focus_count(n_t: int, rho: float) -> int:
    """k = floor(rho * n(t)), in double precision.

    Summary, "Core method": the indicator keeps the top-k masked positions,
    k = floor(rho * n(t)), rho a preset expansion factor and n(t) the number
    of tokens decoded at step t.
    """
    return int(math.floor(float(rho) * int(n_t)))


def rank_select(values, candidates, count: int) -> np.ndarray:
    """The `count` candidates with the largest value, lower index first on equal
    values, returned in ascending index order.  Fewer candidates: all of them."""
    ranked = sorted((int(i) for i in candidates), key=lambda i: (-float(values[i]), i))
    return np.array(sorted(ranked[: max(count, 0)]), dtype=np.int64)


def pcgi_focus(conf, mask, k: int) -> np.ndarray:
    """I_focus: the k still-masked positions with the highest previous confidence.

    Summary, "Core method" and "Method steps" (1): among all positions still
    [MASK], take the top-k by the previous step's confidence c_{t-1}.
    """
    conf = np.asarray(conf, dtype=np.float32)
    candidates = [i for i in range(len(mask)) if mask[i]]
    return rank_select(conf, candidates, k)


def window_active(focus, w: int, L: int) -> np.ndarray:
    """I_active: the union of a window of w positions around each focus position.

    Summary, "Method steps" (2): each candidate is widened to a local window of
    size w.  Reading R1 places floor(w/2) positions before p.
    """
    half = w // 2
    members = set()
    for p in focus:
        start = int(p) - half
        for j in range(start, start + w):
            if 0 <= j < L:
                members.add(j)
    return np.array(sorted(members), dtype=np.int64)


# ------------------------------------------------------------------ attention

def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h (grouped-query attention, reading R2)."""
    return (h * Hkv) // Hq


def attention(Q, K, V, scale: float):
    """softmax(Q K^T * scale) V per head, with its log-sum-exp.

    Q [Hq, n, d], K and V [Hkv, m, d] (fp64) -> O [Hq, n, d], lse [Hq, n].
    No mask: dLLM attention is bidirectional (Summary, "Prerequisites", dLLMs).
    An empty key set gives O = 0 and lse = -inf.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, n, d = Q.shape
    Hkv, m = K.shape[0], K.shape[1]
    O = np.zeros((Hq, n, V.shape[2]))
    lse = np.full((Hq, n), -np.inf)
    if m == 0 or n == 0:
        return O, lse
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        S = (Q[h] @ K[g].T) * scale
        top = S.max(axis=1, keepdims=True)
        E = np.exp(S - top)
        Z = E.sum(axis=1, keepdims=True)
        O[h] = (E / Z) @ V[g]
        lse[h] = (top + np.log(Z))[:, 0]
    return O, lse


def dense_attention(Q_rows, K, V, scale: float):
    """Full attention of the given query rows over all L keys.

    Summary, "Method steps": at a block-entry step the whole sequence attends
    densely (use_sparse = False); in the other steps the first l_dense layers
    run full attention (step (3)), here for the active query rows.
    """
    return attention(Q_rows, K, V, scale)


# ------------------------------------------------------------------ sinks

def sink_scores(Q_rows, K, lse, scale: float) -> np.ndarray:
    """Attention mass each key receives at layer l_dense, summed over heads and rows.

    Summary, "Prerequisites" (attention sinks draw a disproportionate share of
    attention) and "Method steps" (3) (layer l_dense's attention distribution
    identifies the sinks).  Reading R3: score_j = sum_h sum_i
    exp(q_{h,i} . k_{g(h),j} * scale - lse_{h,i}).
    """
    Q_rows = np.asarray(Q_rows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    Hq, Hkv = Q_rows.shape[0], K.shape[0]
    score = np.zeros(K.shape[1])
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        S = (Q_rows[h] @ K[g].T) * scale
        score += np.exp(S - np.asarray(lse[h], dtype=np.float64)[:, None]).sum(axis=0)
    return score


def sink_select(scores, n_sinks: int) -> np.ndarray:
    """I_sink: the n_sinks keys with the largest score, ascending."""
    return rank_select(scores, range(len(scores)), n_sinks)


# ------------------------------------------------------------------ block pruning

def block_means(K, P: int, bs: int) -> np.ndarray:
    """Representative key of each prompt block: the mean of its keys.

    Summary, "Method steps" (4): prompt tokens are split into contiguous
    blocks, each represented by the mean of its keys.  K [Hkv, L, d] ->
    kbar [Hkv, nb, d], nb = ceil(P / bs); a shorter last block is averaged over
    its own keys.
    """
    K = np.asarray(K, dtype=np.float64)
    nb = -(-P // bs)
    kbar = np.zeros((K.shape[0], nb, K.shape[2]))
    for b in range(nb):
        lo, hi = b * bs, min((b + 1) * bs, P)
        kbar[:, b] = K[:, lo:hi].sum(axis=1) / (hi - lo)
    return kbar


def kv_refresh(K, V, rows, K_new, V_new):
    """The approximate KV cache after one refresh: the rows of U(t) take their recomputed
    keys and values, every other row keeps its cached ones.

    Summary, "Prerequisites" (approximate KV cache): K_i = f_K(x^(t))_i for i in U(t),
    otherwise the cached value; the same for V.  K, V [Hkv, L, d]; rows the positions of
    U(t) (distinct; entries outside [0, L) are ignored); K_new, V_new [Hkv, len(rows), d],
    column j holding the new row of position rows[j].  Returns new arrays.
    """
    K2 = np.array(K, dtype=np.float64, copy=True)
    V2 = np.array(V, dtype=np.float64, copy=True)
    L = K2.shape[1]
    for j, r in enumerate(rows):
        r = int(r)
        if 0 <= r < L:
            K2[:, r] = np.asarray(K_new, dtype=np.float64)[:, j]
            V2[:, r] = np.asarray(V_new, dtype=np.float64)[:, j]
    return K2, V2


def refreshed_blocks(rows, P: int, bs: int) -> np.ndarray:
    """The prompt blocks holding a refreshed row: the only block means a refresh can change
    (Summary, "Method steps" (4): a block's representative is the mean of its own keys)."""
    return np.array(sorted({int(r) // bs for r in rows if 0 <= int(r) < P}), dtype=np.int64)


def block_relevance(Q_rows, kbar, scale: float) -> np.ndarray:
    """R_b between the active queries and each block's mean key (reading R4).

    Summary, "Method steps" (4): relevance scores between the candidate queries
    and every block are computed and the top-C blocks kept.
    """
    Q_rows = np.asarray(Q_rows, dtype=np.float64)
    Hq, Hkv = Q_rows.shape[0], kbar.shape[0]
    R = np.zeros(kbar.shape[1])
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        R += (Q_rows[h] @ kbar[g].T).sum(axis=0)
    return R * scale


def top_blocks(R, C: int) -> np.ndarray:
    """The C blocks of highest relevance, ascending (all blocks when C >= nb)."""
    return rank_select(R, range(len(R)), C)


def block_relevance_per_head(Q_rows, kbar, scale: float) -> np.ndarray:
    """R_{g,b} for per-KV-head block selection (reading R16): the part of R_b that the
    query heads of KV head g contribute, R_{g,b} = scale * sum over h with g(h) = g and
    active queries i of q_{h,i} . kbar_{g,b}.  Returns [Hkv, nb]; summed over g it is R_b.

    Summary, "Method steps" (4) scores the blocks against the candidate queries; the
    per-head form keeps one block set per KV head instead of one shared by all heads.
    """
    Q_rows = np.asarray(Q_rows, dtype=np.float64)
    Hq, Hkv = Q_rows.shape[0], kbar.shape[0]
    R = np.zeros((Hkv, kbar.shape[1]))
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        R[g] += (Q_rows[h] @ kbar[g].T).sum(axis=0)
    return R * scale


def block_relevance_max(Q_rows, kbar, scale: float, per_head: bool = False) -> np.ndarray:
    """The max aggregator of the relevance (reading R17): a block scores by its strongest
    single query, R_b = scale * max over heads h and active queries i of
    q_{h,i} . kbar_{g(h),b} ([nb]), or per KV head over the heads of g only ([Hkv, nb]).
    With no active query every block scores -inf.

    Summary, "Independent weaknesses": the block representative and the summed relevance
    can wash out a block that matters to a few queries only; this variant keeps such a
    block's strongest match.
    """
    Q_rows = np.asarray(Q_rows, dtype=np.float64)
    Hq, Hkv, nb = Q_rows.shape[0], kbar.shape[0], kbar.shape[1]
    R = np.full((Hkv, nb), -np.inf)
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        if Q_rows.shape[1]:
            R[g] = np.maximum(R[g], (Q_rows[h] @ kbar[g].T).max(axis=0))
    R = R * scale
    return R if per_head else R.max(axis=0)


def blocks_kept(nb: int, alpha: float) -> int:
    """Top-C from the sparsity ratio alpha (reading R13): alpha is the share of prompt
    blocks pruned, so C = nb - floor(alpha * nb) are kept (the pages' default 0.5 keeps
    half).  Summary, "Reproducibility" and "Limitations" list alpha among the
    hyper-parameters without a formula."""
    return int(nb) - int(math.floor(float(alpha) * int(nb)))


def paper_sink_count(L: int) -> int:
    """N_sinks = floor(0.01 * M) with M read as the sequence length L (reading R14);
    Summary, "Reproducibility"."""
    return int(math.floor(0.01 * int(L)))


def key_set(sinks, blocks, bs: int, P: int, L: int) -> np.ndarray:
    """I_p: sinks, the keys of the selected prompt blocks and the generation region.

    Summary, "Method steps" (5): the sink set and the selected prompt blocks
    form I_p; the generation region [P, L) is added by reading R5.  Each key
    appears once, ascending.
    """
    keys = set(int(j) for j in sinks if j >= 0)
    for b in blocks:
        if b >= 0:
            keys.update(range(int(b) * bs, min((int(b) + 1) * bs, P)))
    keys.update(range(P, L))
    return np.array(sorted(keys), dtype=np.int64)


def sparse_attention(Q_rows, K, V, I_p, scale: float):
    """Attention of the active queries over the key/value pairs in I_p only.

    Summary, "Method steps" (5): sparse attention is computed only over the
    key-value pairs of I_p.
    """
    I_p = np.asarray(I_p, dtype=np.int64)
    return attention(Q_rows, np.asarray(K)[:, I_p], np.asarray(V)[:, I_p], scale)


def sparse_attention_per_head(Q_rows, K, V, key_sets, scale: float):
    """Sparse attention with one key set per KV head: query head h attends over the keys
    of key_sets[g(h)] only (reading R16).  Returns (O [Hq, n, d], lse [Hq, n])."""
    Q_rows = np.asarray(Q_rows, dtype=np.float64)
    Hq, Hkv = Q_rows.shape[0], len(key_sets)
    O = np.zeros(Q_rows.shape)
    lse = np.zeros(Q_rows.shape[:2])
    for h in range(Hq):
        g = kv_head(h, Hq, Hkv)
        I_p = np.asarray(key_sets[g], dtype=np.int64)
        O[h:h + 1], lse[h:h + 1] = attention(Q_rows[h:h + 1], np.asarray(K)[g:g + 1, I_p],
                                             np.asarray(V)[g:g + 1, I_p], scale)
    return O, lse


# ------------------------------------------------------------------ confidence and unmasking

def token_confidence(logits_row):
    """Confidence and predicted token of one masked position.

    Summary, "Prerequisites" (dLLMs): at every denoising step the model gives each
    [MASK] position a probability distribution over the vocabulary and positions are
    unmasked by their confidence.  Reading R12: the confidence is the largest softmax
    probability, c = max_v exp(z_v) / sum_u exp(z_u), and the predicted token is the
    argmax (the lowest token id among equal maxima).  Returns (c, token) in fp64.
    """
    z = np.asarray(logits_row, dtype=np.float64)
    top = z.max()
    token = int(np.flatnonzero(z == top)[0])
    return 1.0 / np.exp(z - top).sum(), token


def unmask_step(logits, positions, mask, n_t: int):
    """One unmasking decision: the confidence c_t of the listed positions and the n(t) of
    them that are unmasked.

    Summary, "Prerequisites" (dLLMs: positions are unmasked by confidence) and "Core
    method" (n(t) is the number of tokens decoded at step t; c_t is the confidence PCGI
    reads at step t+1).  logits [M, V] are the rows of `positions` [M].  Among the rows
    whose position is still masked, the n(t) with the highest confidence are unmasked
    (the lower position first among equal confidences).  Returns (conf, tokens, chosen):
    conf [M] and tokens [M] per row, chosen the unmasked positions, ascending.
    """
    conf = np.zeros(len(positions))
    tokens = np.zeros(len(positions), dtype=np.int64)
    for r, z in enumerate(logits):
        conf[r], tokens[r] = token_confidence(z)
    cand = [r for r in range(len(positions)) if mask[int(positions[r])]]
    ranked = sorted(cand, key=lambda r: (-conf[r], int(positions[r])))
    chosen = np.array(sorted(int(positions[r]) for r in ranked[: max(n_t, 0)]), dtype=np.int64)
    return conf, tokens, chosen


# ------------------------------------------------------------------ dynamic cache update (DCU)
#
# The fifth page (the Dynamic-dLLM article, section "DCU：动态缓存更新") describes a second
# data-parallel workload: which tokens' caches a layer refreshes.  Readings D1-D4 are
# listed in the design notes.

def dcu_distance(x_now, x_prev) -> np.ndarray:
    """Per-token change of a layer's normalised input between adjacent steps (reading D1).

    DCU section: the cosine distance between the normalised token inputs of adjacent
    steps measures how much a token's representation changed.  x_now, x_prev [L, H] ->
    d [L] = 1 - x.y / (|x| |y|), with d = 0 where a norm is zero.
    """
    x = np.asarray(x_now, dtype=np.float64)
    y = np.asarray(x_prev, dtype=np.float64)
    d = np.zeros(x.shape[0])
    for i in range(x.shape[0]):
        nx, ny = math.sqrt(float(x[i] @ x[i])), math.sqrt(float(y[i] @ y[i]))
        if nx > 0.0 and ny > 0.0:
            d[i] = 1.0 - float(x[i] @ y[i]) / (nx * ny)
    return d


def dcu_budgets(activity, total: int) -> np.ndarray:
    """Split of the update budget over layers in proportion to their activity (reading D2).

    DCU section: token-level changes are summed into each layer's activity and the total
    update budget is tilted towards the layers that changed most.  Layer l gets
    floor(total a_l / sum a) tokens; the rest go one each to the layers with the largest
    fractional parts (the lower layer first among equal parts); equal shares when every
    activity is zero.
    """
    a = np.asarray(activity, dtype=np.float64)
    A = a.sum()
    q = np.full(len(a), total / len(a)) if A <= 0.0 else total * a / A
    base = np.floor(q).astype(np.int64)
    frac = q - base
    order = sorted(range(len(a)), key=lambda l: (-frac[l], l))
    for l in order[: total - int(base.sum())]:
        base[l] += 1
    return base


def dcu_mandatory(key_tokens, w_m: int, L: int) -> np.ndarray:
    """The mandatory update window (reading D3): w_m positions around each key token,
    [c - floor(w_m/2), c - floor(w_m/2) + w_m) clipped to [0, L), ascending (the same
    placement as the PCGI windows)."""
    return window_active([c for c in key_tokens if c >= 0], w_m, L)


def dcu_update_set(d, mandatory, budget: int) -> np.ndarray:
    """One layer's update set (reading D4): the mandatory window and the `budget` other
    tokens of largest change (the lower position first among equal changes), ascending."""
    must = set(int(j) for j in mandatory)
    rest = [j for j in range(len(d)) if j not in must]
    picked = rank_select(d, rest, budget)
    return np.array(sorted(must | set(int(j) for j in picked)), dtype=np.int64)


def dcu_select(x_now, x_prev, key_tokens, w_m: int, total: int):
    """Every layer's update set of one sequence: x_now, x_prev [layers, L, H].
    Returns (d [layers, L], activity [layers], budgets [layers], sets [list of arrays])."""
    layers, L = np.asarray(x_now).shape[:2]
    d = np.stack([dcu_distance(x_now[l], x_prev[l]) for l in range(layers)])
    activity = d.sum(axis=1)
    budgets = dcu_budgets(activity, total)
    must = dcu_mandatory(key_tokens, w_m, L)
    return d, activity, budgets, [dcu_update_set(d[l], must, int(budgets[l])) for l in range(layers)]


# ------------------------------------------------------------------ one step

@dataclass
class SparseStep:
    focus: np.ndarray
    active: np.ndarray
    sinks: np.ndarray = None
    sink_scores: np.ndarray = None
    blocks: dict = field(default_factory=dict)     # layer -> selected blocks
    relevance: dict = field(default_factory=dict)  # layer -> R
    out: dict = field(default_factory=dict)        # layer -> O [Hq, n_active, d]
    lse: dict = field(default_factory=dict)        # layer -> lse [Hq, n_active]


def sparse_step(conf, mask, layer_inputs, *, layers: int, l_dense: int, n_t: int,
                rho: float, w: int, P: int, bs: int, C: int, n_sinks: int,
                scale: float, layer_subset=None, dense_tail: int = 0, per_head: bool = False,
                aggregator: str = "sum") -> SparseStep:
    """One non-block-entry denoising step of one sequence, in the pages' order.

    Summary, "Method steps" (1)-(5): PCGI focus, window expansion, dense
    layers 1..l_dense (sinks from layer l_dense), then per deeper layer block
    means, top-C relevance, the key set and sparse attention.
    `layer_inputs(l)` returns (Q [Hq, L, d], K [Hkv, L, d], V [Hkv, L, d]) of
    layer l (0-based).  `layer_subset` limits which layers are evaluated; the
    layer l_dense - 1 is always evaluated because the sinks come from it.
    A one-layer step (layers == l_dense == 1) uses that layer both ways.

    Variants (Summary, "Independent weaknesses" and "Reproducibility"): the last
    `dense_tail` layers attend densely like the first l_dense (reading R15); `per_head`
    keeps one block set per KV head (R16, blocks[l] is then [Hkv, C]); `aggregator`
    "max" scores a block by its strongest query (R17) instead of the sum.
    """
    L = len(mask)
    st = SparseStep(focus=pcgi_focus(conf, mask, focus_count(n_t, rho)), active=None)
    st.active = window_active(st.focus, w, L)
    wanted = set(range(layers)) if layer_subset is None else set(layer_subset)
    wanted.add(l_dense - 1)
    for l in sorted(wanted):
        Q, K, V = layer_inputs(l)
        Qa = np.asarray(Q, dtype=np.float64)[:, st.active]
        if l < l_dense or l >= layers - dense_tail:
            st.out[l], st.lse[l] = dense_attention(Qa, K, V, scale)
            if l == l_dense - 1:
                st.sink_scores = sink_scores(Qa, K, st.lse[l], scale)
                st.sinks = sink_select(st.sink_scores, n_sinks)
        if (l_dense <= l < layers - dense_tail) or layers == l_dense == 1:
            kbar = block_means(K, P, bs)
            if aggregator == "max":
                R = block_relevance_max(Qa, kbar, scale, per_head=per_head)
            elif per_head:
                R = block_relevance_per_head(Qa, kbar, scale)
            else:
                R = block_relevance(Qa, kbar, scale)
            st.relevance[l] = R
            key = l if l >= l_dense else ("sparse", l)
            if per_head:
                st.blocks[l] = np.stack([top_blocks(R[g], C) for g in range(R.shape[0])])
                sets = [key_set(st.sinks, st.blocks[l][g], bs, P, L) for g in range(R.shape[0])]
                st.out[key], st.lse[key] = sparse_attention_per_head(Qa, K, V, sets, scale)
            else:
                st.blocks[l] = top_blocks(R, C)
                I_p = key_set(st.sinks, st.blocks[l], bs, P, L)
                st.out[key], st.lse[key] = sparse_attention(Qa, K, V, I_p, scale)
    return st
