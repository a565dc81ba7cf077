"""Mistakes planted in the oracle (on the CPU) must each fail at least one pin.

Each mutation replaces one oracle function with a plausible wrong version (a
dropped term, a wrong index or sign, a transposed operand, a wrong tie-break)
and runs the pins; the test passes only if some pin raises.
"""
import numpy as np
import pytest

import oracle_checks
from oracle import focus_oracle as O

_orig = {name: getattr(O, name) for name in dir(O) if callable(getattr(O, name))}


def _rank_highest_index(values, candidates, count):
    ranked = sorted((int(i) for i in candidates), key=lambda i: (-float(values[i]), -i))
    return np.array(sorted(ranked[: max(count, 0)]), dtype=np.int64)


def _rank_smallest(values, candidates, count):
    ranked = sorted((int(i) for i in candidates), key=lambda i: (float(values[i]), i))
    return np.array(sorted(ranked[: max(count, 0)]), dtype=np.int64)


def _window_shifted(focus, w, L):
    return _orig["window_active"]([p + 1 for p in focus], w, L)


def _window_centered(focus, w, L):
    members = set()
    for p in focus:
        for j in range(int(p) - w // 2, int(p) + w // 2 + 1):
            if 0 <= j < L:
                members.add(j)
    return np.array(sorted(members), dtype=np.int64)


def _block_means_by_bs(K, P, bs):
    K = np.asarray(K, dtype=np.float64)
    nb = -(-P // bs)
    out = np.zeros((K.shape[0], nb, K.shape[2]))
    for b in range(nb):
        out[:, b] = K[:, b * bs:min((b + 1) * bs, P)].sum(axis=1) / bs
    return out


def _relevance_first_head(Q, kbar, scale):
    return _orig["block_relevance"](np.asarray(Q)[:1], kbar[:1], scale)


def _key_set_no_gen(sinks, blocks, bs, P, L):
    return _orig["key_set"](sinks, blocks, bs, P, P)


def _key_set_block_shift(sinks, blocks, bs, P, L):
    return _orig["key_set"](sinks, [b + 1 for b in blocks if b + 1 < -(-P // bs)], bs, P, L)


def _refreshed_blocks_no_prompt_bound(rows, P, bs):
    return np.array(sorted({int(r) // bs for r in rows if int(r) >= 0}), dtype=np.int64)


def _refreshed_blocks_ceil(rows, P, bs):
    return np.array(sorted({-(-int(r) // bs) for r in rows if 0 <= int(r) < P}), dtype=np.int64)


def _confidence_max_logit(z):
    z = np.asarray(z, dtype=np.float64)
    return float(z.max()), int(np.argmax(z))


def _confidence_argmax_last(z):
    c, _ = _orig["token_confidence"](z)
    z = np.asarray(z, dtype=np.float64)
    return c, int(np.flatnonzero(z == z.max())[-1])


def _unmask_least_confident(logits, positions, mask, n_t):
    conf, tokens, _ = _orig["unmask_step"](logits, positions, mask, n_t)
    cand = [r for r in range(len(positions)) if mask[int(positions[r])]]
    ranked = sorted(cand, key=lambda r: (conf[r], int(positions[r])))
    return conf, tokens, np.array(sorted(int(positions[r]) for r in ranked[:max(n_t, 0)]), dtype=np.int64)


def _unmask_ignores_mask(logits, positions, mask, n_t):
    return _orig["unmask_step"](logits, positions, np.ones(len(mask), dtype=bool), n_t)


def _dcu_similarity(x, y):
    return 1.0 - _orig["dcu_distance"](x, y)


def _dcu_budget_floor_only(activity, total):
    a = np.asarray(activity, dtype=np.float64)
    return np.floor(total * a / a.sum() if a.sum() > 0 else np.full(len(a), total / len(a))).astype(np.int64)


def _dcu_budget_highest_layer_first(activity, total):
    a = np.asarray(activity, dtype=np.float64)
    q = np.full(len(a), total / len(a)) if a.sum() <= 0 else total * a / a.sum()
    base = np.floor(q).astype(np.int64)
    frac = q - base
    for l in sorted(range(len(a)), key=lambda l: (-frac[l], -l))[: total - int(base.sum())]:
        base[l] += 1
    return base


def _dcu_set_without_window(d, mandatory, budget):
    return _orig["dcu_update_set"](d, [], budget)


def _per_head_modulo_group(Q, kbar, scale):
    Q = np.asarray(Q, dtype=np.float64)
    Hq, Hkv = Q.shape[0], kbar.shape[0]
    R = np.zeros((Hkv, kbar.shape[1]))
    for h in range(Hq):
        R[h % Hkv] += (Q[h] @ kbar[h % Hkv].T).sum(axis=0)
    return R * scale


def _max_is_min(Q, kbar, scale, per_head=False):
    return -_orig["block_relevance_max"](-np.asarray(Q), kbar, scale, per_head)


def _max_is_sum(Q, kbar, scale, per_head=False):
    return (_orig["block_relevance_per_head"](Q, kbar, scale) if per_head
            else _orig["block_relevance"](Q, kbar, scale))


def _blocks_kept_is_pruned(nb, alpha):
    return int(np.floor(alpha * nb))


def _sinks_of_prompt(L):
    return _orig["paper_sink_count"](L - 512)


def _per_head_attention_first_key_set(Q, K, V, key_sets, scale):
    return _orig["sparse_attention"](Q, K, V, key_sets[0], scale)


MUTATIONS = {
    "tie_break_highest_index": ("rank_select", _rank_highest_index),
    "select_smallest": ("rank_select", _rank_smallest),
    "pcgi_ignores_mask": ("pcgi_focus",
                          lambda conf, mask, k: _orig["rank_select"](
                              np.asarray(conf, np.float32), range(len(mask)), k)),
    "focus_count_round": ("focus_count", lambda n_t, rho: int(round(rho * n_t))),
    "window_shifted": ("window_active", _window_shifted),
    "window_centered_2h_plus_1": ("window_active", _window_centered),
    "gqa_modulo_mapping": ("kv_head", lambda h, Hq, Hkv: h % Hkv),
    "attention_no_scale": ("attention", lambda Q, K, V, s: _orig["attention"](Q, K, V, 1.0)),
    "attention_k_v_swapped": ("attention", lambda Q, K, V, s: _orig["attention"](Q, V, K, s)),
    "sink_scores_unnormalised": ("sink_scores",
                                 lambda Q, K, lse, s: _orig["sink_scores"](
                                     Q, K, np.zeros_like(np.asarray(lse)), s)),
    "sink_scores_dropped_head": ("sink_scores",
                                 lambda Q, K, lse, s: _orig["sink_scores"](
                                     np.asarray(Q)[1:], K[1:] if len(K) > 1 else K,
                                     np.asarray(lse)[1:], s)),
    "block_means_divide_by_bs": ("block_means", _block_means_by_bs),
    "relevance_first_head_only": ("block_relevance", _relevance_first_head),
    "relevance_sign_flipped": ("block_relevance",
                               lambda Q, kbar, s: -_orig["block_relevance"](Q, kbar, s)),
    "key_set_without_generation_region": ("key_set", _key_set_no_gen),
    "key_set_block_off_by_one": ("key_set", _key_set_block_shift),
    "refreshed_blocks_past_prompt": ("refreshed_blocks", _refreshed_blocks_no_prompt_bound),
    "refreshed_blocks_rounded_up": ("refreshed_blocks", _refreshed_blocks_ceil),
    "confidence_is_max_logit": ("token_confidence", _confidence_max_logit),
    "confidence_argmax_last_tie": ("token_confidence", _confidence_argmax_last),
    "unmask_least_confident": ("unmask_step", _unmask_least_confident),
    "unmask_ignores_mask": ("unmask_step", _unmask_ignores_mask),
    "per_head_relevance_modulo_group": ("block_relevance_per_head", _per_head_modulo_group),
    "max_relevance_is_min": ("block_relevance_max", _max_is_min),
    "max_relevance_is_sum": ("block_relevance_max", _max_is_sum),
    "blocks_kept_is_pruned_count": ("blocks_kept", _blocks_kept_is_pruned),
    "sink_count_of_prompt": ("paper_sink_count", _sinks_of_prompt),
    "per_head_attention_one_key_set": ("sparse_attention_per_head", _per_head_attention_first_key_set),
    "dcu_similarity_not_distance": ("dcu_distance", _dcu_similarity),
    "dcu_budget_floor_only": ("dcu_budgets", _dcu_budget_floor_only),
    "dcu_budget_ties_to_higher_layer": ("dcu_budgets", _dcu_budget_highest_layer_first),
    "dcu_set_without_mandatory_window": ("dcu_update_set", _dcu_set_without_window),
    "sparse_ignores_key_set": ("sparse_attention",
                               lambda Q, K, V, I_p, s: _orig["attention"](Q, K, V, s)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setattr(O, attr, bad)
    caught = []
    for check in oracle_checks.ALL_CHECKS:
        try:
            check()
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
            break
    assert caught, f"no pin catches the planted mistake {name}"
