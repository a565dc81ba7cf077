"""Seeded synthetic inputs for the sparse attention step.

This module only draws inputs: it holds none of the step's arithmetic.  Both
the fp64 oracle and the HIP path receive the arrays made here.

Recipe (shared by every workload in ``workloads.configs``):
  * Q, K, V entries are sigma * N(0, 1) with sigma = 1/8, drawn in fp32 by a
    seeded torch generator on the requested device, then rounded to bf16
    (round-to-nearest-even) for the bf16 workloads.  Draws on "cpu" and on
    "cuda" use different generators: a test compares two paths only on arrays
    drawn once and handed to both.
  * Attention sinks: a vector delta = 3*sigma*u, u in {-1, +1}^d (seeded,
    shared by every sink, head, layer and sequence), is added to the keys at
    the sink positions and to every query row.  Adding it to the keys alone
    leaves the sinks invisible to attention mass when queries are zero-mean,
    so the query offset is part of the reading.
  * Masked slots: `masked` of the G generation positions, drawn without
    replacement.  Prompt positions are never masked.
  * Confidence of the previous step: fp32, U(0,1) or Beta(2,5) on masked
    slots, 0 elsewhere.
  * Logits of the masked rows (the confidence and unmask step): sigma_z * N(0, 1) per
    vocabulary entry (fp32, then bf16 by round-to-nearest-even), plus a peak of
    2 + 6 u (u ~ U(0, 1)) at one seeded token of each row, so confidences spread
    from near 1/V to near 1.
  * Multi-step scenario (the batch-of-4 workload): after each step the
    model's new confidence is c_t = 0.9*c_{t-1} + 0.1*U(0,1) (fp32) and the
    decoder unmasks the n(t) masked positions with the highest c_t, lowest
    index first among equals.  This is the denoising scheduler around the
    step, not a step of the sparse attention path.

Every stream has its own seed, derived from (workload tag, seed, purpose,
indices) by SHA-256, so any one layer or step can be drawn alone.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

from .configs import Workload


def seed_of(wl: Workload, *parts) -> int:
    text = repr((wl.tag, wl.seed) + tuple(parts)).encode()
    return int.from_bytes(hashlib.sha256(text).digest()[:8], "little") & ((1 << 63) - 1)


def _np_rng(wl: Workload, *parts) -> np.random.Generator:
    return np.random.default_rng(seed_of(wl, *parts))


def _torch_gen(wl: Workload, device, *parts) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed_of(wl, *parts))
    return g


def torch_dtype(wl: Workload) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[wl.dtype]


# ---------------------------------------------------------------- small host-side state

def sink_positions(wl: Workload, b: int) -> np.ndarray:
    """Injected sink positions of sequence b, ascending (int64)."""
    if wl.sinks_fixed:
        return np.array(sorted(wl.sinks_fixed), dtype=np.int64)
    rng = _np_rng(wl, "sinks", b)
    return np.sort(rng.choice(wl.P, size=wl.n_sinks, replace=False)).astype(np.int64)


def sink_delta(wl: Workload) -> np.ndarray:
    """The shared sink offset 3*sigma*u, u in {-1,+1}^d (fp32)."""
    rng = _np_rng(wl, "delta")
    u = rng.integers(0, 2, size=wl.d) * 2 - 1
    return (3.0 * wl.sigma * u).astype(np.float32)


def initial_mask(wl: Workload, b: int) -> np.ndarray:
    """bool [L]: True where the slot is still [MASK] at the first step."""
    rng = _np_rng(wl, "mask", b)
    mask = np.zeros(wl.L, dtype=bool)
    mask[wl.P + rng.permutation(wl.G)[: wl.masked]] = True
    return mask


def initial_conf(wl: Workload, b: int, mask: np.ndarray) -> np.ndarray:
    """fp32 [L]: previous-step confidence on masked slots, 0 elsewhere."""
    rng = _np_rng(wl, "conf", b)
    if wl.conf == "uniform":
        vals = rng.random(wl.L, dtype=np.float32)
    elif wl.conf == "beta25":
        vals = rng.beta(2.0, 5.0, size=wl.L).astype(np.float32)
    else:
        raise ValueError(wl.conf)
    return np.where(mask, vals, np.float32(0.0)).astype(np.float32)


def scenario(wl: Workload, b: int):
    """Per-step (mask, previous confidence) of sequence b for all wl.steps steps.

    Entry t holds the mask at the start of step t and the confidence c_{t-1}
    that PCGI reads at step t.  The new confidence and the unmasking follow
    the scheduler rule stated in the module docstring.
    """
    mask = initial_mask(wl, b)
    conf = initial_conf(wl, b, mask)
    states = []
    for t in range(wl.steps):
        states.append((mask.copy(), conf.copy()))
        u = _np_rng(wl, "evolve", b, t).random(wl.L, dtype=np.float32)
        c_new = (np.float32(0.9) * conf + np.float32(0.1) * u).astype(np.float32)
        c_new = np.where(mask, c_new, np.float32(0.0)).astype(np.float32)
        idx = np.flatnonzero(mask)
        order = idx[np.lexsort((idx, -c_new[idx].astype(np.float64)))]
        mask = mask.copy()
        mask[order[: wl.n_t]] = False
        conf = np.where(mask, c_new, np.float32(0.0)).astype(np.float32)
    return states


def step_inputs(wl: Workload, step: int = 0):
    """(conf [B, L] fp32, mask [B, L] uint8) for one step of every sequence."""
    confs, masks = [], []
    for b in range(wl.B):
        m, c = scenario(wl, b)[step]
        confs.append(c)
        masks.append(m.astype(np.uint8))
    return np.stack(confs), np.stack(masks)


# ---------------------------------------------------------------- large tensors

def make_kv(wl: Workload, layer: int, device="cpu"):
    """K, V of one layer: [B, Hkv, L, d] in the workload dtype, sinks injected into K."""
    dev = torch.device(device)
    shape = (wl.B, wl.Hkv, wl.L, wl.d)
    k = torch.randn(shape, generator=_torch_gen(wl, dev, "k", layer), device=dev,
                    dtype=torch.float32)
    k.mul_(wl.sigma)
    delta = torch.from_numpy(sink_delta(wl)).to(dev)
    for b in range(wl.B):
        pos = torch.from_numpy(sink_positions(wl, b)).to(dev)
        k[b, :, pos, :] += delta
    v = torch.randn(shape, generator=_torch_gen(wl, dev, "v", layer), device=dev,
                    dtype=torch.float32)
    v.mul_(wl.sigma)
    dt = torch_dtype(wl)
    return k.to(dt).contiguous(), v.to(dt).contiguous()


def make_q(wl: Workload, layer: int, step: int = 0, device="cpu"):
    """Q of one layer and step for all L rows: [B, Hq, L, d], delta added to every row."""
    dev = torch.device(device)
    shape = (wl.B, wl.Hq, wl.L, wl.d)
    q = torch.randn(shape, generator=_torch_gen(wl, dev, "q", layer, step), device=dev,
                    dtype=torch.float32)
    q.mul_(wl.sigma)
    q += torch.from_numpy(sink_delta(wl)).to(dev)
    return q.to(torch_dtype(wl)).contiguous()


def sample_rows(n_rows: int, count: int, seed: int) -> np.ndarray:
    """Seeded ascending row sample that always holds the first and the last row."""
    rng = np.random.default_rng(seed)
    if count >= n_rows:
        return np.arange(n_rows, dtype=np.int64)
    mid = rng.choice(np.arange(1, n_rows - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, n_rows - 1], mid])).astype(np.int64)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of an fp32 or bf16 tensor to an fp64 numpy array on the host."""
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def make_logits(B: int, M: int, V: int, seed: int, device="cpu", dtype=torch.bfloat16, sigma_z: float = 1.0):
    """Logits [B, M, V] of M masked rows per sequence: sigma_z N(0, 1) plus one peak per row."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    z = torch.randn((B, M, V), generator=g, device=dev, dtype=torch.float32).mul_(sigma_z)
    peak_tok = torch.randint(0, V, (B, M, 1), generator=g, device=dev)
    peak = 2.0 + 6.0 * torch.rand((B, M, 1), generator=g, device=dev)
    z.scatter_add_(2, peak_tok, peak)
    return z.to(dtype).contiguous()


def make_dcu_inputs(B: int, NL: int, L: int, H: int, seed: int, device="cpu", dtype=torch.bfloat16,
                    unchanged: float = 0.25, zero_rows: int = 0):
    """Normalised layer inputs of two adjacent steps, (x_now, x_prev) [B, NL, L, H].

    x_prev ~ N(0, 1).  A token of layer l changes by sigma N(0, 1) with
    sigma = s_l exp(0.75 N(0, 1)), s_l rising from 0.02 at the first layer to 0.3 at the last
    (deeper layers change more); a share `unchanged` of the tokens keeps x_now == x_prev
    exactly (distance 0, so equal distances occur); `zero_rows` tokens per (b, l) are all
    zero in both steps.  Generated one layer at a time on `device`."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    x_now = torch.empty((B, NL, L, H), dtype=dtype, device=dev)
    x_prev = torch.empty((B, NL, L, H), dtype=dtype, device=dev)
    for b in range(B):
        for l in range(NL):
            s_l = 0.02 + 0.28 * (l / max(NL - 1, 1))
            y = torch.randn((L, H), generator=g, device=dev, dtype=torch.float32)
            sigma = s_l * torch.exp(0.75 * torch.randn((L, 1), generator=g, device=dev))
            sigma = sigma * (torch.rand((L, 1), generator=g, device=dev) >= unchanged)
            x = y + sigma * torch.randn((L, H), generator=g, device=dev, dtype=torch.float32)
            if zero_rows:
                rows = torch.randperm(L, generator=g, device=dev)[:zero_rows]
                x[rows] = 0.0
                y[rows] = 0.0
            x_prev[b, l] = y.to(dtype)
            x_now[b, l] = torch.where(sigma > 0, x, y).to(dtype)
    return x_now, x_prev


def make_key_tokens(B: int, n_keys: int, lo: int, hi: int, seed: int, pad: int = 0) -> np.ndarray:
    """[B, n_keys + pad] int32: n_keys distinct positions drawn from [lo, hi) per sequence
    (the tokens decoded at the step), in random order, then `pad` entries of -1."""
    rng = np.random.default_rng(seed)
    out = np.full((B, n_keys + pad), -1, dtype=np.int32)
    for b in range(B):
        out[b, :n_keys] = rng.choice(np.arange(lo, hi), size=n_keys, replace=False)
    return out
