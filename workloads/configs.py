"""The five synthetic workloads of the confidence-guided sparse attention step.

Each workload fixes the shape of one Focus-dLLM denoising step: prompt and
generation lengths, head layout, the PCGI parameters (n(t), rho, w), the block
size and top-C of block pruning, and the number of attention sinks.  The
parameter names follow the Focus-dLLM structured summary page
(paper.rainbus.top/paper/2602.02159), sections "Core method" and "Method steps":
k = floor(rho * n(t)) focus positions, windows of size w, blocks of prompt keys
represented by their mean key, top-C blocks, sinks found at layer l_dense.

Readings taken where the workload descriptions leave a value open:
  * the 32K Dream-shaped batch runs 28 layers (the depth of a Dream-7B-like
    model) with l_dense = 2, 16 sinks and 256 masked slots at the start;
  * the 32K LLaDA-shaped stack draws its confidence from Beta(2, 5), like the
    8K and 16K workloads;
  * sigma = 1/8 for every workload, and the sink offset is 3*sigma per element.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    tag: int                  # stream id mixed into every seed of this workload
    dtype: str                # "f32" or "bf16": the dtype of Q, K, V and O
    B: int                    # independent sequences
    P: int                    # prompt tokens
    G: int                    # generation-block tokens (the region after the prompt)
    masked: int               # generation slots still [MASK] at the first step
    Hq: int                   # query heads
    Hkv: int                  # key/value heads (Hq % Hkv == 0)
    d: int                    # head dim
    n_t: int                  # n(t): tokens decoded per step
    rho: float                # expansion factor (k = floor(rho * n(t)) is computed by each side itself)
    w: int                    # window size around each focus position
    bs: int                   # block size of the prompt partition
    C: int                    # blocks kept by top-C
    n_sinks: int              # sinks kept per sequence
    layers: int               # attention layers in one step
    l_dense: int              # dense layers in a sparse step; sinks come from the last one
    conf: str                 # "uniform" or "beta25" (confidence of masked slots)
    sinks_fixed: tuple = ()   # fixed sink positions (else drawn from [0, P))
    steps: int = 1            # denoising steps (first is a block-entry refresh when > 1)
    sigma: float = 1.0 / 8.0
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def L(self) -> int:
        return self.P + self.G

    @property
    def nb(self) -> int:
        return -(-self.P // self.bs)

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


TINY_2K_F32 = Workload(
    name="tiny_2k_f32_mha4_d64", tag=1, dtype="f32", B=1, P=1984, G=64, masked=32,
    Hq=4, Hkv=4, d=64, n_t=4, rho=2.0, w=8, bs=64, C=8, n_sinks=4, layers=1, l_dense=1,
    conf="uniform", sinks_fixed=(0, 1, 700, 1500), seed=0,
    notes="fp32, one layer; small enough for the oracle to finish in seconds")

CTX8K_MHA = Workload(
    name="ctx8k_mha32_d128_bf16", tag=2, dtype="bf16", B=1, P=7936, G=256, masked=128,
    Hq=32, Hkv=32, d=128, n_t=8, rho=2.0, w=16, bs=64, C=32, n_sinks=8, layers=1, l_dense=1,
    conf="beta25", notes="one sparse layer in LLaDA-8B attention shape")

CTX16K_GQA = Workload(
    name="ctx16k_gqa28x4_d128_bf16", tag=3, dtype="bf16", B=1, P=15872, G=512, masked=256,
    Hq=28, Hkv=4, d=128, n_t=16, rho=2.0, w=16, bs=128, C=32, n_sinks=8, layers=1, l_dense=1,
    conf="beta25", notes="one sparse layer in Dream-7B-like GQA shape")

CTX32K_STACK = Workload(
    name="ctx32k_mha32_d128_bf16_32layers", tag=4, dtype="bf16", B=1, P=32256, G=512,
    masked=256, Hq=32, Hkv=32, d=128, n_t=16, rho=2.0, w=32, bs=128, C=64, n_sinks=16,
    layers=32, l_dense=2, conf="beta25",
    notes="full 32-layer stack in LLaDA-8B shape; sinks found at layer 2, reused by 3..32")

CTX32K_GQA_B4 = Workload(
    name="ctx32k_gqa28x4_d128_bf16_batch4", tag=5, dtype="bf16", B=4, P=32256, G=512,
    masked=256, Hq=28, Hkv=4, d=128, n_t=16, rho=2.0, w=32, bs=128, C=64, n_sinks=16,
    layers=28, l_dense=2, conf="beta25", steps=8,
    notes="batch of 4; one block-entry dense refresh then 7 sparse steps")

# The pages' own hyper-parameters (Summary, "Reproducibility": rho = 4, w = 8, l_dense = 6,
# blocks of 64, sparsity ratio alpha = 0.5, N_sinks = 0.01 M) on the 32K LLaDA-shaped stack:
# nb = 504 blocks, of which alpha = 0.5 prunes 252 (C = 252), and N_sinks = floor(0.01 L) = 327.
CTX32K_PAPER = Workload(
    name="ctx32k_mha32_d128_bf16_paper_defaults", tag=6, dtype="bf16", B=1, P=32256, G=512,
    masked=256, Hq=32, Hkv=32, d=128, n_t=16, rho=4.0, w=8, bs=64, C=252, n_sinks=327,
    layers=32, l_dense=6, conf="beta25",
    notes="the pages' default hyper-parameters at 32K, with all 327 sink positions injected")

ALL = (TINY_2K_F32, CTX8K_MHA, CTX16K_GQA, CTX32K_STACK, CTX32K_GQA_B4)
PRESETS = (CTX32K_PAPER,)
BY_NAME = {w.name: w for w in ALL + PRESETS}
