"""The five verification workloads, as shapes and distribution parameters.

Each workload is one tree-verification step of EAGLE-style speculative
sampling at the attention shape of a public model family (LLaMA2-7B/13B/70B,
Mixtral-8x7B).  The shapes are those of the models the EAGLE pages evaluate
(EAGLE, paperlayer.ai summary of arXiv 2401.15077, §4 Experiments); the
distributions are synthetic stand-ins, since no weights or datasets are used.

Fields follow the notation used throughout the package:
  B batch, Hq/Hkv query/KV heads, d head dim, L committed KV length,
  N draft-tree nodes including the root, V vocabulary size,
  sigma_t std-dev of the target logits, sigma_d std-dev of the draft noise
  (draft logits = target logits + N(0, sigma_d^2)).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class VerifyConfig:
    index: int
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    L: int
    N: int
    V: int
    sigma_t: float
    sigma_d: float
    temperatures: tuple
    tree: str            # "random" | "static" | "eagle2"
    max_depth: int
    qkv_sigma: float = 1.0
    topk: int = 10       # eagle2 expansion width
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def Lmax(self) -> int:
        return self.L + self.N

    def attn_bytes(self) -> int:
        """Algorithmic HBM bytes of one tree-attention launch.

        KV prefix read once per KV head, the tree's own K/V rows, Q read and
        O written (all bf16), plus the 64-bit ancestor mask of every node.
        """
        kv_prefix = self.B * self.Hkv * self.L * self.d * 2 * 2
        kv_tree = self.B * self.Hkv * self.N * self.d * 2 * 2
        q_and_o = self.B * self.N * self.Hq * self.d * 2 * 2
        mask = self.B * self.N * 8
        return kv_prefix + kv_tree + q_and_o + mask

    def vocab_bytes(self) -> int:
        """Target-logit bytes every step must read once (fp32 rows)."""
        return self.B * self.N * self.V * 4

    def attn_flops(self) -> int:
        """QK^T + PV flops over prefix and tree keys (dense, unmasked count)."""
        return 4 * self.B * self.Hq * self.d * self.N * (self.L + self.N)


CONFIGS = [
    VerifyConfig(
        index=0, name="tiny", B=1, Hq=4, Hkv=4, d=64, L=128, N=8, V=1000,
        sigma_t=2.0, sigma_d=1.0, temperatures=(1.0,), tree="random", max_depth=4,
        description="batch 1, 4/4 heads, d64, L128, 8-node random tree, V1000"),
    VerifyConfig(
        index=1, name="llama2-7b", B=1, Hq=32, Hkv=32, d=128, L=2048, N=26, V=32000,
        sigma_t=3.0, sigma_d=1.5, temperatures=(0.0, 1.0), tree="static", max_depth=5,
        description="LLaMA2-7B-shaped layer: batch 1, 32 MHA heads, d128, L2048, 26-node static tree"),
    VerifyConfig(
        index=2, name="llama2-13b", B=4, Hq=40, Hkv=40, d=128, L=4096, N=26, V=32000,
        sigma_t=3.0, sigma_d=1.0, temperatures=(1.0,), tree="static", max_depth=5,
        description="LLaMA2-13B-shaped: batch 4, 40 MHA heads, d128, L4096, 26-node static tree"),
    VerifyConfig(
        index=3, name="llama2-70b-gqa", B=8, Hq=64, Hkv=8, d=128, L=4096, N=26, V=32000,
        sigma_t=3.0, sigma_d=1.0, temperatures=(0.0, 1.0), tree="static", max_depth=5,
        description="LLaMA2-70B-shaped GQA: batch 8, 64/8 heads, d128, L4096, 26-node static tree"),
    VerifyConfig(
        index=4, name="mixtral-eagle2", B=16, Hq=32, Hkv=8, d=128, L=8192, N=60, V=32000,
        sigma_t=3.0, sigma_d=1.0, temperatures=(1.0,), tree="eagle2", max_depth=6,
        description="Mixtral-8x7B attention shape, EAGLE-2 dynamic 60-node tree per sequence"),
]

BY_NAME = {c.name: c for c in CONFIGS}


def get(name_or_index) -> VerifyConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    return BY_NAME[name_or_index]
