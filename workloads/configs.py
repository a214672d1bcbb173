"""Workload definitions for the LatentMoE MXFP4 routed-expert layer.

Shapes follow the Kimi-K3 LatentMoE described on the pages: 896 routed experts,
16 selected per token, two always-on shared experts, experts running in the
3584-wide latent (infervisor.ai "Bringing up Kimi-K3 on day zero", section
"The model we hadn't run"; dev48.org "Kimi K3 on AMD Instinct GPUs with
TokenSpeed", section 4 "Latent MoE"). Weights are MXFP4: E2M1 codes with one
E8M0 exponent per 32 values along the input dimension, bias 127 (same
sections; huggingface.co "Notes from an NVFP4 port of Kimi K3.1 Pro",
introduction). The expert intermediate width (2048) is not fixed by the pages;
it is a stated choice of the workload.

Named workloads:
  tiny            T=8,   L=256,  E=32,  k=4,  I=128   (seed 0)
  decode          T=1,   L=3584, E=896, k=16, I=2048  (seed 1)
  batched_decode  T=64,  same layer                    (seed 2)
  prefill         T=4096, same layer                   (seed 3)
  skewed          T=8192, same layer, logits given with a Zipf(1.2) expert
                  bias and 5% of tokens carrying a 32-way exact tie (seed 4)
plus the same layer at the widths the pages imply or shard to:
  decode_i3072    T=1,    I=Is=3072 (seed 1): the expert width that the
  prefill_i3072   T=4096, I=Is=3072 (seed 3)  per-expert size the pages quote
                  implies (17.72 MiB per NVFP4 expert: huggingface.co "Notes
                  from an NVFP4 port of Kimi K3.1 Pro", the paragraph on
                  per-token expert reads), here in MXFP4
  decode_tp8      T=1,    I=Is=256  (seed 1): one GPU's share of every expert
                  when the experts are split eight ways along the intermediate
                  width (dev48.org "Kimi K3 on AMD Instinct GPUs with
                  TokenSpeed", Figure 2), the router whole
plus smaller parity shapes with ragged tails (not multiples of any tile).

Block workloads (H > 0) add the MoE input step and tail around the layer
(TokenSpeed sections 4.2-4.4): the 7168-wide hidden input u, the running
residual, the packed input weight (router, hidden -> latent, shared gate/up),
the routed RMSNorm weight, the latent -> hidden up-projection and the shared
experts' down projection to the hidden width. There the shared experts (S, Is)
read the hidden input; the routed layer inside has none of its own.
  block_tiny      T=8,    H=512,  L=256,  E=32,  k=4,  I=Is=128 (seed 20)
  block_ragged    T=37,   H=448,  L=320,  E=96,  k=6,  I=Is=192, S=1 (seed 21)
  block_decode    T=1,    H=7168, the K3 layer (seed 22)
  block_batched   T=64,   same (seed 24)
  block_prefill   T=4096, same (seed 23)
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Dims:
    T: int   # tokens
    L: int   # latent width (input of gate/up, output of down)
    E: int   # routed experts
    k: int   # experts selected per token
    I: int   # routed-expert intermediate width
    S: int   # shared experts (always on, weight 1)
    Is: int  # shared-expert intermediate width
    H: int = 0  # hidden width of the MoE block (0: the layer alone)

    @property
    def routes(self) -> int:
        return self.T * self.k


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dims: Dims
    # E8M0 scale distribution: ("uniform", lo, hi) integers inclusive, or
    # ("normal", mean, std) rounded to nearest and clamped to [0, 254].
    scales: Tuple = ("normal", 121.0, 2.0)
    x_std: float = 1.0
    router_std: float = 0.02
    shared_std: float = 0.02
    # Given-logits workloads (the router step is skipped).
    logits_given: bool = False
    zipf_s: float = 1.2
    tie_frac: float = 0.05
    tie_group: int = 32
    note: str = ""

    def with_T(self, T: int, name: Optional[str] = None) -> "Workload":
        return replace(self, dims=replace(self.dims, T=T), name=name or f"{self.name}_T{T}")


_K3 = dict(L=3584, E=896, k=16, I=2048, S=2, Is=2048)

WORKLOADS = {
    "tiny": Workload(
        "tiny", 0, Dims(T=8, L=256, E=32, k=4, I=128, S=2, Is=128),
        scales=("uniform", 120, 130),
        note="tiny LatentMoE layer; oracle finishes instantly"),
    "decode": Workload(
        "decode", 1, Dims(T=1, **_K3),
        note="K3-shaped batch-1 decode, all 896 experts resident"),
    "batched_decode": Workload(
        "batched_decode", 2, Dims(T=64, **_K3),
        note="64 rows, as for speculative verification of 16 users x 4 positions"),
    "prefill": Workload(
        "prefill", 3, Dims(T=4096, **_K3),
        note="prefill chunk, ~73 tokens per expert"),
    "skewed": Workload(
        "skewed", 4, Dims(T=8192, **_K3), logits_given=True,
        note="Zipf(1.2) expert bias on given logits, 5% of tokens tied over 32 experts"),
    # a few decode tokens per call (speculative or concurrent decode), from
    # the decode configuration's token stream
    **{f"decode_t{T}": Workload(
        f"decode_t{T}", 1, Dims(T=T, **_K3),
        note=f"{T} decode tokens per call, the decode layer") for T in (2, 4, 8, 16)},
    "decode_i3072": Workload(
        "decode_i3072", 1, Dims(T=1, **{**_K3, "I": 3072, "Is": 3072}),
        note="K3 decode at the expert width the pages' per-expert size implies"),
    "prefill_i3072": Workload(
        "prefill_i3072", 3, Dims(T=4096, **{**_K3, "I": 3072, "Is": 3072}),
        note="prefill chunk at the expert width the pages' per-expert size implies"),
    "decode_tp8": Workload(
        "decode_tp8", 1, Dims(T=1, **{**_K3, "I": 256, "Is": 256}),
        note="one GPU's eighth of every routed and shared expert, router whole"),
    "block_tiny": Workload(
        "block_tiny", 20, Dims(T=8, L=256, E=32, k=4, I=128, S=2, Is=128, H=512),
        scales=("uniform", 120, 130), note="MoE block around the tiny layer"),
    "block_ragged": Workload(
        "block_ragged", 21, Dims(T=37, L=320, E=96, k=6, I=192, S=1, Is=192, H=448),
        scales=("uniform", 118, 132), note="MoE block with ragged tiles"),
    "block_decode": Workload(
        "block_decode", 22, Dims(T=1, H=7168, **_K3), note="K3 MoE block, one token"),
    "block_batched": Workload(
        "block_batched", 24, Dims(T=64, H=7168, **_K3), note="K3 MoE block, 64 rows"),
    "block_prefill": Workload(
        "block_prefill", 23, Dims(T=4096, H=7168, **_K3), note="K3 MoE block, prefill chunk"),
    # Parity shapes: several tiles plus ragged tails in every dimension.
    "ragged": Workload(
        "ragged", 10, Dims(T=37, L=416, E=48, k=6, I=352, S=2, Is=224),
        scales=("uniform", 118, 132)),
    "ragged_prefill": Workload(
        "ragged_prefill", 11, Dims(T=301, L=544, E=40, k=5, I=480, S=1, Is=160),
        scales=("uniform", 118, 132)),
    "ragged_skew": Workload(
        "ragged_skew", 12, Dims(T=509, L=352, E=64, k=8, I=288, S=2, Is=96),
        scales=("uniform", 118, 132), logits_given=True, tie_group=12),
}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
