"""Workload table for the Double Sparsity decode step.

Five synthetic workloads stand in for the models and long-context benchmarks
the Double Sparsity page (abstract) evaluates on (Llama-2-7B/70B, Mixtral-8x7B;
wiki-2, key-value retrieval, long-context suites), whose weights and data are
not available.  Shapes follow a Llama-2-7B decode step (32 MHA heads, d=128),
a 70B-like GQA step (64 query heads over 8 KV heads), and the 1/16 token and
channel sparsity the page reports.  The block-granular workload follows the
block-max informativeness of the Jenga page (method, item 1; default block 64)
and the top-k key framing of the HiP page (abstract).

This module only describes shapes and seeds.  It holds none of the method's
arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16": element type of q, K, V and the label cache
    B: int              # sequences in the decode batch
    Hq: int             # query heads
    Hkv: int            # key/value heads (Hq % Hkv == 0)
    d: int              # head dimension
    T: int              # valid tokens in the KV cache
    r: int              # label channels per KV head
    block: int          # selection granularity in tokens (1 = token-level)
    k_units: int        # tokens (block == 1) or blocks kept per (sequence, KV head)
    seed_base: int      # root of every seed drawn for this workload
    n_outliers: int = 8
    outlier_scale: float = 6.0
    fixed_outliers: bool = False   # True: channels 0..n_outliers-1 in every head
    T_cap: int = 0      # allocated cache length (0 means T)
    n_calib: int = 256  # calibration queries per query head and keys per KV head
    ragged: bool = False   # True: sequence lengths drawn per sequence in [T // 16, T] (T is the longest)
    tau: float | None = None   # threshold rule (keep units scoring >= tau, at most k_units); None: top-k
    offload: bool = False      # True: K and V live in pinned host memory
    hip: bool = False          # True: hierarchical span search; k_units = spans kept, block = longest final span

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        return self.T_cap if self.T_cap else self.T

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def n_units(self) -> int:
        return -(-self.T // self.block)

    @property
    def k_tok(self) -> int:
        """Tokens attended per (sequence, KV head) when every kept block is whole."""
        return self.k_units * self.block

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, in the order the decode benchmark lists them.
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "f32", B=1, Hq=1, Hkv=1, d=128, T=1024, r=16,
                         block=1, k_units=64, seed_base=1000, fixed_outliers=True),
    "llama7b_16k": Workload("llama7b_16k", "bf16", B=1, Hq=32, Hkv=32, d=128, T=16384,
                            r=16, block=1, k_units=1024, seed_base=2000),
    "batched_32k": Workload("batched_32k", "bf16", B=16, Hq=32, Hkv=32, d=128, T=32768,
                            r=8, block=1, k_units=2048, seed_base=3000),
    "gqa70b_128k": Workload("gqa70b_128k", "bf16", B=8, Hq=64, Hkv=8, d=128, T=131072,
                            r=8, block=1, k_units=8192, seed_base=4000),
    "block64_256k": Workload("block64_256k", "bf16", B=1, Hq=32, Hkv=32, d=128, T=262144,
                             r=16, block=64, k_units=64, seed_base=5000),
}

WORKLOAD_ORDER = ["tiny_f32", "llama7b_16k", "batched_32k", "gqa70b_128k", "block64_256k"]

# A decode batch of sequences of unequal lengths (a serving batch): the Llama-2-7B
# shape of llama7b_16k, eight sequences whose lengths are drawn uniformly from
# [1024, 16384] (gen.seq_lengths), the first one at the full 16384.
RAGGED_WORKLOADS = {
    "ragged_16k": Workload("ragged_16k", "bf16", B=8, Hq=32, Hkv=32, d=128, T=16384, r=16, block=1, k_units=1024,
                           seed_base=6000, ragged=True),
}
WORKLOADS.update(RAGGED_WORKLOADS)
RAGGED_ORDER = ["ragged_16k"]

# The threshold rule (Jenga page, core method item 1: positive-only head
# aggregation, block-wise max over 64-token blocks, a layer threshold): a GQA
# batch with four query heads per KV head, at most 128 blocks kept per row.
# tau = 650 on these inputs keeps between 0 and all 128 blocks per row (mean
# about 60): some rows keep nothing, some are capped.
THRESHOLD_WORKLOADS = {
    "jenga_gqa_32k": Workload("jenga_gqa_32k", "bf16", B=4, Hq=32, Hkv=8, d=128, T=32768, r=16, block=64,
                              k_units=128, seed_base=7000, tau=650.0),
}
WORKLOADS.update(THRESHOLD_WORKLOADS)
THRESHOLD_ORDER = ["jenga_gqa_32k"]

# Offloaded KV (Double Sparsity page, abstract: the method combines with
# offloading; it reports its offloading result at 256K tokens): the shape of
# block64_256k, with K and V in pinned host memory and only the label cache in
# HBM, so each step reads the kept 64-token blocks across the host link.
OFFLOAD_WORKLOADS = {
    "offload_256k": Workload("offload_256k", "bf16", B=1, Hq=32, Hkv=32, d=128, T=262144, r=16, block=64,
                             k_units=64, seed_base=5000, offload=True),
}
WORKLOADS.update(OFFLOAD_WORKLOADS)
OFFLOAD_ORDER = ["offload_256k"]

# Hierarchical span search (HiP page, abstract: O(log T) rounds, contexts of
# millions of tokens): one million tokens, a 32/8 GQA group of a Llama-like
# model, 64 spans of at most 64 tokens kept per KV head (4,096 of 1,048,576
# tokens).  No label cache is used.
HIP_WORKLOADS = {
    "hip_1m": Workload("hip_1m", "bf16", B=2, Hq=32, Hkv=8, d=128, T=1 << 20, r=16, block=64, k_units=64,
                       seed_base=8000, hip=True),
}
WORKLOADS.update(HIP_WORKLOADS)
HIP_ORDER = ["hip_1m"]

# The decode benchmark's headline workload: T=16K, 32 heads, bf16.
HEADLINE = "llama7b_16k"


def get(name: str) -> Workload:
    return WORKLOADS[name]


# Seeds.  Each (sequence, KV head) unit owns an independent PCG64 stream so any
# slice of a large cache can be regenerated on its own.
def model_seed(w: Workload) -> int:
    return w.seed_base


def unit_seed(w: Workload, b: int, g: int) -> int:
    return w.seed_base + 1_000_003 * (b + 1) + 7919 * (g + 1)


def calib_seed(w: Workload) -> int:
    return w.seed_base + 17


def lengths_seed(w: Workload) -> int:
    return w.seed_base + 29
