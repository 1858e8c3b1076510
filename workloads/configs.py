"""The five synthetic workloads of the routed LoRA delta.

Shapes follow the pages: the fused QKV lane with GQA k/v slices (xLLM PR #2014,
"New subsystems", LoRAQKVParallelLinear), the fused gate/up column-parallel lane
and the o_proj / down_proj row-parallel lanes (same section), and one GPU's
share of a row-parallel layer whose A factor is cut by input columns
(TensorFold PR #47, first and third commit messages: attention wo_b and the
shared expert's w2, the latter reading an fp16 hidden state).

Values and structure are synthetic: no trained adapter or dataset is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class LaneSpec:
    """One projection the delta is added to.

    h_in     columns of A (and of x) this GPU holds
    h_out    output width of each slice (q|k|v, gate|up, or a single slice)
    x_dtype  "bf16" or "fp16" (the shared expert's w2 reads an fp16 hidden state)
    tp_size  >1 for a row-parallel share: the full A has h_in * tp_size columns
             and this GPU holds columns [tp_rank*h_in, (tp_rank+1)*h_in)
    """
    name: str
    h_in: int
    h_out: tuple
    x_dtype: str = "bf16"
    tp_size: int = 1
    tp_rank: int = 0

    @property
    def h_in_full(self) -> int:
        return self.h_in * self.tp_size

    @property
    def a_col0(self) -> int:
        return self.h_in * self.tp_rank

    @property
    def h_out_total(self) -> int:
        return sum(self.h_out)


@dataclass(frozen=True)
class WorkloadSpec:
    """Batch structure, adapter population and lanes of one workload.

    Decode rows are sequences of length 1.  A decode row is base (adapter id 0)
    with probability base_prob, otherwise its adapter is drawn by `popularity`
    ("uniform" or "zipf" with exponent zipf_s over adapter ranks 1..n).
    Prefill sequences have lengths uniform in [prefill_len[0], prefill_len[1]]
    and draw their adapter uniformly (never base).

    rank_mode "list" gives adapter i rank ranks[i]; "choice" draws each
    adapter's rank uniformly from `ranks`.  scale_mode "alpha" gives
    scale = alpha / rank (PEFT's lora_alpha / r), "fixed" gives `scale`,
    "uniform" draws from scale_range.
    """
    name: str
    seed: int
    lanes: tuple
    n_adapters: int
    ranks: tuple
    rank_mode: str = "list"
    scale_mode: str = "alpha"
    alpha: float = 32.0
    scale: float = 1.0
    scale_range: tuple = (0.5, 4.0)
    max_rank: int = 16
    max_loras: int = 0
    decode_rows: int = 0
    base_prob: float = 0.0
    popularity: str = "uniform"
    zipf_s: float = 1.1
    prefill_seqs: int = 0
    prefill_len: tuple = (128, 128)
    description: str = ""

    @property
    def n_seq(self) -> int:
        return self.decode_rows + self.prefill_seqs


TINY = WorkloadSpec(
    name="tiny", seed=0,
    lanes=(LaneSpec("proj", 64, (64,)),),
    n_adapters=2, ranks=(4, 4), rank_mode="list",
    scale_mode="fixed", scale=2.0, max_rank=4,
    decode_rows=8, base_prob=1.0 / 3.0, popularity="uniform",
    description="T=8 decode rows, 64->64, 2 adapters rank 4 scale 2, "
                "slot uniform in {0,1,2}",
)

DECODE_MIX = WorkloadSpec(
    name="decode_mix", seed=1,
    lanes=(LaneSpec("qkv", 4096, (4096, 1024, 1024)),),
    n_adapters=8, ranks=(16,) * 8, rank_mode="list",
    scale_mode="alpha", alpha=32.0, max_rank=16,
    decode_rows=256, base_prob=0.25, popularity="uniform",
    description="T=256 decode rows, fused QKV 4096->4096|1024|1024 "
                "(32 q heads, 8 kv heads, head_dim 128), 8 adapters r=16 "
                "alpha=32, 25% base",
)

PREFILL = WorkloadSpec(
    name="prefill", seed=2,
    lanes=(LaneSpec("o_proj", 4096, (4096,)),
           LaneSpec("gate_up", 4096, (14336, 14336))),
    n_adapters=6, ranks=(8, 8, 16, 16, 64, 64), rank_mode="list",
    scale_mode="alpha", alpha=32.0, max_rank=64,
    prefill_seqs=8, prefill_len=(128, 2048),
    description="8 prefill sequences of length U{128..2048}, one adapter per "
                "sequence from 6 (ranks 8,8,16,16,64,64 padded to 64), "
                "o_proj 4096->4096 and gate_up 4096->2x14336",
)

MANY_TENANTS = WorkloadSpec(
    name="many_tenants", seed=3,
    lanes=(LaneSpec("down_proj", 17408, (5120,)),
           LaneSpec("o_proj", 5120, (5120,))),
    n_adapters=64, ranks=(8, 16, 32, 64), rank_mode="choice",
    scale_mode="uniform", scale_range=(0.5, 4.0), max_rank=64, max_loras=64,
    decode_rows=1024, base_prob=0.10, popularity="zipf", zipf_s=1.1,
    description="T=1024 decode rows, 64 adapters with Zipf(1.1) popularity "
                "and 10% base, down_proj 17408->5120 and o_proj 5120->5120, "
                "ranks U{8,16,32,64}, scales U[0.5,4], max_loras=64",
)

TP_SHARE = WorkloadSpec(
    name="tp_share", seed=4,
    lanes=(LaneSpec("attn_out", 2048, (7168,), "bf16", tp_size=8, tp_rank=3),
           LaneSpec("shexp_w2", 2048, (7168,), "fp16", tp_size=8, tp_rank=3)),
    n_adapters=32, ranks=(8, 16, 32, 64, 128), rank_mode="choice",
    scale_mode="alpha", alpha=32.0, max_rank=128,
    decode_rows=3584, base_prob=0.25, popularity="uniform",
    prefill_seqs=4, prefill_len=(128, 128),
    description="one GPU's 1/8 share of row-parallel attention-out and "
                "shared-expert w2 (16384->7168, A cut by input columns), "
                "32 adapters ranks U{8..128}, 3584 decode rows + 4x128 prefill",
)

CONFIGS = (TINY, DECODE_MIX, PREFILL, MANY_TENANTS, TP_SHARE)


def config_by_name(name: str) -> WorkloadSpec:
    for c in CONFIGS:
        if c.name == name:
            return c
    raise KeyError(f"unknown workload {name!r}; known: "
                   f"{[c.name for c in CONFIGS]}")
