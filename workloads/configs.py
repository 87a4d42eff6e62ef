"""The five MoE-layer workloads and their routing distributions.

Shapes only; no arithmetic of the method lives here. The router, layout,
permute, expert and combine steps are implemented twice, independently: in
``oracle/`` (CPU, test infrastructure) and in ``combine_top_router_amd``
(HIP, the product). Both consume the tensors that ``workloads.gen`` makes
from these descriptions.

Shapes follow the families the AutoEP pages name as presets (DeepSpeed
"AutoEP" commit text, section "Supported presets": Mixtral, Qwen3-MoE,
DeepSeek-V3), and the DeepSeek-V3 split-plan measurement shape of
DeepSpeed PR #8190 ("Derive AutoEP rank splits ...", section
"Measurements": EP=8, 256 experts, 1024 tokens per rank, top_k 8, with the
balanced / mild skew / severe skew token distributions).
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class MoEConfig:
    """One MoE layer as one GPU runs it.

    ``ep_size`` virtual ranks split the tokens into contiguous source chunks
    and the experts into contiguous destination blocks; ``local_rank`` picks
    the block of experts this GPU holds (-1: all experts are local).
    """

    name: str
    num_tokens: int  # T
    hidden: int  # H
    num_experts: int  # E
    top_k: int
    inter: int  # I (SwiGLU intermediate size)
    ep_size: int = 1
    local_rank: int = -1
    align: int = 128
    dists: tuple = ("balanced",)
    shares: tuple = (-1,)  # local ranks the parity tests run

    @property
    def num_local_experts(self) -> int:
        return self.num_experts if self.local_rank < 0 else self.num_experts // self.ep_size

    def local_experts(self, local_rank=None) -> range:
        r = self.local_rank if local_rank is None else local_rank
        if r < 0:
            return range(self.num_experts)
        el = self.num_experts // self.ep_size
        return range(r * el, (r + 1) * el)

    def m_cap(self, local_rank=None) -> int:
        """Worst-case number of local rows: every token sends min(k, E_loc)
        assignments here and every local expert pads by align - 1 rows."""
        r = self.local_rank if local_rank is None else local_rank
        el = self.num_experts if r < 0 else self.num_experts // self.ep_size
        return self.num_tokens * min(self.top_k, el) + el * (self.align - 1)


CONFIGS = {
    "tiny": MoEConfig(
        name="tiny", num_tokens=64, hidden=128, num_experts=8, top_k=2, inter=256,
        ep_size=2, local_rank=-1, align=128, dists=("balanced",), shares=(-1, 0, 1),
    ),
    "mixtral_8x7b": MoEConfig(
        name="mixtral_8x7b", num_tokens=4096, hidden=4096, num_experts=8, top_k=2,
        inter=14336, ep_size=1, local_rank=-1, align=128, dists=("balanced",),
    ),
    "qwen3_30b_a3b": MoEConfig(
        name="qwen3_30b_a3b", num_tokens=8192, hidden=2048, num_experts=128, top_k=8,
        inter=768, ep_size=1, local_rank=-1, align=128, dists=("zipf",),
    ),
    "deepseek_v3_ep8_share": MoEConfig(
        name="deepseek_v3_ep8_share", num_tokens=8192, hidden=7168, num_experts=256,
        top_k=8, inter=2048, ep_size=8, local_rank=0, align=128,
        dists=("balanced", "mild", "severe"), shares=(0,),
    ),
    "deepseek_v3_large": MoEConfig(
        name="deepseek_v3_large", num_tokens=65536, hidden=7168, num_experts=256,
        top_k=8, inter=2048, ep_size=1, local_rank=-1, align=128, dists=("severe",),
    ),
}

# Order of the configurations as the workload list gives them (0-based).
CONFIG_ORDER = ("tiny", "mixtral_8x7b", "qwen3_30b_a3b", "deepseek_v3_ep8_share",
                "deepseek_v3_large")


def get(name: str) -> MoEConfig:
    return CONFIGS[name]
