"""The synthetic workloads: shapes, sync fractions and input recipes (no arithmetic).

Each workload is one forward of a CAAT sublayer, or of an attention-output-projection
sublayer followed by an MLP sublayer ("pair"), with all P tensor-parallel ranks
emulated on one device.  Inputs are seeded normals from ``synth``; weights are
N(0, 0.02^2); gamma = 1 and beta = 0 unless a test asks otherwise.
"""
from dataclasses import dataclass, field
from typing import Tuple

ATTN_OUT = "attn_out"   # row-parallel out-projection only: partial = ctx_m . O_m
MLP = "mlp"             # column-parallel GEMM + activation, then row-parallel GEMM


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str                      # "f32" or "bf16": storage dtype of every tensor
    P: int                          # emulated tensor-parallel ranks
    h: int                          # hidden size
    ffn: int                        # FFN size of the full (unsharded) MLP
    T: int                          # tokens (batch x sequence)
    p: float                        # sync fraction
    act: str                        # "gelu" | "gelu_tanh" | "swiglu"
    norm: str                       # "layernorm" | "rmsnorm"
    sublayers: Tuple[str, ...]      # (MLP,) or (ATTN_OUT, MLP)
    eps: float = 1e-5
    replicated_x: bool = False      # the MLP input is one draw copied to every rank
    heads: int = 0                  # attention heads (all ranks); the full block splits them
    seq: int = 0                    # sequence length: T = (T / seq) sequences (full block)
    note: str = ""
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def f_s(self) -> int:
        return self.ffn // self.P


TINY_MLP_F32 = Workload(
    "tiny-mlp-fp32", "f32", P=2, h=256, ffn=1024, T=128, p=0.5, act="gelu",
    norm="layernorm", sublayers=(MLP,), replicated_x=True,
    note="P=2, h=256, ffn=1024 (512 per shard), T=128, x replicated per rank")

PAIR_130M_BF16 = Workload(
    "130m-pair-bf16", "bf16", P=4, h=768, ffn=3072, T=4096, p=0.5, act="gelu",
    norm="layernorm", sublayers=(ATTN_OUT, MLP), heads=12, seq=2048,
    note="h=768, ffn=3072, P=4, T=4096 (2 x 2048); out-projection then MLP")

MLP_1P1B_BF16 = Workload(
    "1.1b-mlp-bf16", "bf16", P=8, h=2048, ffn=5632, T=8192, p=0.5, act="swiglu",
    norm="rmsnorm", sublayers=(MLP,),
    note="h=2048, SwiGLU ffn=5632 (704 per shard), P=8, T=8192 (4 x 2048); p swept")

PREFILL_7B_BF16 = Workload(
    "7b-prefill-pair-bf16", "bf16", P=8, h=4096, ffn=11008, T=8192, p=0.5, act="swiglu",
    norm="rmsnorm", sublayers=(ATTN_OUT, MLP), heads=32, seq=4096,
    note="h=4096, SwiGLU ffn=11008 (1376 per shard), P=8, T=8192 (2 x 4096)")

DECODE_7B_BF16 = Workload(
    "7b-decode-pair-bf16", "bf16", P=8, h=4096, ffn=11008, T=64, p=0.5, act="swiglu",
    norm="rmsnorm", sublayers=(ATTN_OUT, MLP), heads=32,
    note="7B prefill weights, decode batch T in {1, 8, 64}")

SWEEP_P_1P1B = (1.0, 0.5, 0.25)
DECODE_T = (1, 8, 64)

ALL = {w.name: w for w in (TINY_MLP_F32, PAIR_130M_BF16, MLP_1P1B_BF16,
                           PREFILL_7B_BF16, DECODE_7B_BF16)}


def with_(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (e.g. T or p)."""
    from dataclasses import replace
    return replace(w, **changes)
