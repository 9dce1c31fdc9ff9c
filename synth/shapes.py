"""Model shapes and decode workloads.

The speed workload on the pages is a 2B-class dense fp16 decoder with 25
layers and a 4096-token context, decoded at batch 1 (hakusoku.com story 7519,
section on the memory-bandwidth limit; aether-echoes operator view, sections
"how it was done" and "the model").  The pages name no normalisation,
position encoding, activation or widths; the shapes below are the stand-in
workloads this implementation is measured on.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ffn: int
    vocab: int          # embedding rows
    lm_vocab: int       # LM-head rows (== vocab unless the head is a shard)
    max_ctx: int
    rms_eps: float = 1e-5
    rope_base: float = 10000.0
    # mixture of experts: n_experts > 0 replaces every layer's MLP by
    # n_experts SwiGLU experts of width d_ffn with FP8 (E4M3) weights, of
    # which a router picks top_k per token
    n_experts: int = 0
    top_k: int = 0
    # expert weights as OCP MXFP4 blocks (E2M1 pairs, an E8M0 scale per 32)
    # instead of E4M3 codes with a float32 scale per row
    mxfp4: bool = False

    @property
    def qkv_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def moe(self) -> bool:
        return self.n_experts > 0

    def with_(self, **kw) -> "ModelShape":
        return replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    name: str
    shape: ModelShape
    prompt_len: int
    steps: int
    batch: int
    weight_seed: int = 0
    prompt_seed: int = 1
    lane: bool = False  # weights are lane 0's slice of the full model's tensors
    description: str = ""


TINY = ModelShape(n_layers=2, d_model=256, n_heads=4, head_dim=64, d_ffn=1024,
                  vocab=4096, lm_vocab=4096, max_ctx=128)
DENSE_2B = ModelShape(n_layers=25, d_model=2560, n_heads=20, head_dim=128,
                      d_ffn=6912, vocab=65536, lm_vocab=65536, max_ctx=4096)
# One lane of an 8-way tensor-parallel split of DENSE_2B: 3 of the 20 heads,
# 864 of the 6912 FFN columns and an 8192-row vocabulary shard of the LM head.
LANE_2B = DENSE_2B.with_(n_heads=3, d_ffn=864, lm_vocab=8192)
# dense2b's attention, embedding and LM head with a mixture-of-experts MLP:
# 32 experts of width 1728 in FP8, 4 active per token, so the active MLP is
# dense2b's 6912 columns at half the bytes.
MOE_2B = DENSE_2B.with_(d_ffn=1728, n_experts=32, top_k=4)
TINY_MOE = TINY.with_(d_ffn=256, n_experts=8, top_k=2)
# the same experts in MXFP4
MOE_2B_MX = MOE_2B.with_(mxfp4=True)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, prompt_len=16, steps=32, batch=1,
                     description="2 layers, d 256, 4x64 heads, ffn 1024, vocab 4096"),
    "dense2b": Workload("dense2b", DENSE_2B, prompt_len=128, steps=512, batch=1,
                        description="25 layers, d 2560, 20x128 heads, ffn 6912, vocab 65536"),
    "lane2b": Workload("lane2b", LANE_2B, prompt_len=128, steps=1024, batch=1, lane=True,
                       description="one 8-way TP lane of dense2b: 3 heads, ffn 864, 8192-row LM shard"),
    "dense2b_long": Workload("dense2b_long", DENSE_2B, prompt_len=3968, steps=128, batch=1,
                             description="dense2b from a 3968-token prompt to the 4096 cap"),
    "moe2b": Workload("moe2b", MOE_2B, prompt_len=128, steps=512, batch=1,
                      description="dense2b attention with 32 FP8 experts of width 1728, top-4 routing"),
    "moe2b_mx": Workload("moe2b_mx", MOE_2B_MX, prompt_len=128, steps=512, batch=1,
                         description="moe2b with MXFP4 experts (E2M1 pairs, an E8M0 scale per 32 weights)"),
    "dense2b_b8": Workload("dense2b_b8", DENSE_2B, prompt_len=256, steps=256, batch=8,
                           description="dense2b, 8 sequences of 256 prompt tokens decoded together"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def shape_for(name: str) -> ModelShape:
    return WORKLOADS[name].shape
