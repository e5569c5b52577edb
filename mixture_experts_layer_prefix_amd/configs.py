"""Workload shapes of the MoE layer forward.

Five synthetic workloads, each named by what it is.  The shapes follow the
model families the pages name as examples (Mixtral-8x7B-sized experts, an
8-expert top-2 layer, a 64-expert Switch-style top-1 layer with a capacity
limit, and a DeepSeek-V3-style fine-grained layer with one shared expert):
  - yunthe.com, "MoE混合专家模型实战", opening paragraph (Mixtral 8x7B and
    DeepSeek-V3 parameter counts) and section "MoE架构的稀疏激活原理与
    Transformer实现" (8 experts, top-2, FFN = Linear, GELU, Linear);
  - lmnt.cn MoE walkthrough, section 3.3 (capacity factor);
  - wiblog.cn "MoE 专家路由如何实现稀疏激活", section on fine-grained and
    shared experts.

Nothing in this module computes any step of the layer.
"""
from __future__ import annotations

import dataclasses
from typing import Optional


@dataclasses.dataclass(frozen=True)
class MoEShape:
    name: str
    T: int                 # tokens in the batch
    d_model: int
    d_ff: int
    n_experts: int         # routed experts N
    top_k: int             # K
    dtype: str             # "f32" or "bf16": x, expert weights, intermediates, out
    capacity_factor: Optional[float] = None   # None: dropless
    d_ff_shared: int = 0   # 0: no shared expert
    router_bias: bool = False      # router Linear has a bias (tiny fp32 layer)
    expert_bias: bool = False      # expert Linears have biases (tiny fp32 layer)
    logit_offset: Optional[str] = None   # None | "normal" | "zipf": per-expert additive logit term
    sel_bias: bool = False         # per-expert selection-only bias ~ U(-0.5, 0.5)
    aux_alpha: float = 0.0         # >0: also compute alpha*N*sum(f*P)
    index: int = 0                 # position in the list below; keys the input streams
    weight_quant: str = "none"     # "int8" / "int4": routed w1 / w2 quantised per output row

    @property
    def M_max(self) -> int:
        """Upper bound on the number of (token, expert) rows: T*K."""
        return self.T * self.top_k

    def with_(self, **kw) -> "MoEShape":
        return dataclasses.replace(self, **kw)


TINY_FP32 = MoEShape(
    name="tiny_fp32", T=64, d_model=64, d_ff=128, n_experts=8, top_k=2, dtype="f32",
    router_bias=True, expert_bias=True, index=0)

MIXTRAL_PREFILL = MoEShape(
    name="mixtral_8x7b_prefill", T=4096, d_model=4096, d_ff=14336, n_experts=8, top_k=2,
    dtype="bf16", index=1)

DECODE = MoEShape(
    name="decode_t32_e64", T=32, d_model=4096, d_ff=11008, n_experts=64, top_k=2,
    dtype="bf16", logit_offset="normal", index=2)

SWITCH_CAPACITY = MoEShape(
    name="switch_top1_capacity", T=8192, d_model=2048, d_ff=8192, n_experts=64, top_k=1,
    dtype="bf16", capacity_factor=1.25, logit_offset="zipf", aux_alpha=0.01, index=3)

DEEPSEEK_FINE = MoEShape(
    name="deepseek_v3_fine_grained", T=4096, d_model=7168, d_ff=2048, n_experts=256, top_k=8,
    dtype="bf16", d_ff_shared=2048, sel_bias=True, index=4)

ALL = [TINY_FP32, MIXTRAL_PREFILL, DECODE, SWITCH_CAPACITY, DEEPSEEK_FINE]

# The weight-bandwidth-bound workloads again with INT8 routed expert weights
# (lmnt.cn walkthrough §4.3: experts compressed to INT8 for inference).  Same
# seeded bf16 weights as the workload they derive from (same index); each
# side quantises them itself.
INT8 = [DECODE.with_(name="decode_t32_e64_w8", weight_quant="int8"),
        SWITCH_CAPACITY.with_(name="switch_top1_capacity_w8", weight_quant="int8"),
        DEEPSEEK_FINE.with_(name="deepseek_v3_fine_grained_w8", weight_quant="int8")]

# The same three again with INT4 routed expert weights (lmnt.cn walkthrough
# §4.3 names INT4 beside INT8; yunthe.com's deployment section cites 4-bit
# weight-only formats).
INT4 = [DECODE.with_(name="decode_t32_e64_w4", weight_quant="int4"),
        SWITCH_CAPACITY.with_(name="switch_top1_capacity_w4", weight_quant="int4"),
        DEEPSEEK_FINE.with_(name="deepseek_v3_fine_grained_w4", weight_quant="int4")]

BY_NAME = {c.name: c for c in ALL + INT8 + INT4}
