"""Shapes of the five hybrid-head workloads.

Layer shapes follow the 1.5B column of the Hymba paper's architecture table
(Hymba: A Hybrid-head Architecture for Small Language Models, Appendix E,
Table 11: hidden 1600, 25 attention heads in 5 query groups, SSM state 16,
window 1024) and its 128 meta tokens (§2.3 and the authors' OpenReview reply on
the number of meta tokens).  Head dim 64 and d_inner 3200 are the two free
widths of that table fixed by the workload definitions below.

The block around the layer (pre-norms, residuals and the MLP) uses the same
table's MLP hidden width, 5504 at 1.5B, and its 32 blocks with 3 full-attention
layers (first, middle, last).

This module holds data only: no arithmetic of the method lives here.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class LayerDims:
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    d_inner: int
    d_state: int
    d_conv: int
    n_meta: int
    dtype: str  # "f32" or "bf16"
    eps: float = 1e-6
    rope_base: float = 0.0  # rotary embedding base of Q and K; 0: none
    ssm_heads: int = 0      # Mamba2 SSM heads (per-head Delta and scalar A); 0: Mamba

    @property
    def attn_width(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def dt_width(self) -> int:
        """Columns of the dt block: one per SSM head (Mamba2) or per channel."""
        return self.ssm_heads or self.d_inner

    def n_in(self, kv_producer: bool = True) -> int:
        kv = 2 * self.n_kv_heads * self.head_dim if kv_producer else 0
        return self.attn_width + kv + 2 * self.d_inner + self.dt_width + 2 * self.d_state

    @property
    def fused_width(self) -> int:
        return self.attn_width + self.d_inner

    def as_dict(self) -> dict:
        return dict(d_model=self.d_model, n_heads=self.n_heads,
                    n_kv_heads=self.n_kv_heads, head_dim=self.head_dim,
                    d_inner=self.d_inner, d_state=self.d_state,
                    d_conv=self.d_conv, n_meta=self.n_meta, eps=self.eps,
                    rope_base=self.rope_base, ssm_heads=self.ssm_heads)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    seed: int
    dims: LayerDims
    batch: int
    seqlen: int
    window: int
    is_global: bool


@dataclass(frozen=True)
class DecodeLayer:
    is_global: bool
    kv_producer: bool
    cache: str  # name of the KV cache this layer uses


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    dims: LayerDims
    batch: int
    context: int          # real positions already in the cache before the step
    window: int
    global_cap: int       # real slots of a global cache
    layers: Tuple[DecodeLayer, ...] = field(default_factory=tuple)


TINY = LayerDims(d_model=64, n_heads=2, n_kv_heads=1, head_dim=32, d_inner=128,
                 d_state=16, d_conv=4, n_meta=4, dtype="f32")
HYMBA_1P5B = LayerDims(d_model=1600, n_heads=25, n_kv_heads=5, head_dim=64,
                       d_inner=3200, d_state=16, d_conv=4, n_meta=128,
                       dtype="bf16")

CFG0_TINY = PrefillWorkload("tiny_f32_n64", 0, TINY, batch=1, seqlen=64,
                            window=16, is_global=False)
CFG1_SWA_8K = PrefillWorkload("swa_prefill_b1_n8192", 1, HYMBA_1P5B, batch=1,
                              seqlen=8192, window=1024, is_global=False)
CFG2_GLOBAL_8K = PrefillWorkload("global_prefill_b1_n8192", 2, HYMBA_1P5B,
                                 batch=1, seqlen=8192, window=1024,
                                 is_global=True)
CFG3_DECODE = DecodeWorkload(
    "decode_b128_ctx8192", 3, HYMBA_1P5B, batch=128, context=8191,
    window=1024, global_cap=8192,
    layers=(DecodeLayer(False, True, "swa"), DecodeLayer(False, False, "swa"),
            DecodeLayer(True, True, "global")))
CFG4_SWA_32K = PrefillWorkload("swa_prefill_b2_n32768", 4, HYMBA_1P5B, batch=2,
                               seqlen=32768, window=1024, is_global=False)

CONFIGS = (CFG0_TINY, CFG1_SWA_8K, CFG2_GLOBAL_8K, CFG3_DECODE, CFG4_SWA_32K)


def shrink(w: PrefillWorkload, **kw) -> PrefillWorkload:
    """A copy of a prefill workload with some fields replaced (test sizes)."""
    dims_kw = {k: kw.pop(k) for k in list(kw) if hasattr(w.dims, k)}
    dims = replace(w.dims, **dims_kw) if dims_kw else w.dims
    return replace(w, dims=dims, **kw)


MLP_HIDDEN_1P5B = 5504     # Table 11, 1.5B column
MLP_HIDDEN_TINY = 96


@dataclass(frozen=True)
class StackWorkload:
    """A decode step through a stack of blocks.

    Full-attention layers own a linear cache of global_cap slots; sliding-window
    layers pair up in order (the first of a pair produces K/V into a ring of
    `window` slots, the second reads it); an unpaired window layer produces
    for itself.
    """
    name: str
    seed: int
    dims: LayerDims
    d_ff: int
    batch: int
    context: int
    window: int
    global_cap: int
    n_layers: int
    global_layers: Tuple[int, ...]

    def layer_plan(self):
        """[(is_global, kv_producer, cache name)] per layer."""
        plan, pending = [], None
        for i in range(self.n_layers):
            if i in self.global_layers:
                plan.append((True, True, f"g{i}"))
                pending = None
            elif pending is None:
                plan.append((False, True, f"r{i}"))
                pending = f"r{i}"
            else:
                plan.append((False, False, pending))
                pending = None
        return plan


STACK_DECODE = StackWorkload("stack32_decode_b128_ctx8192", 5, HYMBA_1P5B, MLP_HIDDEN_1P5B,
                             batch=128, context=8191, window=1024, global_cap=8192,
                             n_layers=32, global_layers=(0, 15, 31))
