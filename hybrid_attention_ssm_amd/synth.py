"""Seeded synthetic inputs for the hybrid-head layer.

Both the GPU path and the CPU oracle consume these arrays; this module holds
only random draws and storage rounding, none of the layer's arithmetic.

Recipe (one numpy PCG64 generator per workload, seeded with the workload seed,
draws in this fixed order):
  1. x      [B, n, d]          ~ N(0, 1)
  2. R      [m, d]             ~ N(0, 1)            (meta tokens)
  3. W_in   [N_in, d]          ~ N(0, 1/d)          (rows Q|K|V|xs|z|dt|B|C)
  4. dt     [D]                ~ exp(U[ln 1e-3, ln 1e-1]);  b_dt = log(expm1(dt))
     so that softplus(b_dt) is log-uniform in [1e-3, 1e-1]
  5. A      [D, N]             = -exp(U[ln 1, ln 16])
  6. conv_w [D, k]             ~ N(0, 1/k);  conv_b = 0
  7. W_out  [d, H*hd + D]      ~ N(0, 1/(H*hd + D))
  8. beta_attn = beta_ssm = 1
With `varied` (the parity tests' recipe, so that the per-channel weights are
exercised; the benchmark workloads keep 6 and 8 as above), the layer draws
after step 7:
 12. conv_b    [D]             ~ 0.1 N(0, 1)
 13. beta_attn [H*hd]          ~ U[0.5, 2]
 14. beta_ssm  [D]             ~ U[0.5, 2]
A block (pre-norm, layer, residual, pre-norm, MLP, residual) draws its layer
(3-8), then:
  9. g1, g2 [d]                ~ 1 + 0.1 N(0, 1)    (RMSNorm gains, fp32)
 10. W_gu   [2 d_ff, d]        ~ N(0, 1/d)          (rows 2i gate i, 2i+1 up i)
 11. W_down [d, d_ff]          ~ N(0, 1/d_ff)
For bf16 workloads x, R, W_in, conv_w and W_out are rounded to bf16 once
(round to nearest even); every consumer sees the rounded values, and so are
W_gu and W_down.  A, b_dt, the betas and the norm gains stay fp32.  A consumer layer (no K/V projection) drops the K and V
rows of the same draw, so it shares every other weight with its producer.

The stage hooks take their inputs from recipes of their own (one generator,
seeded, draws in this order):
  attention: q [B, n, H*hd], k, v [B, G, n, hd], meta_k, meta_v [G, m, hd],
             all ~ N(0, 1), rounded to the storage type;
  SSM:       A and conv_w as in steps 5-6, conv_b ~ 0.1 N(0, 1), then
             xs [B*n, D] ~ N(0, 1) (fp32), z [B*n, D] ~ N(0, 1) (storage type),
             delta [B*n, D or S] ~ exp(U[ln 1e-3, ln 1e-1]) (fp32),
             B|C [B*n, 2N] ~ N(0, 1), h0 [D, N] ~ N(0, 1),
             conv_tail [k-1, D] ~ N(0, 1) (fp32).
"""
from __future__ import annotations

import numpy as np

from .configs import DecodeWorkload, LayerDims, PrefillWorkload, StackWorkload


def round_bf16(a) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); keep float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(a.shape)


def _store(dims: LayerDims, a) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dims.dtype == "bf16" else a


def _normal(rng, shape, std=1.0) -> np.ndarray:
    out = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out


def layer_weights(rng, dims: LayerDims, kv_producer: bool = True, varied: bool = False) -> dict:
    """Draw one layer's parameters (steps 3-8 of the recipe; with `varied`,
    steps 12-14 replace the constant conv bias and betas)."""
    d, D, N, k = dims.d_model, dims.d_inner, dims.d_state, dims.d_conv
    Wa, kv = dims.attn_width, dims.n_kv_heads * dims.head_dim
    w_in = _store(dims, _normal(rng, (dims.n_in(True), d), (1.0 / d) ** 0.5))
    if not kv_producer:
        w_in = np.ascontiguousarray(np.concatenate([w_in[:Wa], w_in[Wa + 2 * kv:]]))
    dtw = dims.dt_width                       # D channels, or Mamba2 heads
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=dtw))
    dt_bias = np.log(np.expm1(dt)).astype(np.float32)
    a_shape = (dims.ssm_heads,) if dims.ssm_heads else (D, N)
    A = (-np.exp(rng.uniform(np.log(1.0), np.log(16.0), size=a_shape))).astype(np.float32)
    conv_w = _store(dims, _normal(rng, (D, k), (1.0 / k) ** 0.5))
    conv_b = np.zeros(D, np.float32)
    w_out = _store(dims, _normal(rng, (d, Wa + D), (1.0 / (Wa + D)) ** 0.5))
    beta_attn, beta_ssm = np.ones(Wa, np.float32), np.ones(D, np.float32)
    if varied:
        conv_b = _normal(rng, (D,), 0.1)
        beta_attn = rng.uniform(0.5, 2.0, size=Wa).astype(np.float32)
        beta_ssm = rng.uniform(0.5, 2.0, size=D).astype(np.float32)
    return dict(w_in=w_in, dt_bias=dt_bias, A=A, conv_w=conv_w, conv_b=conv_b,
                beta_attn=beta_attn, beta_ssm=beta_ssm, w_out=w_out, kv_producer=bool(kv_producer))


def block_weights(rng, dims: LayerDims, d_ff: int, kv_producer: bool = True,
                  varied: bool = False) -> dict:
    """Draw one block's parameters: its layer, then steps 9-11 of the recipe."""
    d = dims.d_model
    mixer = layer_weights(rng, dims, kv_producer, varied)
    g1 = (1.0 + 0.1 * _normal(rng, (d,))).astype(np.float32)
    g2 = (1.0 + 0.1 * _normal(rng, (d,))).astype(np.float32)
    w_gu = _store(dims, _normal(rng, (2 * d_ff, d), (1.0 / d) ** 0.5))
    w_down = _store(dims, _normal(rng, (d, d_ff), (1.0 / d_ff) ** 0.5))
    return dict(mixer=mixer, norm1=g1, norm2=g2, w_gate_up=w_gu, w_down=w_down, d_ff=int(d_ff))


def block_inputs(w: PrefillWorkload, d_ff: int, kv_producer: bool = True, seed=None,
                 varied: bool = False) -> dict:
    """x, meta tokens R and one block's weights for a prefill workload."""
    dims = w.dims
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x = _store(dims, _normal(rng, (w.batch, w.seqlen, dims.d_model)))
    R = _store(dims, _normal(rng, (dims.n_meta, dims.d_model)))
    return dict(x=x, R=R, weights=block_weights(rng, dims, d_ff, kv_producer, varied))


def prefill_inputs(w: PrefillWorkload, kv_producer: bool = True, seed=None,
                   varied: bool = False) -> dict:
    """x, meta tokens R and the layer weights for a prefill workload."""
    dims = w.dims
    rng = np.random.default_rng(w.seed if seed is None else seed)
    x = _store(dims, _normal(rng, (w.batch, w.seqlen, dims.d_model)))
    R = _store(dims, _normal(rng, (dims.n_meta, dims.d_model)))
    weights = layer_weights(rng, dims, kv_producer, varied)
    return dict(x=x, R=R, weights=weights)


def decode_inputs(w: DecodeWorkload, seed=None, varied: bool = False) -> dict:
    """Weights, caches, SSM states and new tokens for a decode workload.

    Draw order: per layer (in layer order) its weights; then per cache (sorted
    by name) meta K, meta V, cache K, cache V; then per layer h [B, D, N]
    (fp32), its conv tail [B, k-1, D] and its new token x_t [B, d]; all N(0, 1).
    Every sequence holds `context` real positions before the step.
    """
    dims = w.dims
    rng = np.random.default_rng(w.seed if seed is None else seed)
    G, m, hd = dims.n_kv_heads, dims.n_meta, dims.head_dim
    B, D, N, k = w.batch, dims.d_inner, dims.d_state, dims.d_conv
    layers = []
    for spec in w.layers:
        layers.append(dict(spec=spec, weights=layer_weights(rng, dims, spec.kv_producer, varied)))
    caches = {}
    for name in sorted({s.cache for s in w.layers}):
        is_ring = name != "global"
        cap = w.window if is_ring else w.global_cap
        caches[name] = dict(
            meta_k=_store(dims, _normal(rng, (G, m, hd))),
            meta_v=_store(dims, _normal(rng, (G, m, hd))),
            k=_store(dims, _normal(rng, (B, G, cap, hd))),
            v=_store(dims, _normal(rng, (B, G, cap, hd))),
            len=np.full(B, w.context, np.int32), cap=cap, is_ring=is_ring)
    for lay in layers:
        lay["h"] = _normal(rng, (B, D, N))
        lay["conv"] = _store(dims, _normal(rng, (B, k - 1, D)))
        lay["x_t"] = _store(dims, _normal(rng, (B, dims.d_model)))
    return dict(layers=layers, caches=caches)


def stack_inputs(w: StackWorkload, steps: int, varied: bool = False, seed=None) -> dict:
    """Weights, caches, SSM states and stack inputs for decode steps through a
    stack of blocks (w.layer_plan()).

    Draw order: per block (in order) its weights (block recipe); then per cache
    (in order of first use) meta K, meta V, cache K, cache V; then per block h
    [B, D, N] (fp32) and its conv history [B, k-1, D]; then the stack input of
    each step x [steps, B, d]; all N(0, 1).  Every sequence holds `context`
    real positions before the first step.
    """
    dims = w.dims
    rng = np.random.default_rng(w.seed if seed is None else seed)
    G, m, hd = dims.n_kv_heads, dims.n_meta, dims.head_dim
    B, D, N, k = w.batch, dims.d_inner, dims.d_state, dims.d_conv
    plan = w.layer_plan()
    blocks = [dict(is_global=g, kv_producer=p, cache=c,
                   weights=block_weights(rng, dims, w.d_ff, p, varied)) for g, p, c in plan]
    caches = {}
    for g, _, name in plan:
        if name in caches:
            continue
        cap = w.global_cap if g else w.window
        caches[name] = dict(
            meta_k=_store(dims, _normal(rng, (G, m, hd))),
            meta_v=_store(dims, _normal(rng, (G, m, hd))),
            k=_store(dims, _normal(rng, (B, G, cap, hd))),
            v=_store(dims, _normal(rng, (B, G, cap, hd))),
            len=np.full(B, w.context, np.int32), cap=cap, is_ring=not g)
    for blk in blocks:
        blk["h"] = _normal(rng, (B, D, N))
        blk["conv"] = _store(dims, _normal(rng, (B, k - 1, D)))
    x = _store(dims, _normal(rng, (steps, B, dims.d_model)))
    return dict(blocks=blocks, caches=caches, x=x)


def attn_stage_inputs(dims: LayerDims, batch: int, seqlen: int, seed: int) -> dict:
    """Inputs of the attention stage hook (the recipe in the module header)."""
    rng = np.random.default_rng(seed)
    H, G, hd, m = dims.n_heads, dims.n_kv_heads, dims.head_dim, dims.n_meta
    q = _store(dims, _normal(rng, (batch, seqlen, H * hd)))
    k = _store(dims, _normal(rng, (batch, G, seqlen, hd)))
    v = _store(dims, _normal(rng, (batch, G, seqlen, hd)))
    mk = _store(dims, _normal(rng, (G, m, hd)))
    mv = _store(dims, _normal(rng, (G, m, hd)))
    return dict(q=q, k=k, v=v, meta_k=mk, meta_v=mv)


def ssm_stage_inputs(dims: LayerDims, batch: int, seqlen: int, seed: int) -> dict:
    """Inputs of the SSM stage hook (the recipe in the module header); row-major
    [B*n, ...] arrays."""
    rng = np.random.default_rng(seed)
    D, N, k, R = dims.d_inner, dims.d_state, dims.d_conv, batch * seqlen
    a_shape = (dims.ssm_heads,) if dims.ssm_heads else (D, N)
    A = (-np.exp(rng.uniform(np.log(1.0), np.log(16.0), size=a_shape))).astype(np.float32)
    conv_w = _store(dims, _normal(rng, (D, k), (1.0 / k) ** 0.5))
    conv_b = _normal(rng, (D,), 0.1)
    xs = _normal(rng, (R, D))
    z = _store(dims, _normal(rng, (R, D)))
    delta = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), size=(R, dims.dt_width))).astype(np.float32)
    bc = _normal(rng, (R, 2 * N))
    h0 = _normal(rng, (D, N))
    conv_tail = _normal(rng, (k - 1, D))
    return dict(A=A, conv_w=conv_w, conv_b=conv_b, xs=xs, z=z, delta=delta, bc=bc, h0=h0,
                conv_tail=conv_tail)
