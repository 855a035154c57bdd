"""Helpers that drive libhymba_hh through its Python binding for the tests.

Every call goes through the C ABI (hybrid_attention_ssm_amd.binding); the
tensors referenced by the ctypes structs stay alive until the stream is
synchronised.
"""
from __future__ import annotations

import numpy as np
import torch

from hybrid_attention_ssm_amd import binding as hb
from hybrid_attention_ssm_amd.configs import LayerDims

TOL = {"f32": 1e-4, "bf16": 3e-2}


def rel_err(got, want) -> float:
    """max |got - want| / rms(want)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(np.abs(got - want).max()) / max(rms, 1e-30)


def np_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run_meta_prefix(dims: LayerDims, weights: dict, R: np.ndarray):
    """hh_meta_prefix of the layer (with no meta tokens: no meta K/V, and the
    SSM state and conv history start from zero)."""
    sd = hb.storage_dtype(dims)
    layer = hb.upload_weights(dims, weights)
    if dims.n_meta == 0:
        return layer, dict(k=None, v=None, h0=None, conv_tail=None)
    meta = hb.hh_meta_prefix(layer, hb.to_device(R, sd))
    torch.cuda.synchronize()
    return layer, meta


def run_prefill(dims: LayerDims, weights: dict, R, x, window, is_global, producer=None,
                cache_cap=None, cache_ring=True, cache_fill=0.0):
    """Meta prefix + prefill on the GPU.

    producer: result dict of the producer layer's run_prefill (for a consumer).
    cache_cap: allocate a decode cache of this many slots (producer only),
    pre-filled with `cache_fill`.  Returns tensors (kept alive) and numpy views.
    """
    sd = hb.storage_dtype(dims)
    dev = "cuda"
    B, n, d = x.shape
    G, hd, D, N, k = dims.n_kv_heads, dims.head_dim, dims.d_inner, dims.d_state, dims.d_conv
    layer, meta = run_meta_prefix(dims, weights, R)
    xt = hb.to_device(x, sd)
    out = torch.empty(B, n, d, dtype=sd, device=dev)
    h = torch.empty(B, D, N, dtype=torch.float32, device=dev)
    conv = torch.empty(B, k - 1, D, dtype=torch.float32, device=dev)
    keep = dict(layer=layer, meta=meta, x=xt, out=out, h=h, conv=conv)
    if layer.kv_producer:
        mk, mv = meta["k"], meta["v"]
        full_k = torch.empty(B, G, n, hd, dtype=sd, device=dev)
        full_v = torch.empty(B, G, n, hd, dtype=sd, device=dev)
        ck = cv = length = None
        cap = 0
        if cache_cap:
            cap = cache_cap
            ck = torch.full((B, G, cap, hd), cache_fill, dtype=sd, device=dev)
            cv = torch.full((B, G, cap, hd), cache_fill, dtype=sd, device=dev)
            length = torch.zeros(B, dtype=torch.int32, device=dev)
        kv = hb.make_kv(full_k, full_v, ck, cv, length, cap, cache_ring)
        keep.update(full_k=full_k, full_v=full_v, cache_k=ck, cache_v=cv, len=length)
    else:
        mk, mv = producer["meta"]["k"], producer["meta"]["v"]
        kv = hb.make_kv(producer["full_k"], producer["full_v"])
        keep.update(full_k=producer["full_k"], full_v=producer["full_v"])
        keep["meta"] = dict(meta, k=mk, v=mv)
    mstruct = hb.make_meta(mk, mv, meta["h0"], meta["conv_tail"])
    hb.hh_prefill(layer, xt, mstruct, window, is_global, out, kv=kv, state_h=h, state_conv=conv)
    torch.cuda.synchronize()
    keep["kv"] = kv
    return keep


def oracle_weights(w: dict) -> dict:
    return {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in w.items()}
