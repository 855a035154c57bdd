"""Helpers that drive libhymba_hh through its Python binding for the tests.

Every call goes through the C ABI (hybrid_attention_ssm_amd.binding); the
tensors referenced by the ctypes structs stay alive until the stream is
synchronised.

Output buffers, the workspace and the caches are allocated inside guard
bands: every byte of a buffer and of its guards starts as 0xFF (a NaN in
fp32 and bf16).  After a call, `check_guards` asserts that no kernel wrote
outside a buffer (the guards keep their bytes) and `assert_written` that an
output holds no NaN (every element was written).
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


UNIT_ROUNDOFF = {"f32": 2.0 ** -24, "bf16": 2.0 ** -8}


def rel_err_stored(got, want, dtype) -> float:
    """rel_err of a result stored in `dtype` ("f32" or "bf16"), allowing each
    element its own rounding to that type (the unit roundoff times |want|)
    before the comparison with the RMS-relative bar."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    excess = np.maximum(np.abs(got - want) - UNIT_ROUNDOFF[dtype] * np.abs(want), 0.0)
    rms = float(np.sqrt(np.mean(want * want)))
    return float(excess.max() / rms) if rms > 0 else float(excess.max())


def np_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


GUARD_BYTES = 4096
_guarded = []          # (buffer, payload bytes) of every guarded allocation since the last check


def guarded(shape, dtype, device="cuda", fill=None) -> torch.Tensor:
    """A tensor inside guard bands of GUARD_BYTES on each side.  Its bytes and
    the guards' start as 0xFF (NaN); `fill` overwrites the payload."""
    es = torch.empty((), dtype=dtype).element_size()
    n = int(np.prod(shape)) if len(shape) else 1
    nbytes = n * es
    buf = torch.full((nbytes + 2 * GUARD_BYTES,), 0xFF, dtype=torch.uint8, device=device)
    t = buf[GUARD_BYTES:GUARD_BYTES + nbytes].view(dtype).view(*shape)
    if fill is not None:
        t.fill_(fill)
    _guarded.append((buf, nbytes))
    return t


def check_guards():
    """Every guard band allocated in this test so far still holds 0xFF (the
    list is cleared between tests by an autouse fixture in conftest.py)."""
    bad = []
    for buf, nbytes in _guarded:
        lo, hi = buf[:GUARD_BYTES], buf[GUARD_BYTES + nbytes:]
        if not (bool((lo == 0xFF).all()) and bool((hi == 0xFF).all())):
            bad.append(nbytes)
    assert not bad, f"writes outside {len(bad)} buffer(s) of {bad} bytes"


def release_guards():
    _guarded.clear()


def assert_written(name, t: torch.Tensor):
    """No NaN left from the poison fill: every element was written."""
    nan = int(torch.isnan(t.float()).sum())
    assert nan == 0, f"{name}: {nan} of {t.numel()} elements never written"


def poisoned_workspace(nbytes, device="cuda") -> torch.Tensor:
    return guarded((max(int(nbytes), 256),), torch.uint8, device)


def run_meta_prefix(dims: LayerDims, weights: dict, R: np.ndarray):
    """hh_meta_prefix of the layer (with no meta tokens: no meta K/V, and the
    SSM state and conv history start from zero)."""
    sd = hb.storage_dtype(dims)
    layer = hb.upload_weights(dims, weights)
    if dims.n_meta == 0:
        return layer, dict(k=None, v=None, h0=None, conv_tail=None)
    need = hb.hh_meta_prefix_workspace_size(dims, layer.kv_producer)
    meta = hb.hh_meta_prefix(layer, hb.to_device(R, sd), ws=poisoned_workspace(need))
    torch.cuda.synchronize()
    for name in ("k", "v", "h0", "conv_tail"):
        if meta.get(name) is not None:
            assert_written("meta " + name, meta[name])
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
    out = guarded((B, n, d), sd, dev)
    h = guarded((B, D, N), torch.float32, dev)
    conv = guarded((B, k - 1, D), torch.float32, dev)
    keep = dict(layer=layer, meta=meta, x=xt, out=out, h=h, conv=conv)
    if layer.kv_producer:
        mk, mv = meta["k"], meta["v"]
        full_k = guarded((B, G, n, hd), sd, dev)
        full_v = guarded((B, G, n, hd), sd, dev)
        ck = cv = length = None
        cap = 0
        if cache_cap:
            cap = cache_cap
            ck = guarded((B, G, cap, hd), sd, dev, fill=cache_fill)
            cv = guarded((B, G, cap, hd), sd, dev, fill=cache_fill)
            length = guarded((B,), torch.int32, dev, fill=0)
        kv = hb.make_kv(full_k, full_v, ck, cv, length, cap, cache_ring)
        keep.update(full_k=full_k, full_v=full_v, cache_k=ck, cache_v=cv, len=length)
    else:
        mk, mv = producer["meta"]["k"], producer["meta"]["v"]
        kv = hb.make_kv(producer["full_k"], producer["full_v"])
        keep.update(full_k=producer["full_k"], full_v=producer["full_v"])
        keep["meta"] = dict(meta, k=mk, v=mv)
    mstruct = hb.make_meta(mk, mv, meta["h0"], meta["conv_tail"])
    ws = poisoned_workspace(hb.hh_prefill_workspace_size(dims, B, n, layer.kv_producer))
    hb.hh_prefill(layer, xt, mstruct, window, is_global, out, kv=kv, state_h=h, state_conv=conv, ws=ws)
    torch.cuda.synchronize()
    for name in ("out", "h", "conv") + (("full_k", "full_v") if layer.kv_producer else ()):
        assert_written(name, keep[name])
    check_guards()
    keep["kv"] = kv
    keep["ws"] = ws
    return keep


def oracle_weights(w: dict) -> dict:
    return {k: (v.astype(np.float64) if isinstance(v, np.ndarray) else v) for k, v in w.items()}
